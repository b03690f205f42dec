// Internal interface between the C-ABI layer (fa_api.cpp) and the HIP kernel files.
// Nothing here is exported from libfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One [B, H, N, d] tensor view: element strides of batch, head and token; d stride 1.
struct View {
    const void* p;
    int64_t sb, sh, sn;
};

// Sequence layout shared by the forward and backward arguments. Fixed length: sequence b
// is the b-th [N, d] slab of every tensor (batch stride). Packed variable length
// (cu != nullptr): sequence b is rows cu[b] .. cu[b+1]-1 of [total, d] tensors (the batch
// stride is unused), at most N rows long; LSE and D are then [H, total].
// Grouped heads: K, V (and dK, dV) have Hkv heads; query head h reads head h / (H / Hkv).
struct Layout {
    int B, H, Hkv, N, d;
    const int32_t* cu;
    int64_t total;
};

struct FwdArgs {
    Layout L;
    View q, k, v;
    void* o;
    int64_t osb, osh, osn;
    float* lse;
    int causal;
    float scale;
    // element type of q, k, v: bf16 (f8 == 0) or fp8 e4m3 (f8 != 0, real value = code x
    // descale; the score descale qk_desc is the product of the Q and K descales)
    int f8;
    float qk_desc;
    float v_desc;
    // block-sparse mode (kv_offsets != nullptr)
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    int64_t nnz;
    // optional visit log of the block-sparse kernels: byte [(b * H + h) * 2 * nnz + 2 * e + half]
    // is set to 1 when sequence b, head h takes half `half` of list entry e into its softmax
    uint8_t* visits = nullptr;
};

struct BwdArgs {
    View q, k, v, o, dout;
    const float* lse;
    void* dq;
    int64_t dqsb, dqsh, dqsn;
    void* dk;
    int64_t dksb, dksh, dksn;
    void* dv;
    int64_t dvsb, dvsh, dvsn;
    float* delta;  // workspace: fp32 -D, laid out like the LSE, then the LSE in the exp2 domain
    Layout L;
    int causal;
    float scale;
    // block-sparse mode (kv_offsets != nullptr): query-side lists for dQ, key-side lists
    // (for every key block, the query blocks that list it) for dK and dV; nnz entries each.
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    const int32_t* q_offsets;
    const int32_t* q_indices;
    int64_t nnz;
    // Stored-dS mode (head dimension 128; nullptr: dQ recomputes S and dP): workspace regions
    // for the dS tiles, ds_bh elements per (sequence, query head), and (block-sparse) one int32
    // per list entry for the key-side position of each query-side entry.
    uint16_t* ds = nullptr;
    int64_t ds_bh = 0;
    int32_t* ds_pos = nullptr;
};

// Launch the forward kernels on `stream`; returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Launch the backward kernels on `stream`.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Size of the library-owned backward workspace (one per GPU).
constexpr size_t kStaticWorkspaceBytes = (size_t)32 << 20;
// Device address of the current device's library-owned workspace (set up on first use).
hipError_t static_workspace(void** ptr);

}  // namespace fa
