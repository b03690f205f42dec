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

struct FwdArgs {
    View q, k, v;
    void* o;
    int64_t osb, osh, osn;
    float* lse;
    int B, H, N, d;
    int causal;
    float scale;
    // block-sparse mode (kv_offsets != nullptr)
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    int64_t nnz;
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
    float* delta;  // workspace: fp32 [B, H, N]
    int B, H, N, d;
    int causal;
    float scale;
};

// Launch the forward kernels on `stream`; returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Launch the backward kernels on `stream`.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
