// C ABI of libfa.so: host-side argument validation, block-list utilities and launches.
// Declarations, argument meanings and the passages they follow are in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "fa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return FA_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // B, H, N each stay well inside int32
// Query rows of one call (B*H*N, or H*total when packed): every launch then stays below 2^31
// work-items (the backward's dK/dV grid has four per key row) and its workgroup indices in int.
constexpr int64_t kMaxRowsFwd = (int64_t)1 << 30;
constexpr int64_t kMaxRowsBwd = (int64_t)1 << 29;
// Token stride in elements: the tile loaders address a 64-row tile with 32-bit byte offsets.
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;
// Work-items of the largest launch of a call, from its grid (N: the longest sequence when
// packed): forward, 512 threads per 256 query rows (dense) or 256 per 128 (block-sparse);
// backward, 512 threads per 128 keys (dK, dV) and 256 per 128 query rows (dQ). Keeping it
// at most 2^31 keeps the 32-bit grid size and the kernels' int workgroup indices from
// wrapping; the row limits above alone do not (a batch of tiny sequences, or a packed
// batch of many sequences with one long one, has far more workgroups than rows / 128).
constexpr int64_t kMaxItems = (int64_t)1 << 31;
int64_t launch_items(const fa_attn_desc& d, bool backward) {
    const int64_t bh = d.B * d.H, u128 = (d.N + 127) / 128, u256 = (d.N + 255) / 256;
    if (backward) return bh * u128 * 512;
    const int64_t dense = bh * u256 * 512, sparse = bh * u128 * 256;
    return dense > sparse ? dense : sparse;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int64_t B, int64_t H, int64_t N, int64_t d) {
    if (B < 0 || H < 0 || N < 0)
        return fail(FA_ERR_SHAPE, "negative size B=%lld H=%lld N=%lld", (long long)B, (long long)H, (long long)N);
    if (B > kMaxDim || H > kMaxDim || N > kMaxDim || B * H > kMaxDim)
        return fail(FA_ERR_SHAPE, "size too large B=%lld H=%lld N=%lld", (long long)B, (long long)H, (long long)N);
    if (d != 64 && d != 128) return fail(FA_ERR_HEADDIM, "head dimension %lld not supported (64 or 128)", (long long)d);
    return FA_OK;
}

// Pointer and strides of one tensor; `mult` is the element count of 16 bytes (8 for bf16,
// 16 for fp8), so that every row starts 16-byte aligned.
int check_tensor(const char* name, const void* p, const fa_strides& s, int mult = 8) {
    if (!p) return fail(FA_ERR_NULL, "%s is NULL", name);
    if (!aligned16(p)) return fail(FA_ERR_LAYOUT, "%s is not 16-byte aligned", name);
    if ((s.b % mult) || (s.h % mult) || (s.n % mult))
        return fail(FA_ERR_LAYOUT, "%s strides (%lld, %lld, %lld) are not multiples of %d elements", name,
                    (long long)s.b, (long long)s.h, (long long)s.n, mult);
    if (s.b < 0 || s.h < 0 || s.n < 0) return fail(FA_ERR_LAYOUT, "%s has a negative stride", name);
    if (s.n > kMaxRowStride)
        return fail(FA_ERR_LAYOUT, "%s token stride %lld exceeds %lld elements", name, (long long)s.n,
                    (long long)kMaxRowStride);
    return FA_OK;
}

int check_device() {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(FA_ERR_HIP, "no HIP device available (%s)", hipGetErrorString(e));
    }
    return FA_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

fa::View view(const void* p, const fa_strides& s) { return fa::View{p, s.b, s.h, s.n}; }

bool packed(const fa_attn_desc& d) { return d.cu_seqlens != nullptr; }
bool empty_problem(const fa_attn_desc& d) {
    return d.B == 0 || d.H == 0 || d.N == 0 || (packed(d) && d.total == 0);
}

// Sizes, head grouping, sequence layout, scale and block lists of a descriptor.
int check_desc(const fa_attn_desc* dp, bool backward) {
    if (!dp) return fail(FA_ERR_NULL, "desc is NULL");
    const fa_attn_desc& d = *dp;
    int st = check_sizes(d.B, d.H, d.N, d.d);
    if (st) return st;
    if (d.H_kv < 0 || d.H_kv > kMaxDim) return fail(FA_ERR_SHAPE, "bad H_kv %lld", (long long)d.H_kv);
    if (d.H > 0 && (d.H_kv == 0 || d.H % d.H_kv != 0))
        return fail(FA_ERR_SHAPE, "H=%lld is not a multiple of H_kv=%lld", (long long)d.H, (long long)d.H_kv);
    if (packed(d) && (d.total < 0 || d.total > kMaxDim))
        return fail(FA_ERR_SHAPE, "bad packed row count total=%lld", (long long)d.total);
    if (packed(d) && d.total * d.H > kMaxDim)
        return fail(FA_ERR_SHAPE, "H * total too large (%lld * %lld)", (long long)d.H, (long long)d.total);
    const int64_t rows = packed(d) ? d.H * d.total : d.B * d.H * d.N;
    const int64_t max_rows = backward ? kMaxRowsBwd : kMaxRowsFwd;
    if (rows > max_rows)
        return fail(FA_ERR_SHAPE, "%lld query rows in one call exceed %lld", (long long)rows, (long long)max_rows);
    const int64_t items = launch_items(d, backward);
    if (items > kMaxItems)
        return fail(FA_ERR_SHAPE, "a launch would need %lld work-items, more than %lld (B=%lld H=%lld N=%lld)",
                    (long long)items, (long long)kMaxItems, (long long)d.B, (long long)d.H, (long long)d.N);
    if (!std::isfinite(d.scale)) return fail(FA_ERR_ARG, "scale is not finite");
    if (d.dtype != FA_DTYPE_BF16 && d.dtype != FA_DTYPE_FP8_E4M3) return fail(FA_ERR_ARG, "unknown dtype %d", d.dtype);
    if (d.dtype == FA_DTYPE_FP8_E4M3) {
        if (backward) return fail(FA_ERR_ARG, "the backward takes bf16 tensors only");
        if (!std::isfinite(d.q_descale) || !std::isfinite(d.k_descale) || !std::isfinite(d.v_descale))
            return fail(FA_ERR_ARG, "a descale is not finite");
        if (!std::isfinite(d.scale * d.q_descale * d.k_descale))
            return fail(FA_ERR_ARG, "scale * q_descale * k_descale overflows");
    }
    if (!d.kv_offsets && (d.kv_indices || d.q_offsets || d.q_indices))
        return fail(FA_ERR_NULL, "block lists given without kv_offsets");
    if (d.kv_offsets) {
        if (d.block_size != 128) return fail(FA_ERR_SHAPE, "block size %lld not supported (128)", (long long)d.block_size);
        if (d.nnz < 0) return fail(FA_ERR_LIST, "negative nnz");
        if (!d.kv_indices && d.nnz > 0) return fail(FA_ERR_NULL, "kv_indices is NULL");
        if (backward) {
            if (!d.q_offsets) return fail(FA_ERR_NULL, "q_offsets is NULL (key-side lists are needed for dK, dV)");
            if (!d.q_indices && d.nnz > 0) return fail(FA_ERR_NULL, "q_indices is NULL");
        }
    }
    return FA_OK;
}

fa::Layout layout(const fa_attn_desc& d) {
    fa::Layout L;
    L.B = (int)d.B; L.H = (int)d.H; L.Hkv = (int)d.H_kv; L.N = (int)d.N; L.d = (int)d.d;
    L.cu = d.cu_seqlens;
    L.total = packed(d) ? d.total : 0;
    return L;
}

// With nnz == 0 the kernels read no index; any valid pointer stands in for a NULL one.
const int32_t* or_other(const int32_t* p, const int32_t* other) { return p ? p : other; }

int check_lse(const float* lse) {
    if (!lse) return fail(FA_ERR_NULL, "lse is NULL");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FA_ERR_LAYOUT, "lse is not 4-byte aligned");
    return FA_OK;
}

// Tensors of a backward call.
int check_bwd_tensors(const void* q, const fa_strides& sq, const void* k, const fa_strides& sk, const void* v,
                      const fa_strides& sv, const void* o, const fa_strides& so, const void* dout,
                      const fa_strides& sdo, const float* lse, const void* dq, const fa_strides& sdq, const void* dk,
                      const fa_strides& sdk, const void* dv, const fa_strides& sdv) {
    int st;
    if ((st = check_tensor("q", q, sq)) || (st = check_tensor("k", k, sk)) || (st = check_tensor("v", v, sv)) ||
        (st = check_tensor("o", o, so)) || (st = check_tensor("dout", dout, sdo)) ||
        (st = check_tensor("dq", dq, sdq)) || (st = check_tensor("dk", dk, sdk)) ||
        (st = check_tensor("dv", dv, sdv)) || (st = check_lse(lse)))
        return st;
    return FA_OK;
}

fa_attn_desc plain_desc(int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale) {
    fa_attn_desc x;
    std::memset(&x, 0, sizeof x);
    x.B = B; x.H = H; x.H_kv = H; x.N = N; x.d = d;
    x.causal = causal;
    x.scale = scale;
    return x;
}

// The forward of fa_attn_fwd; with `visits` set (block-sparse only, checked by the caller)
// the kernels also write the visit log, which is zero-filled first on the same stream.
int attn_fwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
             fa_strides sv, void* o, fa_strides so, float* lse, uint8_t* visits, void* stream) {
    int st = check_desc(desc, false);
    if (st) return st;
    const fa_attn_desc& d = *desc;
    if (visits && !d.kv_offsets) return fail(FA_ERR_ARG, "a visit log needs block-sparse lists (kv_offsets)");
    if (empty_problem(d)) return ok();
    const bool f8 = d.dtype == FA_DTYPE_FP8_E4M3;
    const int m = f8 ? 16 : 8;
    if ((st = check_tensor("q", q, sq, m)) || (st = check_tensor("k", k, sk, m)) ||
        (st = check_tensor("v", v, sv, m)) || (st = check_tensor("o", o, so)) || (st = check_lse(lse)))
        return st;
    if ((st = check_device())) return st;
    fa::FwdArgs a;
    a.f8 = f8;
    a.qk_desc = f8 ? d.q_descale * d.k_descale : 1.0f;
    a.v_desc = f8 ? d.v_descale : 1.0f;
    a.L = layout(d);
    a.q = view(q, sq);
    a.k = view(k, sk);
    a.v = view(v, sv);
    a.o = o;
    a.osb = so.b; a.osh = so.h; a.osn = so.n;
    a.lse = lse;
    a.causal = d.causal != 0;
    a.scale = d.scale;
    a.kv_offsets = d.kv_offsets;
    a.kv_indices = d.kv_offsets ? or_other(d.kv_indices, d.kv_offsets) : nullptr;
    a.nnz = d.kv_offsets ? d.nnz : 0;
    a.visits = nullptr;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (visits && a.nnz > 0) {
        const size_t bytes = (size_t)d.B * (size_t)d.H * 2 * (size_t)a.nnz;
        if (hipMemsetAsync(visits, 0, bytes, s) != hipSuccess) return launched(hipGetLastError(), "visit log fill");
        a.visits = visits;
    }
    return launched(fa::launch_fwd(a, s), "forward");
}

}  // namespace

extern "C" {

int fa_attn_fwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
                fa_strides sv, void* o, fa_strides so, float* lse, void* stream) {
    return attn_fwd(desc, q, sq, k, sk, v, sv, o, so, lse, nullptr, stream);
}

int fa_attn_fwd_visits(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk,
                       const void* v, fa_strides sv, void* o, fa_strides so, float* lse, uint8_t* visits,
                       void* stream) {
    if (!visits) return fail(FA_ERR_NULL, "visits is NULL");
    return attn_fwd(desc, q, sq, k, sk, v, sv, o, so, lse, visits, stream);
}

size_t fa_attn_bwd_workspace_bytes(const fa_attn_desc* desc) {
    if (!desc || desc->B <= 0 || desc->H <= 0 || desc->N <= 0) return 0;
    const int64_t rows = packed(*desc) ? desc->total : desc->B * desc->N;
    if (rows <= 0) return 0;
    const size_t bytes = 2 * (size_t)desc->H * (size_t)rows * sizeof(float);   // D and the exp2-domain LSE
    return (bytes + 255) & ~(size_t)255;
}

}  // extern "C"

namespace {

// dS tiles of the stored-dS backward per (sequence, query head); 0 when the mode does not apply.
int64_t ds_tiles(const fa_attn_desc& d) {
    if (d.d != 128) return 0;
    const int64_t nqb = (d.N + 127) / 128;
    if (d.kv_offsets) return d.nnz > 0 ? d.nnz : 0;
    return d.causal ? nqb * (nqb + 1) / 2 : nqb * nqb;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int attn_bwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
             fa_strides sv, const void* o, fa_strides so, const void* dout, fa_strides sdo, const float* lse,
             void* dq, fa_strides sdq, void* dk, fa_strides sdk, void* dv, fa_strides sdv, void* workspace,
             size_t workspace_bytes, bool allow_ds, void* stream) {
    int st = check_desc(desc, true);
    if (st) return st;
    const fa_attn_desc& d = *desc;
    if (empty_problem(d)) return ok();
    if ((st = check_bwd_tensors(q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv))) return st;
    const size_t need = fa_attn_bwd_workspace_bytes(desc);
    if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(FA_ERR_LAYOUT, "workspace is not 16-byte aligned");
    if ((st = check_device())) return st;
    fa::BwdArgs a;
    a.q = view(q, sq);
    a.k = view(k, sk);
    a.v = view(v, sv);
    a.o = view(o, so);
    a.dout = view(dout, sdo);
    a.lse = lse;
    a.dq = dq; a.dqsb = sdq.b; a.dqsh = sdq.h; a.dqsn = sdq.n;
    a.dk = dk; a.dksb = sdk.b; a.dksh = sdk.h; a.dksn = sdk.n;
    a.dv = dv; a.dvsb = sdv.b; a.dvsh = sdv.h; a.dvsn = sdv.n;
    a.delta = static_cast<float*>(workspace);
    a.L = layout(d);
    a.causal = d.causal != 0;
    a.scale = d.scale;
    const bool sparse = d.kv_offsets != nullptr;
    a.kv_offsets = sparse ? d.kv_offsets : nullptr;
    a.kv_indices = sparse ? or_other(d.kv_indices, d.kv_offsets) : nullptr;
    a.q_offsets = sparse ? d.q_offsets : nullptr;
    a.q_indices = sparse ? or_other(d.q_indices, d.q_offsets) : nullptr;
    a.nnz = sparse ? d.nnz : 0;
    // A workspace that also holds the dS tiles selects the stored-dS schedule. Its layout
    // after the per-row values (each part 256-byte aligned): block-sparse, the key-side
    // position of every query-side entry; then the tiles, ds_bh elements per (sequence,
    // query head).
    const size_t need_ds = allow_ds ? fa_attn_bwd_ds_workspace_bytes(desc) : 0;
    if (need_ds && workspace_bytes >= need_ds) {
        unsigned char* w = static_cast<unsigned char*>(workspace) + need;
        if (sparse) {
            a.ds_pos = reinterpret_cast<int32_t*>(w);
            w += round256((size_t)d.nnz * sizeof(int32_t));
        }
        a.ds = reinterpret_cast<uint16_t*>(w);
        a.ds_bh = ds_tiles(d) * 128 * 128;
    }
    return launched(fa::launch_bwd(a, static_cast<hipStream_t>(stream)), "backward");
}

}  // namespace

extern "C" {

size_t fa_attn_bwd_ds_workspace_bytes(const fa_attn_desc* desc) {
    const size_t base = fa_attn_bwd_workspace_bytes(desc);
    if (!base || desc->dtype != FA_DTYPE_BF16) return 0;
    const int64_t tiles = ds_tiles(*desc);
    if (tiles <= 0) return 0;
    // B * H * tiles * 32 KB, refused (0) beyond 2^56 bytes
    const double est = (double)desc->B * (double)desc->H * (double)tiles * 32768.0;
    if (est > 7.2e16) return 0;
    const size_t pos = desc->kv_offsets ? round256((size_t)desc->nnz * sizeof(int32_t)) : 0;
    return base + pos + (size_t)desc->B * (size_t)desc->H * (size_t)tiles * 32768u;
}

int fa_attn_bwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
                fa_strides sv, const void* o, fa_strides so, const void* dout, fa_strides sdo, const float* lse,
                void* dq, fa_strides sdq, void* dk, fa_strides sdk, void* dv, fa_strides sdv, void* workspace,
                size_t workspace_bytes, void* stream) {
    return attn_bwd(desc, q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv, workspace,
                    workspace_bytes, true, stream);
}

static_assert(FA_NOALLOC_WORKSPACE_BYTES == fa::kStaticWorkspaceBytes, "header and library disagree");

int fa_attn_bwd_noalloc(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk,
                        const void* v, fa_strides sv, const void* o, fa_strides so, const void* dout,
                        fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk, fa_strides sdk,
                        void* dv, fa_strides sdv, void* stream) {
    int st = check_desc(desc, true);
    if (st) return st;
    if (empty_problem(*desc)) return ok();
    if ((st = check_bwd_tensors(q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv))) return st;
    const size_t need = fa_attn_bwd_workspace_bytes(desc);
    if (need > fa::kStaticWorkspaceBytes)
        return fail(FA_ERR_WORKSPACE, "the problem needs %zu bytes of workspace; the library-owned one holds %zu",
                    need, fa::kStaticWorkspaceBytes);
    if ((st = check_device())) return st;
    void* ws = nullptr;
    const hipError_t e = fa::static_workspace(&ws);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "library-owned workspace unavailable: %s", hipGetErrorString(e));
    return attn_bwd(desc, q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv, ws,
                    fa::kStaticWorkspaceBytes, false, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
           int64_t d, fa_strides sq, fa_strides sk, fa_strides sv, fa_strides so, int causal, float scale,
           void* stream) {
    const fa_attn_desc x = plain_desc(B, H, N, d, causal, scale);
    return fa_attn_fwd(&x, q, sq, k, sk, v, sv, o, so, lse, stream);
}

int fa_sparse_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t d, fa_strides sq, fa_strides sk, fa_strides sv, fa_strides so,
                  int64_t block_size, const int32_t* kv_offsets, const int32_t* kv_indices, int64_t nnz,
                  int causal, float scale, void* stream) {
    if (block_size != 128) return fail(FA_ERR_SHAPE, "block size %lld not supported (128)", (long long)block_size);
    if (nnz < 0) return fail(FA_ERR_LIST, "negative nnz");
    int st = check_sizes(B, H, N, d);
    if (st) return st;
    if (B == 0 || H == 0 || N == 0) return ok();
    if (!kv_offsets) return fail(FA_ERR_NULL, "kv_offsets is NULL");
    fa_attn_desc x = plain_desc(B, H, N, d, causal, scale);
    x.block_size = block_size;
    x.kv_offsets = kv_offsets;
    x.kv_indices = kv_indices;
    x.nnz = nnz;
    return fa_attn_fwd(&x, q, sq, k, sk, v, sv, o, so, lse, stream);
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
    const fa_attn_desc x = plain_desc(B, H, N, d, 0, 1.0f);
    return fa_attn_bwd_workspace_bytes(&x);
}

size_t fa_bwd_ds_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int causal) {
    const fa_attn_desc x = plain_desc(B, H, N, d, causal, 1.0f);
    return fa_attn_bwd_ds_workspace_bytes(&x);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, fa_strides sq, fa_strides sk,
           fa_strides sv, fa_strides so, fa_strides sdo, fa_strides sdq, fa_strides sdk, fa_strides sdv, int causal,
           float scale, void* workspace, size_t workspace_bytes, void* stream) {
    const fa_attn_desc x = plain_desc(B, H, N, d, causal, scale);
    return fa_attn_bwd(&x, q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv, workspace,
                       workspace_bytes, stream);
}

int fa_transpose_block_lists(int64_t n_blocks, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                             int32_t* t_offsets, int32_t* t_indices) {
    if (n_blocks < 0 || n_blocks > kMaxDim || nnz < 0) return fail(FA_ERR_LIST, "negative or too large sizes");
    if (!offsets || !t_offsets || (nnz > 0 && (!indices || !t_indices))) return fail(FA_ERR_NULL, "NULL pointer");
    int st = fa_check_block_lists(offsets, indices, n_blocks, nnz, 0);
    if (st) return st;
    // Counting sort by key block; walking the query blocks in ascending order leaves every
    // key block's query blocks ascending.
    std::vector<int64_t> fill((size_t)n_blocks + 1, 0);
    for (int64_t t = 0; t < nnz; ++t) ++fill[(size_t)indices[t] + 1];
    for (int64_t kb = 0; kb < n_blocks; ++kb) fill[(size_t)kb + 1] += fill[(size_t)kb];
    for (int64_t kb = 0; kb <= n_blocks; ++kb) t_offsets[kb] = (int32_t)fill[(size_t)kb];
    for (int64_t qb = 0; qb < n_blocks; ++qb)
        for (int64_t t = offsets[qb]; t < offsets[qb + 1]; ++t) t_indices[fill[(size_t)indices[t]]++] = (int32_t)qb;
    return ok();
}

int fa_make_block_lists(int64_t n_blocks, int32_t window, int32_t stride, int causal, int rule, int32_t* offsets,
                        int32_t* indices, int64_t cap, int64_t* nnz) {
    if (n_blocks < 0 || n_blocks > kMaxDim) return fail(FA_ERR_SHAPE, "bad n_blocks %lld", (long long)n_blocks);
    if (window < 0 || stride < 0) return fail(FA_ERR_ARG, "window and stride must be >= 0");
    if (rule != 0 && rule != 1) return fail(FA_ERR_ARG, "rule must be 0 (strided) or 1 (fixed)");
    if (!offsets || !nnz || (cap > 0 && !indices)) return fail(FA_ERR_NULL, "NULL output pointer");
    int64_t count = 0;
    offsets[0] = 0;
    for (int64_t q = 0; q < n_blocks; ++q) {
        const int64_t hi = causal ? q : n_blocks - 1;
        const int64_t wlo = q - window < 0 ? 0 : q - window;
        const int64_t whi = q + window < hi ? q + window : hi;
        for (int64_t k = 0; k <= hi; ++k) {
            bool keep = k >= wlo && k <= whi;
            if (!keep && stride > 0) {
                if (rule == 0) {
                    const int64_t dist = q >= k ? q - k : k - q;
                    keep = dist % stride == 0;
                } else {
                    keep = k % stride == 0;
                }
            }
            if (keep) {
                if (count < cap) indices[count] = (int32_t)k;
                ++count;
            }
        }
        if (count > INT32_MAX) return fail(FA_ERR_CAPACITY, "pattern exceeds int32 offsets");
        offsets[q + 1] = (int32_t)count;
    }
    *nnz = count;
    if (count > cap) return fail(FA_ERR_CAPACITY, "indices capacity %lld, %lld needed", (long long)cap, (long long)count);
    return ok();
}

int fa_check_block_lists(const int32_t* offsets, const int32_t* indices, int64_t n_blocks, int64_t nnz, int causal) {
    if (n_blocks < 0 || nnz < 0) return fail(FA_ERR_LIST, "negative n_blocks or nnz");
    if (!offsets) return fail(FA_ERR_NULL, "offsets is NULL");
    if (nnz > 0 && !indices) return fail(FA_ERR_NULL, "indices is NULL");
    if (offsets[0] != 0) return fail(FA_ERR_LIST, "offsets[0] = %d, expected 0", offsets[0]);
    for (int64_t q = 0; q < n_blocks; ++q) {
        const int64_t lo = offsets[q], hi = offsets[q + 1];
        if (hi < lo) return fail(FA_ERR_LIST, "offsets decrease at block %lld", (long long)q);
        if (hi > nnz) return fail(FA_ERR_LIST, "offsets[%lld] = %lld exceeds nnz %lld", (long long)q + 1, (long long)hi, (long long)nnz);
        for (int64_t t = lo; t < hi; ++t) {
            const int64_t k = indices[t];
            if (k < 0 || k >= n_blocks)
                return fail(FA_ERR_LIST, "index %lld of block %lld out of range", (long long)k, (long long)q);
            if (causal && k > q)
                return fail(FA_ERR_LIST, "index %lld above causal query block %lld", (long long)k, (long long)q);
            if (t > lo && indices[t - 1] >= k)
                return fail(FA_ERR_LIST, "indices of block %lld not strictly ascending", (long long)q);
        }
    }
    if (offsets[n_blocks] != nnz)
        return fail(FA_ERR_LIST, "offsets[n_blocks] = %d differs from nnz %lld", offsets[n_blocks], (long long)nnz);
    return ok();
}

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
        case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM";
        case FA_ERR_LAYOUT: return "FA_ERR_LAYOUT";
        case FA_ERR_LIST: return "FA_ERR_LIST";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        case FA_ERR_ARG: return "FA_ERR_ARG";
        case FA_ERR_CAPACITY: return "FA_ERR_CAPACITY";
        default: return "FA_ERR_UNKNOWN";
    }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
