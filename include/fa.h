/*
 * fa.h - C ABI of the MI355X (gfx950) tiled exact attention library, libfa.so.
 *
 * What the library computes. Exact multi-head attention O = softmax(Q K^T * scale + mask) V
 * ("Flash MSA Attention Kernel Implementation: A Practical Guide for Production AI",
 * section "Why Standard Attention Broke"), evaluated tile by tile with an online softmax
 * (same page, section "The Flash Core: Tiling Over the Memory Hierarchy"), never writing
 * the N x N score matrix. Masked keys are excluded (a -inf score, never 0: same page,
 * FAQ on NaN debugging). Every call returns the exact result up to floating-point
 * rounding: bf16 inputs, fp32 accumulation, bf16 outputs, fp32 log-sum-exp.
 *
 * Tensors. Q, K, V, O, dO, dQ, dK, dV are bf16 (bfloat16, round-to-nearest-even on write)
 * device buffers of logical shape [B, H, N, d]. Element (b, h, n, c) lives at
 *     ptr + b*stride.b + h*stride.h + n*stride.n + c          (strides in elements)
 * so both (B,H,N,d) and (B,N,H,d) memory layouts are accepted (the pages use both:
 * [num_heads, N, d] in page 1's CUDA kernel, (B, T, H, D_head) in "How to Use Flash MSA
 * Kernels for Long Context", section "Step-by-Step"). Requirements (else FA_ERR_LAYOUT):
 * the head dimension is contiguous; every pointer is 16-byte aligned; every stride is a
 * multiple of 8 elements and non-negative; the token stride (stride.n) is at most 2^24
 * elements. LSE is fp32, contiguous [B, H, N], natural logarithm.
 *
 * Sizes (else FA_ERR_SHAPE): B, H, N (and H_kv, packed total) at most 2^30 each, B*H at
 * most 2^30, at most 2^30 query rows (B*H*N, or H*total when packed) per forward call,
 * 2^29 per backward call, and at most 2^31 work-items in any launch: forward
 * B*H*ceil(N/256)*512 and B*H*ceil(N/128)*256, backward B*H*ceil(N/128)*512 (with packed
 * sequences N is the longest sequence, so a batch of many sequences with one long one can
 * hit this limit before the row limit); the kernels index workgroups and grids with 32-bit
 * integers.
 *
 * Ownership and execution. The caller allocates and owns every buffer (device memory for
 * tensors, lists and workspace; host memory only where a parameter says "host"). The
 * library keeps no state between calls except a per-thread error detail string, allocates
 * nothing, launches asynchronously on the given HIP stream (a hipStream_t passed as
 * void*; NULL is the default stream) and never synchronises: outputs are valid once the
 * stream has reached the launches. There is no fallback path of any kind: a call either
 * launches the gfx950 kernels or returns an error status. Calls are thread-safe.
 *
 * Errors. Every entry point returns FA_OK (0) or one of the FA_ERR_* codes below.
 * Arguments are validated on the host before any HIP call; fa_last_error() gives a
 * human-readable detail for the calling thread's most recent failure.
 * Sizes B, H or N equal to 0 are a valid empty problem: FA_OK, nothing launched.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_NULL 1       /* a required pointer is NULL                                 */
#define FA_ERR_SHAPE 2      /* B, H or N negative or too large; sparse block size unsupported */
#define FA_ERR_HEADDIM 3    /* d is not 64 or 128                                           */
#define FA_ERR_LAYOUT 4     /* pointer or stride not 16-byte aligned, token stride > 2^24    */
#define FA_ERR_LIST 5       /* block lists fail fa_check_block_lists (host checks only)     */
#define FA_ERR_WORKSPACE 6  /* backward workspace missing or too small                      */
#define FA_ERR_HIP 7        /* HIP runtime error (no device, launch failure, ...)           */
#define FA_ERR_ARG 8        /* other invalid argument (scale not finite, bad rule, ...)     */
#define FA_ERR_CAPACITY 9   /* a host output array is too small                             */

/* Element types of q, k, v in fa_attn_desc.dtype. */
#define FA_DTYPE_BF16 0      /* bfloat16 (every entry point)                                */
#define FA_DTYPE_FP8_E4M3 1  /* OCP fp8 e4m3 with per-tensor descales (fa_attn_fwd only)    */

/* Element strides of one [B, H, N, d] tensor; the d stride is 1. */
typedef struct fa_strides {
    int64_t b;
    int64_t h;
    int64_t n;
} fa_strides;

/*
 * fa_fwd - dense or causal attention forward with log-sum-exp write-out.
 *
 * Defined by the forward tile loop of "Flash MSA Attention Kernel Implementation: A
 * Practical Guide for Production AI" (sections "The Flash Core: Tiling Over the Memory
 * Hierarchy" and "Code: A Complete Flash Attention Forward Kernel in CUDA"): for each
 * query row i, O_i = sum_j P_ij V_j with P_ij = exp(S_ij - m_i) / l_i over the allowed
 * keys j, S = scale * Q K^T. With causal != 0 a key j is allowed only if j <= i (a key
 * after the query is masked). The same page stores the per-row max m and sum l for the
 * backward; this library stores their combination LSE_i = m_i + ln(l_i).
 *
 * q, k, v : device bf16, logical [B, H, N, d], strides sq, sk, sv.
 * o       : device bf16 output, logical [B, H, N, d], strides so (may alias nothing else).
 * lse     : device fp32 output, contiguous [B, H, N].
 * B, H, N : sizes (>= 0). N may be any value; there is no tile-multiple requirement.
 * d       : head dimension, 64 or 128.
 * causal  : 0 = full attention, nonzero = causal (j <= i).
 * scale   : score multiplier, any finite float (1/sqrt(d) is the usual choice; the pages
 *           use it in every kernel). Not finite -> FA_ERR_ARG.
 * stream  : hipStream_t (NULL = default stream).
 */
FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t d,
           fa_strides sq, fa_strides sk, fa_strides sv, fa_strides so,
           int causal, float scale, void* stream);

/*
 * fa_sparse_fwd - block-sparse (Flash-MSA) attention forward with log-sum-exp write-out.
 *
 * Defined in "How Does Flash-MSA Sparse Attention Work", section "How Flash-MSA Sparse
 * Attention Works": the sequence is cut into blocks of block_size tokens and a
 * precomputed index list names, for every query block, the key blocks it attends to;
 * the mask is applied inside the tile loop, so only listed key blocks enter the online
 * softmax and unlisted ones are never loaded. The result is exact attention over the
 * allowed keys: key j is allowed for query i iff block(j) is listed for block(i) and,
 * with causal != 0, j <= i. A query row with no allowed key gets O = 0 and LSE = -inf.
 *
 * block_size : tokens per block; this version supports 128 (FA_ERR_SHAPE otherwise).
 *              The last block may be partial (N need not be a multiple).
 * kv_offsets : device int32 [nb + 1], nb = ceil(N / block_size). Query block qb lists
 *              kv_indices[kv_offsets[qb] .. kv_offsets[qb+1]).
 * kv_indices : device int32 [nnz], key block numbers, ascending and unique per query block.
 * nnz        : number of elements of kv_indices.
 * The lists are shared by every batch and head. They must pass fa_check_block_lists;
 * the kernels stay in bounds whatever the list contents (offsets are clamped to
 * [0, nnz], indices outside [0, nb), and with causal masking indices above the query
 * block, are skipped), but duplicated or unsorted entries give undefined results.
 * Other arguments as in fa_fwd.
 */
FA_API int fa_sparse_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t N, int64_t d,
                  fa_strides sq, fa_strides sk, fa_strides sv, fa_strides so,
                  int64_t block_size, const int32_t* kv_offsets, const int32_t* kv_indices,
                  int64_t nnz, int causal, float scale, void* stream);

/*
 * fa_bwd_workspace_bytes - device workspace fa_bwd needs: two fp32 per query row (the row
 * dot products D_i = dO_i . O_i and the row's LSE converted for base-2 exponentials),
 * B*H*N*8 bytes rounded up to 256.
 */
FA_API size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * fa_bwd_ds_workspace_bytes - the workspace that lets fa_bwd keep dS instead of recomputing
 * it (see fa_bwd): fa_bwd_workspace_bytes(...) plus B*H*T*32768 bytes, T = n(n+1)/2 causal or
 * n*n otherwise with n = ceil(N / 128) (one bf16 128 x 128 tile per pair of key and query
 * blocks the backward visits). 0 where that mode does not exist (d = 64, empty problems).
 */
FA_API size_t fa_bwd_ds_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int causal);

/*
 * fa_bwd - attention backward by recomputation from the stored log-sum-exp.
 *
 * Defined in "Flash MSA Attention Kernel Implementation: A Practical Guide for Production
 * AI", section "The Backward Pass: The Real Beast": the forward keeps O and the softmax
 * statistics instead of the N x N matrix; the backward recomputes P_ij = exp(S_ij - LSE_i)
 * tile by tile and forms dP = dO V^T, dS = P o (dP - D) with D_i = sum_j P_ij dP_ij
 * (= dO_i . O_i), dV = P^T dO, and, through S = scale * Q K^T, dQ = scale * dS K and
 * dK = scale * dS^T Q. Accumulation is fp32; dq, dk, dv are written as bf16.
 *
 * q, k, v, o, dout : device bf16 inputs (o and lse are the forward's outputs for q, k, v).
 * lse              : device fp32 [B, H, N] from fa_fwd with the same causal and scale.
 * dq, dk, dv       : device bf16 outputs, logical [B, H, N, d].
 * workspace        : device buffer of at least fa_bwd_workspace_bytes(...) bytes,
 *                    16-byte aligned; its contents on entry are ignored.
 * Other arguments as in fa_fwd. The kernels are deterministic (no atomics).
 *
 * Two schedules compute this function. With workspace_bytes >= fa_bwd_ds_workspace_bytes(...)
 * (> 0) the dK/dV pass, which forms every dS tile for the dK product anyway, also writes it
 * (bf16, as rounded for that product) into the workspace, and the dQ pass reads it back: one
 * matrix product per tile instead of three. With a smaller workspace the dQ pass recomputes
 * S, P, dP and dS from Q, K, V, dO and the LSE. Both are exact up to rounding (the
 * recomputed dS can differ from the stored one in the last bits of its fp32 value before
 * bf16 rounding); each is deterministic.
 */
FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int64_t B, int64_t H, int64_t N, int64_t d,
           fa_strides sq, fa_strides sk, fa_strides sv, fa_strides so, fa_strides sdo,
           fa_strides sdq, fa_strides sdk, fa_strides sdv,
           int causal, float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_attn_desc - the general problem description taken by fa_attn_fwd, fa_attn_bwd and
 * fa_attn_bwd_workspace_bytes. It extends the calls above in three ways, each of which
 * leaves the computed function exact attention:
 *
 * Grouped key/value heads ("Flash MSA Attention Kernel Implementation: A Practical Guide
 * for Production AI", FAQ on grouped-query and multi-query attention: the tiling is the
 * same, K and V heads are shared by several query heads). K, V, dK and dV have H_kv heads;
 * query head h reads K/V head h / (H / H_kv) (consecutive query heads share a K/V head;
 * H_kv = H is plain multi-head attention, H_kv = 1 multi-query attention). dK and dV of a
 * K/V head are the sums over the query heads that read it.
 *
 * Packed variable-length sequences (same page, section "The Production Pipeline: From
 * Kernel to Service", on request batching: the softmax of every tile ignores padding; and
 * "How to Use Flash MSA Kernels for Long Context", FAQ on flash-batch inference, which
 * points to a variable-length entry point for sequences of different lengths). With
 * cu_seqlens != NULL the B sequences are packed one after another along the token axis of
 * [total, heads, d] tensors: sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1 and
 * attends only to itself (causal positions and block numbers count from its first row).
 * Element (row r, head h, c) of a packed tensor lives at ptr + r*stride.n + h*stride.h + c;
 * stride.b is unused. N is then an upper bound on every sequence's length (the longest
 * sequence); rows of a longer sequence past N are not computed. LSE (and the backward
 * workspace) are fp32 [H, total]. The kernels clamp the offsets to [0, total], so any
 * offset values keep every access inside the tensors; the caller must still pass
 * ascending offsets with cu_seqlens[0] = 0 and cu_seqlens[B] <= total to get results.
 *
 * Block-sparse masks (as in fa_sparse_fwd) with kv_offsets != NULL. For the backward
 * ("How Does Flash-MSA Sparse Attention Work", FAQ on training: the backward reuses the
 * forward's tiling and masking and recomputes the scores) the dK/dV pass also needs the
 * same pattern seen from the key side: q_offsets / q_indices, for every key block the
 * ascending query blocks whose lists name it, as produced by fa_transpose_block_lists.
 * With packed sequences the lists apply to every sequence, block numbers counted from the
 * sequence's first row; they must cover ceil(N / block_size) blocks.
 *
 * FP8 inputs (forward only; "How to Use Flash MSA Kernels for Long Context", FAQ on FP16
 * vs FP8, names FP8 attention; "Flash MSA Attention Kernel Implementation: A Practical
 * Guide for Production AI", section "Optimization Tricks That Actually Matter", runs the
 * tile's matrix products in FP8 and keeps the softmax in fp32). With
 * dtype = FA_DTYPE_FP8_E4M3, q, k and v hold OCP e4m3 codes (1 byte, strides in bytes,
 * multiples of 16) and each tensor's real values are code x descale (q_descale, k_descale,
 * v_descale; finite). The scores Q K^T are computed on the fp8 matrix cores from the codes
 * (exact products, fp32 accumulation) and scaled by scale * q_descale * k_descale; V is
 * widened to bf16 exactly and P V runs as in the bf16 path, O is multiplied by v_descale.
 * The result is exact attention over the dequantized inputs to the same rounding as the
 * bf16 path: o stays bf16, lse fp32. The descales are ignored for bf16.
 */
typedef struct fa_attn_desc {
    int64_t B;                  /* sequences (batch)                                          */
    int64_t H;                  /* query heads                                                */
    int64_t H_kv;               /* key/value heads, H % H_kv == 0 (else FA_ERR_SHAPE)          */
    int64_t N;                  /* tokens per sequence; packed: upper bound on every length    */
    int64_t d;                  /* head dimension, 64 or 128                                   */
    int causal;                 /* nonzero: key j allowed for query i only if j <= i           */
    float scale;                /* score multiplier, finite                                    */
    const int32_t* cu_seqlens;  /* NULL, or device int32 [B + 1]: packed sequence offsets     */
    int64_t total;              /* packed mode: rows of the packed tensors                     */
    int64_t block_size;         /* block-sparse mode: 128                                      */
    const int32_t* kv_offsets;  /* NULL (dense), or device int32 [nb + 1]: query-side lists    */
    const int32_t* kv_indices;  /* device int32 [nnz]                                          */
    int64_t nnz;                /* entries of kv_indices (and of q_indices)                    */
    const int32_t* q_offsets;   /* backward, block-sparse: device int32 [nb + 1], key side     */
    const int32_t* q_indices;   /* device int32 [nnz]                                          */
    int dtype;                  /* FA_DTYPE_BF16 or FA_DTYPE_FP8_E4M3 (forward only)           */
    float q_descale;            /* fp8: real value = code x descale                           */
    float k_descale;
    float v_descale;
} fa_attn_desc;

/*
 * fa_attn_fwd - forward with log-sum-exp write-out for any fa_attn_desc (the function of
 * fa_fwd, or of fa_sparse_fwd when kv_offsets != NULL, with grouped heads and packed
 * sequences as described there). q, o: H heads; k, v: H_kv heads. lse: fp32 [B, H, N]
 * contiguous, or [H, total] when packed. Errors as in fa_fwd and fa_sparse_fwd; FA_ERR_SHAPE
 * also for H not a multiple of H_kv or a bad total; FA_ERR_NULL for NULL desc; FA_ERR_ARG for
 * an unknown dtype or a descale that is not finite; FA_ERR_LAYOUT for fp8 strides that are
 * not multiples of 16 bytes.
 */
FA_API int fa_attn_fwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk,
                       const void* v, fa_strides sv, void* o, fa_strides so, float* lse, void* stream);

/*
 * fa_attn_fwd_visits - fa_attn_fwd for a block-sparse desc (kv_offsets != NULL) that also
 * records which tiles each query block took into its softmax, so that a caller can check
 * that every query block visits exactly the key blocks its list names, less the ones the
 * causal mask or the sequence end removes ("How Does Flash-MSA Sparse Attention Work",
 * section "How Flash-MSA Sparse Attention Works": the kernel walks a query block's index
 * list and nothing else; unlisted blocks are never loaded). Same outputs as fa_attn_fwd,
 * bit for bit.
 * visits : device uint8 [B * H, nnz, 2] (b-major: row b * H + h), written by the call: it
 *          is zero-filled on `stream` (an asynchronous memset), then byte
 *          [(b * H + h) * 2 * nnz + 2 * e + half] is set to 1 when sequence b, head h took
 *          the 64 keys 128 * kv_indices[e] + 64 * half .. +63 of list entry e into the softmax
 *          of its query block (the block whose list range holds e). Skipped entries (index
 *          out of range, above the diagonal under causal masking, or a half past the
 *          sequence end or past the query block's last row) stay 0.
 * Errors as in fa_attn_fwd; FA_ERR_NULL for visits == NULL; FA_ERR_ARG for a dense desc.
 */
FA_API int fa_attn_fwd_visits(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k,
                              fa_strides sk, const void* v, fa_strides sv, void* o, fa_strides so, float* lse,
                              uint8_t* visits, void* stream);

/*
 * fa_attn_bwd_workspace_bytes - device workspace fa_attn_bwd needs: two fp32 per query row
 * and query head (H * B * N, or H * total when packed) times 8 bytes, rounded up to 256.
 * 0 for an empty problem or a NULL desc.
 */
FA_API size_t fa_attn_bwd_workspace_bytes(const fa_attn_desc* desc);

/*
 * fa_attn_bwd_ds_workspace_bytes - the workspace with which fa_attn_bwd keeps dS (the
 * stored-dS schedule described at fa_bwd): fa_attn_bwd_workspace_bytes(desc), plus (block-
 * sparse) nnz int32 rounded up to 256 bytes, plus B*H*T*32768 bytes of bf16 dS tiles with
 * T = n(n+1)/2 dense causal, n*n dense non-causal (n = ceil(N / 128), N the longest
 * sequence when packed) or nnz block-sparse. 0 where that schedule does not exist (head
 * dimension 64, fp8, nnz = 0, empty problems, or more than 2^56 bytes).
 */
FA_API size_t fa_attn_bwd_ds_workspace_bytes(const fa_attn_desc* desc);

/*
 * fa_attn_bwd - backward by recomputation (the function of fa_bwd) for any fa_attn_desc:
 * grouped heads (dk, dv have H_kv heads and sum over their query heads), packed sequences,
 * and block-sparse masks (kv_offsets / kv_indices for dQ, q_offsets / q_indices for dK and
 * dV; both describe the same pattern, which must be the one the forward used). o and lse
 * are the forward's outputs for the same desc. The kernels are deterministic (no atomics).
 * A workspace of at least fa_attn_bwd_ds_workspace_bytes(desc) (> 0) selects the stored-dS
 * schedule, as at fa_bwd; block-sparse, that schedule takes a query-side entry's dS from the
 * key-side entry that names the same pair of blocks, so with lists that do not describe the
 * same pattern, entries without such a mate contribute nothing to dQ.
 * Errors as in fa_bwd; FA_ERR_NULL also when block-sparse and q_offsets is NULL; FA_ERR_ARG
 * when dtype is not FA_DTYPE_BF16 (the backward is bf16).
 */
FA_API int fa_attn_bwd(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk,
                       const void* v, fa_strides sv, const void* o, fa_strides so, const void* dout,
                       fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk, fa_strides sdk,
                       void* dv, fa_strides sdv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_attn_bwd_noalloc - fa_attn_bwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, function, kernels and results (bit for bit) as fa_attn_bwd with a workspace
 * smaller than fa_attn_bwd_ds_workspace_bytes (dQ by recomputation), without the workspace: the per-row values D_i it needs live in a device array the library owns, one
 * per GPU, of FA_NOALLOC_WORKSPACE_BYTES, held until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine). Its first call on a device
 * looks up that device's array once (with the device current); later calls reuse it.
 *
 * Limit: problems whose workspace (fa_attn_bwd_workspace_bytes) exceeds
 * FA_NOALLOC_WORKSPACE_BYTES, i.e. more than 4,194,304 (query head, row) pairs, return
 * FA_ERR_WORKSPACE. The array is fully rewritten by every call before it is read, so no
 * state carries over between calls, but every call on one GPU shares it: calls that
 * overlap on one GPU (different streams, or threads without ordering) race and give wrong
 * results; serialize them, e.g. on one stream.
 * Errors as in fa_attn_bwd.
 */
#define FA_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
FA_API int fa_attn_bwd_noalloc(const fa_attn_desc* desc, const void* q, fa_strides sq, const void* k, fa_strides sk,
                               const void* v, fa_strides sv, const void* o, fa_strides so, const void* dout,
                               fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk, fa_strides sdk,
                               void* dv, fa_strides sdv, void* stream);

/*
 * fa_transpose_block_lists - host: the key-side form of CSR block lists. For every key
 * block kb, t_indices[t_offsets[kb] .. t_offsets[kb+1]) lists in ascending order the query
 * blocks whose lists name kb (the walk the backward's dK/dV pass makes; "How Does
 * Flash-MSA Sparse Attention Work", FAQ on training). The input must pass
 * fa_check_block_lists (causal = 0), else FA_ERR_LIST. All pointers host; t_offsets has
 * n_blocks + 1 entries, t_indices nnz.
 */
FA_API int fa_transpose_block_lists(int64_t n_blocks, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                                    int32_t* t_offsets, int32_t* t_indices);

/*
 * fa_make_block_lists - host generator of the block-sparse pattern used with fa_sparse_fwd.
 *
 * "How Does Flash-MSA Sparse Attention Work", section "How Flash-MSA Sparse Attention
 * Works", names a local window of +-W positions and the fixed "strided" pattern of Child
 * et al. (2019). At block granularity, query block q lists the union of
 *   window : key blocks k with |q - k| <= window (k <= q when causal), and
 *   stride : rule 0 ("strided") key blocks with |q - k| divisible by stride,
 *            rule 1 ("fixed")   key blocks with k divisible by stride
 *            (k <= q when causal; stride 0 disables the strided part),
 * sorted ascending without repeats, in CSR form.
 *
 * offsets : host int32 [n_blocks + 1] output.
 * indices : host int32 [cap] output. If the pattern needs more than cap entries the
 *           call returns FA_ERR_CAPACITY and *nnz holds the needed count.
 * nnz     : host output, number of entries written (or needed).
 */
FA_API int fa_make_block_lists(int64_t n_blocks, int32_t window, int32_t stride, int causal, int rule,
                        int32_t* offsets, int32_t* indices, int64_t cap, int64_t* nnz);

/*
 * fa_check_block_lists - host validation of CSR block lists (all pointers host).
 * FA_OK iff offsets[0] == 0, offsets are non-decreasing, offsets[n_blocks] == nnz, every
 * index is in [0, n_blocks), each query block's indices are strictly ascending, and,
 * when causal != 0, no index exceeds its query block. Otherwise FA_ERR_LIST (FA_ERR_NULL
 * for null pointers with n_blocks > 0).
 */
FA_API int fa_check_block_lists(const int32_t* offsets, const int32_t* indices, int64_t n_blocks,
                         int64_t nnz, int causal);

/* Static string naming a status code ("FA_OK", "FA_ERR_SHAPE", ...). Never NULL. */
FA_API const char* fa_status_str(int status);

/* Detail of the calling thread's most recent failed call ("" if none). Never NULL. */
FA_API const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
