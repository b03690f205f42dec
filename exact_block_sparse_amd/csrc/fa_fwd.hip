// Attention forward for gfx950: dense, causal and block-sparse (Flash-MSA) variants.
//
// Method: the tiled forward with an online softmax of "Flash MSA Attention Kernel
// Implementation: A Practical Guide for Production AI" (sections "The Flash Core: Tiling
// Over the Memory Hierarchy" and "Code: A Complete Flash Attention Forward Kernel in
// CUDA"): a workgroup owns a block of query rows and walks the key/value tiles, keeping a
// running max m and running sum l per row and rescaling its output accumulator when m
// grows. Causal masking skips tiles past the query block and applies -inf inside the
// diagonal tile (same page, "Optimization Tricks That Actually Matter"). The block-sparse
// variant walks only the key blocks named by a precomputed per-query-block index list
// ("How Does Flash-MSA Sparse Attention Work", section "How Flash-MSA Sparse Attention
// Works"): unlisted blocks are never loaded and never enter the softmax.
//
// MI355X mapping (design of this file, not the pages'):
// * each wave64 owns 32 query rows. Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16, so the 32 scores of a query over a 32-key block sit in one
//   lane and its partner lane 32 away: the row max needs one cross-half exchange
//   (v_permlane32_swap) and the row sum none until the end;
// * key/value tiles of 64 keys go through LDS, fetched with raw buffer loads whose hardware
//   range check zero-fills rows past the sequence end. K and V are stored row-major; P.V
//   reads its V^T operands with the transposing LDS read ds_read_b64_tr_b16. bf16 tiles at
//   head dimension 128 are loaded straight into LDS, unpadded, with 16-byte chunks XOR-
//   swizzled per row; the other cases (head dimension 64, fp8) are staged through registers
//   into padded rows (272-byte K rows, 320-byte V rows). Both layouts keep every LDS read
//   free of bank conflicts on the 64-bank LDS;
// * the running max is set by a row's first tile and raised only when a tile's
//   probabilities pass 2^8 (in the exp2 domain), detected from the tile's row-sum parts
//   rather than from a tile max; the O rescale stays rare and no step computes a max over
//   its scores. The result is the same function; only the reference point of the
//   exponentials moves;
// * O^T = V^T P^T accumulates in fp32 registers; P is rounded to bf16 only as an MFMA
//   operand; exp is computed as exp2 with scale*log2(e) folded into one FMA;
// * dense kernel ("ping-pong"): 8 waves and 256 query rows per workgroup, in two groups of
//   four that alternate phase by phase: while one group runs its matrix products (P.V of
//   the previous tile, then S of the current one) the other runs its softmax on the vector
//   ALU. Each SIMD holds one wave of each group, so one wave's products and the other's
//   softmax are issued side by side (they overlap only in part: each slows the other).
//   Tiles cycle through four LDS stages (loaded into LDS) or three (register-staged), so
//   loads run two tiles ahead;
// * sparse kernel: 4 waves and one 128-row block per workgroup (the list granularity),
//   two workgroups per CU, each step in one go, two LDS stages, workgroups in plain order;
// * the LSE is written in natural log, O as bf16.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBK = 64;            // keys per pipeline step
constexpr int kSparseBlock = 128;
constexpr float kSumLimit = 0x1p8f;     // largest part of a tile's row sum allowed without a rescale

template <int D, bool F8 = false>
struct Cfg {
    // K tile row stride: bf16 rows of D elements padded to D + 8 (272 bytes at D = 128), or
    // fp8 rows of D bytes padded by 16 (144 bytes): both keep 16-byte row reads conflict-free.
    static constexpr int KROWB = F8 ? D + 16 : 2 * (D + 8);
    static constexpr int KS = KROWB / 2;         // K tile row stride in LDS (uint16 units)
    static constexpr int VS = D + 32;            // V tile row stride in LDS (bf16 elements)
    static constexpr int KEL = kBK * KS;
    static constexpr int VEL = kBK * VS;
    static constexpr int BUF = KEL + VEL;        // elements per pipeline stage
    static constexpr int CR = D / 8;             // 16-byte chunks per row
    static constexpr int KSTEPS = D / 16;        // MFMA k-steps over the head dimension (bf16)
    static constexpr int KSTEPS8 = D / 64;       // ... with fp8 operands
    static constexpr int CR8 = D / 16;           // 16-byte chunks per fp8 row
    static constexpr int CB = D / 32;            // 32-wide head-dimension blocks of O
    static_assert((BUF * 2) % 16 == 0, "stage size must keep 16-byte alignment");
};

struct Params {
    const void* q;    // bf16 or fp8 (e4m3) elements
    const void* k;
    const void* v;
    uint16_t* o;
    float* lse;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, osb, osh, osn;
    int B, H, N;      // N: rows per sequence (packed: the longest sequence's bound)
    int G;            // query heads per K/V head
    const int32_t* cu;   // packed sequence offsets [B + 1], or nullptr
    int64_t total;       // packed rows
    int nqb;          // query blocks (of the workgroup's row count) per head
    int gh;           // (head, sequence) pairs whose query blocks are ordered together
    float c;          // scale * log2(e) (fp8: times the Q and K descales)
    float vdesc;      // V descale (fp8), 1 for bf16
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    int64_t nnz;
    uint8_t* visits;  // block-sparse visit log [B * H, nnz, 2], or nullptr
};

// Per-thread staging of one K/V step: 16-byte row chunks of K and V.
template <int D, int NT>
struct Stage {
    using C = Cfg<D>;
    static constexpr int KCH = kBK * C::CR / NT;
    static_assert(KCH >= 1 && kBK * C::CR % NT == 0, "chunks must divide evenly");
    u32x4 k[KCH];
    u32x4 v[KCH];
    uint32_t koff[KCH];   // byte offsets (relative to the step's first row), fixed per thread
    uint32_t voff[KCH];
    int klds[KCH];        // LDS element offsets of the chunks
    int vlds[KCH];

    __device__ void init(int tid, int64_t ksn, int64_t vsn) {
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            const int id = tid + j * NT;
            const int row = id / C::CR, ch = id % C::CR;
            koff[j] = (uint32_t)(((int64_t)row * ksn + 8 * ch) * 2);
            voff[j] = (uint32_t)(((int64_t)row * vsn + 8 * ch) * 2);
            klds[j] = row * C::KS + 8 * ch;
            vlds[j] = C::KEL + row * C::VS + 8 * ch;
        }
    }
    __device__ void load(const uint16_t* kbase, const uint16_t* vbase, int64_t ksn, int64_t vsn, int kt0, int N) {
        const auto kr = make_rsrc(kbase + (int64_t)kt0 * ksn, rows_bytes(kt0, N, ksn, D, kBK));
        const auto vr = make_rsrc(vbase + (int64_t)kt0 * vsn, rows_bytes(kt0, N, vsn, D, kBK));
#pragma unroll
        for (int j = 0; j < KCH; ++j) k[j] = buf_load16(kr, koff[j], 0);
#pragma unroll
        for (int j = 0; j < KCH; ++j) v[j] = buf_load16(vr, voff[j], 0);
    }
    __device__ void store(uint16_t* buf) const {
#pragma unroll
        for (int j = 0; j < KCH; ++j) *reinterpret_cast<u32x4*>(buf + klds[j]) = k[j];
#pragma unroll
        for (int j = 0; j < KCH; ++j) *reinterpret_cast<u32x4*>(buf + vlds[j]) = v[j];
    }
};

// Per-thread staging of one K/V step from fp8 (e4m3) tensors: 16-byte row chunks. K stays
// fp8 in LDS (the scores run on the fp8 MFMA); V is widened to bf16 on its way to LDS (an
// exact conversion) so that P.V is the bf16 product of the bf16 path.
template <int D, int NT>
struct Stage8 {
    using C = Cfg<D, true>;
    static constexpr int TOT = kBK * C::CR8;           // chunks per tile and tensor
    static constexpr int CH = (TOT + NT - 1) / NT;
    static_assert(TOT % NT == 0 || NT % TOT == 0, "chunks must divide evenly");
    u32x4 k[CH];
    u32x4 v[CH];
    uint32_t koff[CH], voff[CH];
    int klds[CH], vlds[CH];
    bool ok[CH];

    __device__ void init(int tid, int64_t ksn, int64_t vsn) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int id = tid + j * NT;
            ok[j] = id < TOT;
            const int row = (id % TOT) / C::CR8, ch = id % C::CR8;
            koff[j] = (uint32_t)((int64_t)row * ksn + 16 * ch);
            voff[j] = (uint32_t)((int64_t)row * vsn + 16 * ch);
            klds[j] = row * C::KS + 8 * ch;
            vlds[j] = C::KEL + row * C::VS + 16 * ch;
        }
    }
    __device__ void load(const uint8_t* kbase, const uint8_t* vbase, int64_t ksn, int64_t vsn, int kt0, int N) {
        const auto kr = make_rsrc(kbase + (int64_t)kt0 * ksn, rows_bytes(kt0, N, ksn, D, kBK, 1));
        const auto vr = make_rsrc(vbase + (int64_t)kt0 * vsn, rows_bytes(kt0, N, vsn, D, kBK, 1));
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (ok[j]) k[j] = buf_load16(kr, koff[j], 0);
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (ok[j]) v[j] = buf_load16(vr, voff[j], 0);
    }
    __device__ void store(uint16_t* buf) const {
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (ok[j]) *reinterpret_cast<u32x4*>(buf + klds[j]) = k[j];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (ok[j]) {
                u32x4 lo, hi;
                fp8x16_to_bf16(v[j], lo, hi);
                *reinterpret_cast<u32x4*>(buf + vlds[j]) = lo;
                *reinterpret_cast<u32x4*>(buf + vlds[j] + 8) = hi;
            }
    }
};

template <int D, int NT, bool F8> struct StageOf { using type = Stage<D, NT>; };
template <int D, int NT> struct StageOf<D, NT, true> { using type = Stage8<D, NT>; };
template <bool F8> struct ElemOf { using type = uint16_t; };
template <> struct ElemOf<true> { using type = uint8_t; };

// Q rows as MFMA B operands (column = query, k-group = half): bf16, 8 values per 16-wide
// k-step, or fp8, 32 values per 64-wide k-step.
template <int D, bool F8> struct QFrag { bf16x8 v[D / 16]; };
template <int D> struct QFrag<D, true> { i32x8 v[D / 64]; };

// Per-wave state of 32 query rows.
template <int D, bool F8>
struct Rows {
    using C = Cfg<D, F8>;
    QFrag<D, F8> qf;        // Q rows as B operands
    f32x16 o[C::CB];        // O^T accumulators
    float m_run;            // running max (exp2 domain)
    float l4[4];            // this lane's row sum in four interleaved parts (short add chains)
    float m_neg;            // -m_run, or 0 while m_run is -inf (the exponent's offset)
    float t_thr;            // a part of a tile's row sum above it raises m_run: -1 while
                            // m_run is -inf (every tile then sets it), else kSumLimit
    f32x16 s[2];            // scores of the current 64-key step (two 32-key blocks)
    bf16x8 pb[2][2];        // probabilities of the current step as bf16 B operands
};

// The kernels score with a non-negative scale: for a negative one they flip the sign of
// their Q fragments (exact in bf16 and e4m3: the sign bit alone) and use its magnitude, so
// the scores come out exactly negated and score x |scale| is bit for bit score x scale.
// Then the largest scaled score of a tile is always its largest raw score, scaled.
template <int D, bool F8>
__device__ __forceinline__ float signed_scale(Rows<D, F8>& w, float c) {
    if (c >= 0.0f) return c;
#pragma unroll
    for (int j = 0; j < (int)(sizeof(w.qf.v) / sizeof(w.qf.v[0])); ++j) {
        if constexpr (F8) w.qf.v[j] ^= (int)0x80808080u;
        else w.qf.v[j] = as_bf16x8(__builtin_bit_cast(u32x4, w.qf.v[j]) ^ 0x80008000u);
    }
    return -c;
}

// S^T = K Q^T for one 64-key step. Row i of each 32-key block; the two blocks' chains alternate.
template <int D, bool F8>
__device__ __forceinline__ void scores(const uint16_t* buf, Rows<D, F8>& w, int i, int hf) {
    using C = Cfg<D, F8>;
    w.s[0] = f32x16{};
    w.s[1] = f32x16{};
    if constexpr (!F8) {
        const uint16_t* kr = buf + i * C::KS + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                w.s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(kr + 32 * kb * C::KS + 16 * ks), w.qf.v[ks], w.s[kb]);
        // Issue the K reads several products ahead of their use, so that the LDS latency is
        // covered by earlier products rather than waited for before each one.
        constexpr int N = 2 * C::KSTEPS, AHEAD = N < 6 ? N : 6;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
        for (int k = 0; k < N - AHEAD; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    } else {
        // lane (key i, half hf) reads the 32 bytes 32*hf + 64*ks .. of its K row
        const uint8_t* kr = reinterpret_cast<const uint8_t*>(buf) + i * C::KROWB + 32 * hf;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS8; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint8_t* a = kr + 32 * kb * C::KROWB + 64 * ks;
                w.s[kb] = mfma32_f8(join8(*reinterpret_cast<const u32x4*>(a), *reinterpret_cast<const u32x4*>(a + 16)),
                                    w.qf.v[ks], w.s[kb]);
            }
    }
}

// Probabilities of one step against the current running max, their sums in the lane's four
// row-sum parts (t4, this tile only) and their bf16 MFMA operands.
template <int D, bool F8>
__device__ __forceinline__ void probs(Rows<D, F8>& w, float ce, float (&t4)[4]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            float pr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pr[e] = fast_exp2(fmaf(w.s[kb][8 * st + e], ce, w.m_neg));
                t4[e & 3] = (kb == 0 && st == 0 && e < 4) ? pr[e] : t4[e & 3] + pr[e];
            }
            w.pb[kb][st] = pack8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
        }
}

// Online softmax update for one step: mask (diagonal or tail tiles only), probabilities,
// fp32 row sum, bf16 operands, and the running max. `masked` is uniform across the wave.
//
// The running max is only a reference point for the exponent: any value at or below the
// true row max gives the same normalised result, as long as no probability overflows. So
// it is set from the first tile that has a key and afterwards raised only when a part of a
// tile's row sum passes 2^8. That is detected from the tile's row-sum parts, which bound
// each of their terms, instead of a tile max over all 32 scores every step; on the rare
// tile that trips it the scores are still in registers and the step is redone against its
// own max. Range alone would allow far more (2^64 keeps fp32 and bf16 safe), but a row
// dominated by a few keys is only as accurate as their bf16-rounded probabilities, which
// are exact (1) for the key that set the max: letting the max lag far behind made such
// rows' outputs less accurate, so the limit keeps the old bound on each probability.
template <int D, bool F8, bool CAUSAL>
__device__ __forceinline__ void softmax(Rows<D, F8>& w, bool masked, int kt0, int qrow, int N, float c,
                                        int hf) {
    using C = Cfg<D, F8>;
    // In masked tiles the scores are scaled here and masked keys (past the sequence end,
    // or after the query under causal masking) become -inf; the exponent below then uses
    // a unit multiplier. Elsewhere the scale is folded into the exponent's FMA.
    float ce = c;
    if (masked) {
        // Element (kb, r) holds key kt0 + 4 hf + 32 kb + 8 (r / 4) + r % 4 (acc_row): one
        // per-lane limit turns both tests (key < N, causal key <= qrow) into a single
        // compare with a compile-time offset.
        int lim = N - 1 - kt0 - 4 * hf;
        if (CAUSAL) lim = min(lim, qrow - kt0 - 4 * hf);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rel = 32 * kb + 8 * (r >> 2) + (r & 3);
                w.s[kb][r] = rel <= lim ? w.s[kb][r] * c : kNegInf;
            }
        ce = 1.0f;
    }
    // The row sum is taken in fp32 over the unrounded probabilities (the LSE needs it);
    // P is rounded to bf16 only as the MFMA operand.
    float t4[4];
    probs(w, ce, t4);
    const float tmax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(t4[0], t4[1]),
                                                     __builtin_elementwise_maximum(t4[2], t4[3]));
    if (__any(tmax > w.t_thr)) {
        // Tile max of the scaled scores: the scale is never negative here (the kernels flip
        // the sign of Q instead), so it is the scaled max of the raw scores. The
        // NaN-propagating maximum needs no quieting of its inputs (a NaN row keeps its max).
        float mt = __builtin_elementwise_maximum(w.s[0][0], w.s[1][0]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = __builtin_elementwise_maximum(mt, w.s[kb][r]);
        mt = pair_max(mt);
        mt *= ce;
        const bool need = mt > w.m_run;
        const float m_new = need ? mt : w.m_run;
        const float alpha = need ? fast_exp2(w.m_run - m_new) : 1.0f;
        w.m_run = m_new;
        w.m_neg = (m_new == kNegInf) ? 0.0f : -m_new;
        w.t_thr = (m_new == kNegInf) ? -1.0f : kSumLimit;
#pragma unroll
        for (int j = 0; j < 4; ++j) w.l4[j] *= alpha;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.o[cb][r] *= alpha;
        probs(w, ce, t4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) w.l4[j] += t4[j];
}

// O^T += V^T P^T. B element e of k-step st in half hf is key 16*st + 8*(e/4) + 4*hf + e%4 of
// the 32-key block (the accumulator row order). The A operand (V^T: row = head-dim column,
// k = key) comes from the row-major V tile through two transposing reads: lane j of each
// 16-lane group addresses V[key0 + j/4][col0 + 4*(j%4)] and receives the 4 keys of column
// col0 + j.
template <int D, bool F8>
__device__ __forceinline__ void pv(const uint16_t* buf, Rows<D, F8>& w, int i, int hf) {
    using C = Cfg<D, F8>;
    const int g16 = (i >> 4) & 1, j16 = i & 15;
    const uint16_t* vr = buf + C::KEL + (4 * hf + (j16 >> 2)) * C::VS + 16 * g16 + 4 * (j16 & 3);
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
        bf16x8 a[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const uint16_t* p0 = vr + (32 * kb + 16 * st) * C::VS + 32 * cb;
                const u32x2 lo = lds_read_tr4(p0);
                const u32x2 hi = lds_read_tr4(p0 + 8 * C::VS);
                u32x4 x;
                x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
                a[kb][st] = as_bf16x8(x);
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st) w.o[cb] = mfma32(a[kb][st], w.pb[kb][st], w.o[cb]);
    }
    // Keep about ten transposing reads in flight ahead of the products (two per product),
    // so the LDS latency is covered; left to itself the scheduler may issue each product
    // right behind its own two reads when register pressure around the call is high.
    constexpr int READS = 8 * C::CB, MF = 4 * C::CB, AHEAD = 10, PAIRS = (READS - AHEAD) / 2;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int k = 0; k < PAIRS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF - PAIRS, 0);
}

// Empty running state of a wave's rows: O = 0, no running max, zero row sums.
template <int D, bool F8>
__device__ __forceinline__ void init_rows(Rows<D, F8>& w) {
    using C = Cfg<D, F8>;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) w.o[cb] = f32x16{};
    w.m_run = kNegInf;
    w.m_neg = 0.0f;
    w.t_thr = -1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) w.l4[j] = 0.0f;
}

template <int D, bool F8>
__device__ __forceinline__ void load_q(Rows<D, F8>& w, const typename ElemOf<F8>::type* qp, int64_t qsn, int qrow,
                                       int N, int hf) {
    using C = Cfg<D, F8>;
    if constexpr (!F8) {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            w.qf.v[ks] = as_bf16x8(load16(qp + (int64_t)qrow * qsn + 16 * ks + 8 * hf, qrow < N));
    } else {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS8; ++ks) {
            const uint8_t* a = qp + (int64_t)qrow * qsn + 64 * ks + 32 * hf;
            w.qf.v[ks] = join8(load16b(a, qrow < N), load16b(a + 16, qrow < N));
        }
    }
    init_rows(w);
}

// Row pitch of the epilogue's LDS staging area (bytes; the 16-byte pad spreads the row writes
// of a wave evenly over the banks) and the area of one wave (its 32 rows).
template <int D> constexpr uint32_t kEpiPitch = 2 * D + 16;
template <int D> constexpr uint32_t kEpiWaveB = 32 * kEpiPitch<D>;

// O = O^T / l as bf16; LSE = (m + log2 l) * ln 2. `obase` and `lbase` point at row 0 of the
// sequence's head. A lane holds 4-value pieces of one row, so stored directly every store
// instruction would write 64 scattered 8-byte pieces; instead the wave writes its 32 rows
// into its own LDS area (`lds_wave`: all LDS reads of the loop are done, which the loop's
// last barrier guarantees) and stores whole rows from there, 16 lanes per row, 16 bytes
// each, non-temporal (the kernel never reads O back). The wave only reads back what it wrote, so no barrier is needed (a wave's LDS
// operations complete in order; the wait below is only for the compiler's benefit).
template <int D, bool F8>
__device__ __forceinline__ void epilogue(const Rows<D, F8>& w, uint16_t* obase, int64_t osn, float* lbase, int qrow,
                                         int N, int hf, float vdesc, uint32_t lds_wave, int i) {
    using C = Cfg<D, F8>;
    constexpr uint32_t PITCH = kEpiPitch<D>;
    constexpr int CHUNKS = D / 8;              // 16-byte pieces of a row
    constexpr int ROWS = 64 / CHUNKS;          // rows per store instruction
    const float l_tot = pair_sum((w.l4[0] + w.l4[1]) + (w.l4[2] + w.l4[3]));
    const float inv = l_tot > 0.0f ? vdesc / l_tot : 0.0f;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 val;
            val[0] = (__bf16)(w.o[cb][4 * j + 0] * inv);
            val[1] = (__bf16)(w.o[cb][4 * j + 1] * inv);
            val[2] = (__bf16)(w.o[cb][4 * j + 2] * inv);
            val[3] = (__bf16)(w.o[cb][4 * j + 3] * inv);
            *(__attribute__((address_space(3))) bf16x4*)(uintptr_t)(lds_wave + i * PITCH +
                                                                    2 * (32 * cb + 8 * j + 4 * hf)) = val;
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    const int lane = 32 * hf + i, qw0 = qrow - i, ch = lane % CHUNKS;
#pragma unroll
    for (int k = 0; k < 32 / ROWS; ++k) {
        const int r = k * ROWS + lane / CHUNKS;
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(lds_wave + r * PITCH + 16 * ch);
        if (qw0 + r < N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (int64_t)(qw0 + r) * osn + 8 * ch));
    }
    if (hf == 0 && qrow < N) lbase[qrow] = l_tot > 0.0f ? (w.m_run + log2f(l_tot)) * kLn2 : kNegInf;
}

// ----------------------------------------------------------------------------- dense, ping-pong
constexpr int kPPThreads = 512;   // 8 waves, two groups of four
constexpr int kPPRows = 256;      // query rows per workgroup
constexpr int kPPBufs = 3;

// (head, sequence) pair and query block of a dense workgroup. The hardware id is first
// remapped so that each XCD receives a contiguous share of the logical ids (xcd_remap).
// Logical ids run over groups of gh (head, sequence) pairs; within a group, block-major
// (all the group's pairs at one query block, then the next block), so that under causal
// masking the longest blocks of the whole group start first and an XCD's share does not
// end on one pair's long blocks. gh = 1 is plain head-major order.
template <bool CAUSAL>
__device__ __forceinline__ void dense_block(const Params& p, int hw, int grid, int& bh, int& qblk) {
    const int logical = xcd_remap(hw, grid);
    if (p.gh > 1) {
        const int span = p.gh * p.nqb, g = logical / span, r = logical % span;
        const int pairs = p.B * p.H, gsz = min(p.gh, pairs - g * p.gh);
        bh = g * p.gh + r % gsz;
        qblk = r / gsz;
    } else {
        bh = logical / p.nqb;
        qblk = logical % p.nqb;
    }
    if (CAUSAL) qblk = p.nqb - 1 - qblk;   // longest query blocks first
}

template <int D, bool CAUSAL, bool F8>
__global__ __launch_bounds__(kPPThreads, 1) void fwd_pingpong_kernel(Params p) {
    using C = Cfg<D, F8>;
    using E = typename ElemOf<F8>::type;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kPPBufs * C::BUF];
    static_assert(sizeof(smem) >= (kPPThreads / 64) * kEpiWaveB<D>, "the epilogue stages every wave's rows in LDS");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int role = wave >> 2;   // group 1 runs one phase behind group 0

    int bh, qblk;
    dense_block<CAUSAL>(p, blockIdx.x, gridDim.x, bh, qblk);
    const int hh = bh / p.B, b = bh % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qblk * kPPRows;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const E* kp = static_cast<const E*>(p.k) + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const E* vp = static_cast<const E*>(p.v) + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);

    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kPPRows - 1, N - 1);

    Rows<D, F8> w;
    load_q<D, F8>(w, static_cast<const E*>(p.q) + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn), p.qsn, qrow, N, hf);

    int T = (N + kBK - 1) / kBK;
    if (CAUSAL) T = min(T, qlast / kBK + 1);
    // Steps this wave takes part in: all of them, or under causal masking those whose first
    // key is not past the wave's last row.
    const int Tw = CAUSAL ? min(T, (qw0 + 31) / kBK + 1) : T;
    const bool rows_valid = qw0 < N;

    typename StageOf<D, kPPThreads, F8>::type st;
    st.init(tid, p.ksn, p.vsn);
    if (T > 0) {
        st.load(kp, vp, p.ksn, p.vsn, 0, N);
        st.store(smem);
    }
    // Settle every outstanding load (the Q fragments included) so that no wait on them is
    // left inside the loop; then start the loads of step 1.
    __builtin_amdgcn_s_waitcnt(0);
    const float c = signed_scale(w, p.c);   // after the wait: Q is in registers
    if (T > 1) st.load(kp, vp, p.ksn, p.vsn, kBK, N);
    __syncthreads();

    // Phase ph: group g works on local phase lp = ph - g. Even lp = 2t: P.V of step t-1 and
    // S of step t (MFMA); odd lp = 2t+1: softmax of step t (VALU). At the start of even
    // phase 2s the loaded step s+1 is stored into buffer (s+1) % 3, whose previous occupant,
    // step s-2, was last read in phase 2s-1 (group 1's P.V); step s+1 is first read in phase
    // 2s+2. Then the loads of step s+2 are issued.
    for (int ph = 0; ph < 2 * T + 2; ++ph) {
        if ((ph & 1) == 0) {
            const int s = ph >> 1;
            if (s + 1 < T) st.store(smem + ((s + 1) % kPPBufs) * C::BUF);
            if (s + 2 < T) st.load(kp, vp, p.ksn, p.vsn, (s + 2) * kBK, N);
        }
        const int lp = ph - role;
        if (lp >= 0 && rows_valid) {
            const int t = lp >> 1;
            if ((lp & 1) == 0) {
                // The matrix-product phase issues ahead of the other wave's softmax on its SIMD.
                __builtin_amdgcn_s_setprio(1);
                if (t >= 1 && t - 1 < Tw) pv<D, F8>(smem + ((t - 1) % kPPBufs) * C::BUF, w, i, hf);
                if (t < Tw) scores<D, F8>(smem + (t % kPPBufs) * C::BUF, w, i, hf);
                __builtin_amdgcn_s_setprio(0);
            } else if (t < Tw) {
                const int kt = t * kBK;
                const bool masked = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qw0);
                softmax<D, F8, CAUSAL>(w, masked, kt, qrow, N, c, hf);
            }
        }
        __syncthreads();
    }
    epilogue<D, F8>(w, p.o + seq_off(sp, b, hh, p.osb, p.osh, p.osn), p.osn,
                    p.lse + seq_stat_off(sp, b, hh, p.H, p.N, p.total), qrow, N, hf, p.vdesc,
                    lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kEpiWaveB<D>, i);
}

// ----------------------------------------------------------------------------- dense, ping-pong,
// tiles loaded straight into LDS (bf16, head dimension 128)
//
// Same phases as fwd_pingpong_kernel, but the K and V tiles travel from memory to LDS with
// buffer loads that write LDS directly (no staging registers, no LDS store instructions).
// One such load writes 16 bytes per lane at consecutive addresses, i.e. four whole 256-byte
// rows per wave instruction, so the tiles are kept unpadded and conflicts are avoided by
// placing 16-byte chunk c of row r at chunk slot c ^ swz(r) instead:
// * K (16-byte row reads, 16 rows per pass): swz(r) = r & 15;
// * V (transposing reads, four rows x four chunks per 32 lanes): swz(r) = 4 * (r & 3).
// Each lane loads the chunk that belongs at its slot, so the rows are still read whole.
// Four LDS stages; the loads of step m + 2 are issued at the start of phase 2m (into the
// stage of step m - 2, last read in phase 2m - 1) and have four phases to arrive.
// The loads are issued from inline assembly: the compiler then does not treat them as
// pending LDS stores, which would make every barrier wait for all of them; the waits are
// placed by hand (an odd phase ends with vmcnt(4): only the latest step may be in flight).
constexpr int kDmaBufs = 4;
constexpr int kDmaRowB = kLdsRowB;
constexpr int kDmaTileB = kLdsTileB;
constexpr int kDmaStageB = 2 * kDmaTileB;        // K then V

// Per-lane LDS byte addresses of the swizzled reads in stage 0 (the LDS base of the stages
// included, so that a read's address is one add of the stage offset).
struct DmaAddr {
    uint32_t k[8];   // K: row i, logical chunk 2 * ks + hf (the second 32-key block is +8 KB)
    uint32_t v[4];   // V (transposing reads): per 32-column block cb

    __device__ void init(int i, int hf, uint32_t base) {
        // Hide the base's value (0 for the kernels' single LDS array) from the compiler:
        // known-disjoint address bits make it combine the stage and block offsets with ORs
        // instead of one add plus the read's immediate offset.
        asm("" : "+s"(base));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            k[ks] = base + (uint32_t)(i * kDmaRowB + 16 * ((2 * ks + hf) ^ swz<kSwzRow>(i)));
        const int g16 = (i >> 4) & 1, j16 = i & 15;
        const int row = 4 * hf + (j16 >> 2);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int chunk = 4 * cb + 2 * g16 + ((j16 & 3) >> 1);
            v[cb] = base + (uint32_t)(kDmaTileB + row * kDmaRowB + 16 * (chunk ^ swz<kSwzTr>(row)) + 8 * (j16 & 1));
        }
    }
};

// S^T = K Q^T for one 64-key step from the swizzled stage at byte offset `so` (same products
// as scores()).
__device__ __forceinline__ void scores_sw(uint32_t so, Rows<128, false>& w, const DmaAddr& a) {
    w.s[0] = f32x16{};
    w.s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        uint32_t x = a.k[ks] + so;
        asm("" : "+v"(x));   // one add per column; the block offset goes to the read's immediate
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) w.s[kb] = mfma32(lds16(x + 32 * kDmaRowB * kb), w.qf.v[ks], w.s[kb]);
    }
    constexpr int N = 16, AHEAD = 6;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int k = 0; k < N - AHEAD; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// O^T += V^T P^T from the swizzled stage at byte offset `so` (same products and operand
// layout as pv()).
__device__ __forceinline__ void pv_sw(uint32_t so, Rows<128, false>& w, const DmaAddr& a) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        bf16x8 op[2][2];
        uint32_t xv = a.v[cb] + so;
        asm("" : "+v"(xv));   // one add per column block; row offsets go to the immediates
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint32_t p0 = xv + (32 * kb + 16 * s2) * kDmaRowB;
                const u32x2 lo = lds_tr4(p0);
                const u32x2 hi = lds_tr4(p0 + 8 * kDmaRowB);
                u32x4 x;
                x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
                op[kb][s2] = as_bf16x8(x);
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) w.o[cb] = mfma32(op[kb][s2], w.pb[kb][s2], w.o[cb]);
    }
    constexpr int READS = 32, MF = 16, AHEAD = 10, PAIRS = (READS - AHEAD) / 2;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int k = 0; k < PAIRS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF - PAIRS, 0);
}

// Q of a workgroup's ROWS rows (from q0; rows past N read as zeros) straight into LDS at
// `q_lds`, as ROWS / 64 blocks of 64 rows in the K layout (kSwzRow), with the whole-row loads
// of the K/V tiles: each of the NW waves fetches the same 1-KB pieces of every block as for a
// K tile. `q_lds` and `wave_u` must be wave-uniform (the loads take M0).
template <int NW, int ROWS>
__device__ __forceinline__ void load_q_to_lds(const uint16_t* qp, int64_t qsn, int q0, int N, uint32_t q_lds,
                                              int wave, int wave_u, int lane) {
    constexpr int P = 16 / NW;
    uint32_t qoff[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const int row = 4 * (P * wave + j) + (lane >> 4), slot = lane & 15;
        qoff[j] = (uint32_t)((int64_t)row * qsn * 2 + 16 * (slot ^ swz<kSwzRow>(row)));
    }
#pragma unroll
    for (int blk = 0; blk < ROWS / 64; ++blk) {
        const int r0 = q0 + 64 * blk;
        const i32x4 rq = rsrc_words(qp + (int64_t)r0 * qsn, rows_bytes(r0, N, qsn, 128, 64));
#pragma unroll
        for (int j = 0; j < P; ++j)
            load16_to_lds(rq, qoff[j], q_lds + blk * kLdsTileB + 1024u * (P * (uint32_t)wave_u + j));
    }
}

// The wave's Q fragments (rows 32 wave + i of the workgroup's rows: row 32 (wave & 1) + i of
// block wave / 2) from the layout load_q_to_lds writes; the loads must have arrived.
__device__ __forceinline__ void read_q_frags(Rows<128, false>& w, uint32_t q_lds, int wave, int i, int hf) {
    const int r = 32 * (wave & 1) + i;
    const uint32_t rb = q_lds + (uint32_t)(wave >> 1) * kLdsTileB + (uint32_t)r * 256u;
#pragma unroll
    for (int ks = 0; ks < 128 / 16; ++ks) w.qf.v[ks] = lds16(rb + 16u * (uint32_t)((2 * ks + hf) ^ swz<kSwzRow>(r)));
}

template <bool CAUSAL>
__global__ __launch_bounds__(kPPThreads, 1) void fwd_pingpong_dma_kernel(Params p) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kDmaBufs * kDmaStageB];
    static_assert(sizeof(smem) >= (kPPThreads / 64) * kEpiWaveB<D>, "the epilogue stages every wave's rows in LDS");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int role = wave >> 2;   // group 1 runs one phase behind group 0

    int bh, qblk;
    dense_block<CAUSAL>(p, blockIdx.x, gridDim.x, bh, qblk);
    const int hh = bh / p.B, b = bh % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qblk * kPPRows;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const uint16_t* kp = static_cast<const uint16_t*>(p.k) + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const uint16_t* vp = static_cast<const uint16_t*>(p.v) + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);

    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kPPRows - 1, N - 1);

    Rows<D, false> w;
    init_rows(w);

    int T = (N + kBK - 1) / kBK;
    if (CAUSAL) T = min(T, qlast / kBK + 1);
    const int Tw = CAUSAL ? min(T, (qw0 + 31) / kBK + 1) : T;
    const bool rows_valid = qw0 < N;

    DmaStage<kPPThreads / 64, kSwzRow, kSwzTr> st;
    st.init(wave, lane, p.ksn, p.vsn);
    DmaAddr ad;
    ad.init(i, hf, lds_address(smem));
    // the wave index and the LDS base are uniform: keep them in scalar registers (the loads
    // take their LDS address from M0)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_address(smem);
    // Q: the workgroup's 256 rows go straight into stages 2 and 3 (free until phase 0 loads
    // step 2), read into the fragments below.
    const uint32_t q_lds = lds0 + 2 * kDmaStageB;
    load_q_to_lds<kPPThreads / 64, kPPRows>(static_cast<const uint16_t*>(p.q) + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn),
                                            p.qsn, q0, N, q_lds, wave, wave_u, lane);
    static_assert(kDmaBufs == 4 && 2 * kDmaStageB == (kPPRows / 64) * kLdsTileB, "Q fills stages 2 and 3");
    if (T > 0) st.issue(kp, vp, p.ksn, p.vsn, 0, N, lds0, wave_u);
    if (T > 1) st.issue(kp, vp, p.ksn, p.vsn, kBK, N, lds0 + kDmaStageB, wave_u);
    // Settle every outstanding load (Q and the first two steps) before reading Q.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read_q_frags(w, q_lds, wave, i, hf);
    const float c = signed_scale(w, p.c);   // Q is in registers
    __syncthreads();   // every wave has its Q: phase 0 may load step 2 over it

    // Phase ph: group g works on local phase lp = ph - g. Even lp = 2t: P.V of step t-1 and
    // S of step t (MFMA); odd lp = 2t+1: softmax of step t (VALU).
    for (int ph = 0; ph < 2 * T + 2; ++ph) {
        if ((ph & 1) == 0) {
            const int s2 = (ph >> 1) + 2;
            if (s2 < T) st.issue(kp, vp, p.ksn, p.vsn, s2 * kBK, N, lds0 + (s2 % kDmaBufs) * kDmaStageB, wave_u);
        }
        const int lp = ph - role;
        if (lp >= 0 && rows_valid) {
            const int t = lp >> 1;
            if ((lp & 1) == 0) {
                __builtin_amdgcn_s_setprio(1);
                if (t >= 1 && t - 1 < Tw) pv_sw(((t - 1) % kDmaBufs) * kDmaStageB, w, ad);
                if (t < Tw) scores_sw((t % kDmaBufs) * kDmaStageB, w, ad);
                __builtin_amdgcn_s_setprio(0);
            } else if (t < Tw) {
                const int kt = t * kBK;
                const bool masked = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qw0);
                softmax<D, false, CAUSAL>(w, masked, kt, qrow, N, c, hf);
            }
        }
        // After odd phase 2m+1 the next phase reads step m+1: wait until only the loads of
        // step m+2 (issued at the start of phase 2m, if there is such a step) may still be in
        // flight, i.e. vmcnt(4), or until none are when step m+2 was not loaded.
        if (ph & 1) {
            if ((ph >> 1) + 2 < T) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
            else __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
        }
        __syncthreads();
    }
    epilogue<D, false>(w, p.o + seq_off(sp, b, hh, p.osb, p.osh, p.osn), p.osn,
                       p.lse + seq_stat_off(sp, b, hh, p.H, p.N, p.total), qrow, N, hf, p.vdesc,
                    lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kEpiWaveB<D>, i);
}

// ----------------------------------------------------------------------------- sparse
constexpr int kSpThreads = 256;   // 4 waves, one 128-row block

// Visit log of the block-sparse kernels (only when p.visits is set): the workgroup of
// (sequence b, head hh) marks step tt, i.e. half (tt & 1) of list entry (tt >> 1), as taken
// into its softmax. One lane writes one byte per step, so the log costs a store per step.
__device__ __forceinline__ void log_visit(const Params& p, int b, int hh, int tt, int tid) {
    if (p.visits != nullptr && tid == 0) p.visits[((int64_t)b * p.H + hh) * (2 * p.nnz) + tt] = 1;
}

template <int D, bool CAUSAL, bool F8>
__global__ __launch_bounds__(kSpThreads, 2) void fwd_sparse_kernel(Params p) {
    using C = Cfg<D, F8>;
    using E = typename ElemOf<F8>::type;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];
    static_assert(sizeof(smem) >= (kSpThreads / 64) * kEpiWaveB<D>, "the epilogue stages every wave's rows in LDS");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;

    // Plain order, longest lists first. Consecutive ids go to the 8 XCDs in turn, so all of
    // them work on the same head at once: a strided list reaches back over the whole head,
    // and the head's K/V then stays in the cache the XCDs share (giving each XCD its own
    // heads, as the dense kernel does, overflows it).
    const int bh = blockIdx.x / p.nqb;
    const int qblk = p.nqb - 1 - blockIdx.x % p.nqb;
    const int hh = bh / p.B, b = bh % p.B;   // head-major: the sequences of a head are adjacent
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qblk * kSparseBlock;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const E* kp = static_cast<const E*>(p.k) + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const E* vp = static_cast<const E*>(p.v) + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);

    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kSparseBlock - 1, N - 1);

    Rows<D, F8> w;
    load_q<D, F8>(w, static_cast<const E*>(p.q) + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn), p.qsn, qrow, N, hf);

    // Step t covers half (t & 1) of the listed key block kv_indices[t >> 1]. Offsets are
    // clamped to [0, nnz]; out-of-range and (causal) above-diagonal entries are skipped.
    const int nkb = (N + kSparseBlock - 1) / kSparseBlock;
    int64_t lo = load_uniform(p.kv_offsets, qblk), hi = load_uniform(p.kv_offsets, qblk + 1);
    lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
    hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
    int t = (int)(2 * lo);
    const int t_end = (int)(2 * hi);
    auto step_key = [&](int tt) -> int {   // first key of step tt, or -1 to skip it
        const int kblk = load_uniform(p.kv_indices, tt >> 1);
        if (kblk < 0 || kblk >= nkb || (CAUSAL && kblk > qblk)) return -1;
        const int kt0 = kblk * kSparseBlock + (tt & 1) * kBK;
        if (kt0 >= N || (CAUSAL && kt0 > qlast)) return -1;
        return kt0;
    };
    int kt = -1;
    while (t < t_end && (kt = step_key(t)) < 0) ++t;


    typename StageOf<D, kSpThreads, F8>::type st;
    st.init(tid, p.ksn, p.vsn);
    if (t < t_end) {
        st.load(kp, vp, p.ksn, p.vsn, kt, N);
        st.store(smem);
    }
    // Settle every outstanding load (the Q fragments included) before the loop, so that no
    // wait on them is left inside it.
    __builtin_amdgcn_s_waitcnt(0);
    const float c = signed_scale(w, p.c);   // after the wait: Q is in registers
    __syncthreads();

    int cur = 0;
    while (t < t_end) {
        log_visit(p, b, hh, t, tid);
        int tn = t + 1, ktn = -1;
        while (tn < t_end && (ktn = step_key(tn)) < 0) ++tn;
        const bool has_next = tn < t_end;
        if (has_next) st.load(kp, vp, p.ksn, p.vsn, ktn, N);

        const uint16_t* buf = smem + cur * C::BUF;
        if (qw0 < N && (!CAUSAL || kt <= qw0 + 31)) {
            const bool masked = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qw0);
            // matrix products at raised priority: they issue ahead of the other workgroup's
            // softmax on the same SIMD
            __builtin_amdgcn_s_setprio(1);
            scores<D, F8>(buf, w, i, hf);
            __builtin_amdgcn_s_setprio(0);
            softmax<D, F8, CAUSAL>(w, masked, kt, qrow, N, c, hf);
            __builtin_amdgcn_s_setprio(1);
            pv<D, F8>(buf, w, i, hf);
            __builtin_amdgcn_s_setprio(0);
        }
        if (has_next) st.store(smem + (cur ^ 1) * C::BUF);
        __syncthreads();
        cur ^= 1;
        t = tn;
        kt = ktn;
    }
    epilogue<D, F8>(w, p.o + seq_off(sp, b, hh, p.osb, p.osh, p.osn), p.osn,
                    p.lse + seq_stat_off(sp, b, hh, p.H, p.N, p.total), qrow, N, hf, p.vdesc,
                    lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kEpiWaveB<D>, i);
}

// Block-sparse forward, bf16 at head dimension 128, with the K/V tiles loaded straight into
// LDS in the swizzled layout of fwd_pingpong_dma_kernel: two 32 KB stages per workgroup (two
// workgroups per CU); the loads of the next listed step are issued at the start of a step
// into the other stage and waited for (vmcnt(0)) before the step's closing barrier.
template <bool CAUSAL>
__global__ __launch_bounds__(kSpThreads, 2) void fwd_sparse_dma_kernel(Params p) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kDmaStageB];
    static_assert(sizeof(smem) >= (kSpThreads / 64) * kEpiWaveB<D>, "the epilogue stages every wave's rows in LDS");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;

    // Plain order, longest lists first (as fwd_sparse_kernel).
    const int bh = blockIdx.x / p.nqb;
    const int qblk = p.nqb - 1 - blockIdx.x % p.nqb;
    const int hh = bh / p.B, b = bh % p.B;
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qblk * kSparseBlock;
    if (q0 >= N) return;

    const int hk = hh / p.G;
    const uint16_t* kp = static_cast<const uint16_t*>(p.k) + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const uint16_t* vp = static_cast<const uint16_t*>(p.v) + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);

    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kSparseBlock - 1, N - 1);

    Rows<D, false> w;
    init_rows(w);

    const int nkb = (N + kSparseBlock - 1) / kSparseBlock;
    int64_t lo = load_uniform(p.kv_offsets, qblk), hi = load_uniform(p.kv_offsets, qblk + 1);
    lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
    hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
    int t = (int)(2 * lo);
    const int t_end = (int)(2 * hi);
    auto step_key = [&](int tt) -> int {   // first key of step tt, or -1 to skip it
        const int kblk = load_uniform(p.kv_indices, tt >> 1);
        if (kblk < 0 || kblk >= nkb || (CAUSAL && kblk > qblk)) return -1;
        const int kt0 = kblk * kSparseBlock + (tt & 1) * kBK;
        if (kt0 >= N || (CAUSAL && kt0 > qlast)) return -1;
        return kt0;
    };
    int kt = -1;
    while (t < t_end && (kt = step_key(t)) < 0) ++t;


    DmaStage<kSpThreads / 64, kSwzRow, kSwzTr> st;
    st.init(wave, lane, p.ksn, p.vsn);
    DmaAddr ad;
    ad.init(i, hf, lds_address(smem));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_address(smem);
    // Q: the block's 128 rows go straight into stage 1 (free until the first step loads the
    // next one), read into the fragments below.
    static_assert(kDmaStageB == (kSparseBlock / 64) * kLdsTileB, "Q fills one stage");
    const uint32_t q_lds = lds0 + kDmaStageB;
    load_q_to_lds<kSpThreads / 64, kSparseBlock>(static_cast<const uint16_t*>(p.q) + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn),
                                                 p.qsn, q0, N, q_lds, wave, wave_u, lane);
    if (t < t_end) st.issue(kp, vp, p.ksn, p.vsn, kt, N, lds0, wave_u);
    // Settle every outstanding load (Q and the first step) before reading Q.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read_q_frags(w, q_lds, wave, i, hf);
    const float c = signed_scale(w, p.c);   // Q is in registers
    __syncthreads();   // every wave has its Q: the first step may load the next one over it

    int cur = 0;
    while (t < t_end) {
        log_visit(p, b, hh, t, tid);
        int tn = t + 1, ktn = -1;
        while (tn < t_end && (ktn = step_key(tn)) < 0) ++tn;
        const bool has_next = tn < t_end;
        // the other stage was last read in the previous step, which ended with a barrier
        if (has_next) st.issue(kp, vp, p.ksn, p.vsn, ktn, N, lds0 + (cur ^ 1) * kDmaStageB, wave_u);

        const uint32_t buf = cur * kDmaStageB;
        if (qw0 < N && (!CAUSAL || kt <= qw0 + 31)) {
            const bool masked = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qw0);
            __builtin_amdgcn_s_setprio(1);
            scores_sw(buf, w, ad);
            __builtin_amdgcn_s_setprio(0);
            softmax<D, false, CAUSAL>(w, masked, kt, qrow, N, c, hf);
            __builtin_amdgcn_s_setprio(1);
            pv_sw(buf, w, ad);
            __builtin_amdgcn_s_setprio(0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of the next step
        __syncthreads();
        cur ^= 1;
        t = tn;
        kt = ktn;
    }
    epilogue<D, false>(w, p.o + seq_off(sp, b, hh, p.osb, p.osh, p.osn), p.osn,
                       p.lse + seq_stat_off(sp, b, hh, p.H, p.N, p.total), qrow, N, hf, p.vdesc,
                    lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kEpiWaveB<D>, i);
}

template <int D, bool CAUSAL, bool F8>
hipError_t dispatch(Params p, bool sparse, hipStream_t stream) {
    if (sparse) {
        p.nqb = (p.N + kSparseBlock - 1) / kSparseBlock;
        const int64_t grid = (int64_t)p.B * p.H * p.nqb;
        if constexpr (D == 128 && !F8)
            hipLaunchKernelGGL((fwd_sparse_dma_kernel<CAUSAL>), dim3((unsigned)grid), dim3(kSpThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_sparse_kernel<D, CAUSAL, F8>), dim3((unsigned)grid), dim3(kSpThreads), 0, stream,
                               p);
        return hipGetLastError();
    }
    p.nqb = (p.N + kPPRows - 1) / kPPRows;
    const int64_t grid = (int64_t)p.B * p.H * p.nqb;
    // Short causal sequences (at most 16 query blocks per head): block-major order over
    // groups of (head, sequence) pairs, so that an XCD's share does not end on the longest
    // blocks of its last pairs. A group holds at most the pairs of one XCD's share (B*H/8)
    // and at most eight (B=4 H=32 N=4096: groups of 4 +5 %, of 8 +9 %, of 16 +7 % over
    // plain order). Longer sequences keep plain head-major order: their shares already
    // balance, and groups lose L2 reuse of the K/V stream (N=32768: -4 % with groups of
    // four, -40 % with groups wider than a share); packed batches lost 15-30 % with any group.
    p.gh = 1;
    if (CAUSAL && p.cu == nullptr && p.nqb <= 16) p.gh = max(1, min(8, p.B * p.H / 8));
    if constexpr (D == 128 && !F8)
        hipLaunchKernelGGL((fwd_pingpong_dma_kernel<CAUSAL>), dim3((unsigned)grid), dim3(kPPThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_pingpong_kernel<D, CAUSAL, F8>), dim3((unsigned)grid), dim3(kPPThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(Params p, bool causal, bool sparse, bool f8, hipStream_t stream) {
    if (f8) return causal ? dispatch<D, true, true>(p, sparse, stream) : dispatch<D, false, true>(p, sparse, stream);
    return causal ? dispatch<D, true, false>(p, sparse, stream) : dispatch<D, false, false>(p, sparse, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    Params p;
    p.q = a.q.p;
    p.k = a.k.p;
    p.v = a.v.p;
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.qsb = a.q.sb; p.qsh = a.q.sh; p.qsn = a.q.sn;
    p.ksb = a.k.sb; p.ksh = a.k.sh; p.ksn = a.k.sn;
    p.vsb = a.v.sb; p.vsh = a.v.sh; p.vsn = a.v.sn;
    p.osb = a.osb; p.osh = a.osh; p.osn = a.osn;
    p.B = a.L.B; p.H = a.L.H; p.N = a.L.N;
    p.G = a.L.H / a.L.Hkv;
    p.cu = a.L.cu;
    p.total = a.L.total;
    p.nqb = 0;
    p.gh = 1;
    p.c = a.scale * a.qk_desc * kLog2e;
    p.vdesc = a.v_desc;
    p.kv_offsets = a.kv_offsets;
    p.kv_indices = a.kv_indices;
    p.nnz = a.nnz;
    p.visits = a.visits;
    const bool sparse = a.kv_offsets != nullptr;
    if (a.L.d == 64) return dispatch_d<64>(p, a.causal != 0, sparse, a.f8 != 0, stream);
    return dispatch_d<128>(p, a.causal != 0, sparse, a.f8 != 0, stream);
}

}  // namespace fa
