// Attention backward for gfx950 by recomputation from the stored log-sum-exp.
//
// Method ("Flash MSA Attention Kernel Implementation: A Practical Guide for Production
// AI", section "The Backward Pass: The Real Beast"): the forward keeps O and the row
// statistics instead of the score matrix; the backward recomputes S and
// P = exp(S - LSE) tile by tile and forms dP = dO V^T, dS = P o (dP - D) with
// D_i = sum_j P_ij dP_ij, dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K (the scale
// factors follow from S = scale Q K^T; the page's sketch omits them).
//
// MI355X decomposition (this file's design, not the page's; the page's sketch runs one
// Q tile per block and would need a cross-block reduction for dK and dV):
// 1. pre_kernel: D_i = dO_i . O_i, which equals sum_j P_ij dP_ij because O_i = sum_j P_ij V_j.
//    Bandwidth-bound: it reads O and dO once.
// 2. dkdv16_kernel: a workgroup owns 128 keys (16 per wave, one key per lane column of
//    16x16 products, 8 waves) and walks the query tiles that can see them. K and V of the
//    wave's keys stay in registers as MFMA B operands; S = Q K^T and dP = dO V^T read Q and
//    dO rows from LDS; dV^T += dO^T P and dK^T += Q^T dS read the transposed operands
//    straight from the row-major tiles with ds_read_b64_tr_b16. dK^T, dV^T accumulate in fp32.
// 3. dq_dma_kernel (head dimension 128; dq_kernel at 64): a workgroup owns 128 query rows,
//    as in the forward, and walks the key tiles: S^T = K Q^T and dP^T = V dO^T with Q and dO
//    in registers, then dQ^T += K^T dS^T with K^T read transposed from the row-major K tile.
//    S and dP are thus computed twice (7 matrix products instead of 5) in exchange for no
//    atomics and bitwise-reproducible results.
// 3'. With a workspace large enough to hold every dS tile (head dimension 128), the dK/dV
//    kernel (dkdv_pair_kernel, the head-dimension-128 replacement of dkdv16_kernel) also
//    writes the bf16 dS it forms for the dK product, and dq_ds_kernel computes
//    dQ^T += K^T dS^T from it: 5 products in all, still without atomics.
//
// LDS layouts, all free of bank conflicts for the reads they serve: the dK/dV kernel stages
// its Q and dO tiles through registers into one copy with 288-byte rows, which serves both
// its row reads and its transposing reads; dq_dma_kernel loads K and V straight into LDS as
// unpadded rows with XOR-swizzled 16-byte chunks (one K copy for both read patterns), and
// dq_ds_kernel K and the gathered dS rows the same way;
// dq_kernel keeps a 272-byte row copy and a 320-byte transposed-read copy of K. Tiles are
// fetched with raw buffer loads that zero-fill rows past N.
#include <mutex>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = 64;   // rows per staged tile

template <int D>
struct BCfg {
    static constexpr int RS = D + 8;            // row-read copy stride (elements)
    static constexpr int TS = D + 32;           // transposed-read copy stride (elements)
    static constexpr int RE = kStep * RS;
    static constexpr int TE = kStep * TS;
    static constexpr int CR = D / 8;            // 16-byte chunks per row
    static constexpr int CH = kStep * CR / kThreads;
    static constexpr int KSTEPS = D / 16;
    static constexpr int CB = D / 32;
};

// One 64-row tile of a [N, D] matrix (row stride sn elements) in registers: per thread CH
// 16-byte chunks (NT threads), loaded with a bounds-checked buffer load, stored to one or
// two LDS copies.
template <int D, int NT = kThreads, int RSTR = BCfg<D>::RS, int TSTR = BCfg<D>::TS, int SETS = 1>
struct Tile {
    using C = BCfg<D>;
    static constexpr int CH = kStep * C::CR / NT;
    u32x4 r[SETS][CH];   // SETS register sets: loads for different steps in flight at once
    uint32_t goff[CH];
    int roff[CH], toff[CH];

    __device__ void init(int tid, int64_t sn) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int id = tid + j * NT;
            const int row = id / C::CR, ch = id % C::CR;
            goff[j] = (uint32_t)(((int64_t)row * sn + 8 * ch) * 2);
            roff[j] = row * RSTR + 8 * ch;
            toff[j] = row * TSTR + 8 * ch;
        }
    }
    template <int S = 0>
    __device__ void load(const uint16_t* base, int64_t sn, int r0, int N) {
        const auto rs = make_rsrc(base + (int64_t)r0 * sn, rows_bytes(r0, N, sn, D, kStep));
#pragma unroll
        for (int j = 0; j < CH; ++j) r[S][j] = buf_load16(rs, goff[j], 0);
    }
    template <int S = 0>
    __device__ void store(uint16_t* rowcopy, uint16_t* trcopy) const {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (rowcopy) *reinterpret_cast<u32x4*>(rowcopy + roff[j]) = r[S][j];
            if (trcopy) *reinterpret_cast<u32x4*>(trcopy + toff[j]) = r[S][j];
        }
    }
};

// ----------------------------------------------------------------------------- -D = -rowsum(dO * O)
// Writes -D (negated: it then starts the dP accumulators of the dK/dV pass, which yields dP - D
// with no subtraction) and each row's LSE in the exp2 domain, lse2 = LSE log2(e), with -inf (a
// row with no allowed key) as +inf so that its probabilities exp2(s - lse2) are exactly 0.
template <int D>
__global__ __launch_bounds__(kThreads) void pre_kernel(const uint16_t* o, int64_t osb, int64_t osh, int64_t osn,
                                                       const uint16_t* dout, int64_t dsb, int64_t dsh, int64_t dsn,
                                                       const float* lse, float* delta, float* lse2, int H, int N,
                                                       int64_t rows) {
    constexpr int LPR = D / 8;                       // lanes per row, 8 elements each
    constexpr int RPB = kThreads / LPR;              // rows per block
    const int tid = threadIdx.x;
    const int part = tid % LPR;
    // Grid-stride over blocks of RPB rows: the launch caps the grid, so any row count stays
    // within one launch. The loop bound depends only on the block index (uniform per block).
    for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < rows; r0 += (int64_t)gridDim.x * RPB) {
        const int64_t row = r0 + tid / LPR;
        float acc = 0.0f;
        if (row < rows) {
            const int64_t bh = row / N;
            const int n = (int)(row % N);
            const int b = (int)(bh / H), h = (int)(bh % H);
            const u32x4 x = *reinterpret_cast<const u32x4*>(o + b * osb + h * osh + (int64_t)n * osn + 8 * part);
            const u32x4 y = *reinterpret_cast<const u32x4*>(dout + b * dsb + h * dsh + (int64_t)n * dsn + 8 * part);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc += __uint_as_float(x[w] << 16) * __uint_as_float(y[w] << 16);
                acc += __uint_as_float(x[w] & 0xffff0000u) * __uint_as_float(y[w] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
        if (row < rows && part == 0) {
            delta[row] = -acc;   // stored negated: -D starts the dP accumulators of the dK/dV pass
            const float l = lse[row];
            lse2[row] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
        }
    }
}

// ----------------------------------------------------------------------------- dK, dV
constexpr int kKV_BK = 128;   // keys per workgroup (32 per wave)

struct KVParams {
    const uint16_t *q, *k, *v, *dout;
    const float* lse;
    const float* delta;
    const float* lse2;     // LSE * log2(e), -inf as +inf (written by pre_kernel), laid out like delta
    uint16_t *dk, *dv;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, dsb, dsh, dsn;
    int64_t dksb, dksh, dksn, dvsb, dvsh, dvsn;
    int B, H, Hkv, N, nkb;
    int G;                 // query heads per K/V head
    const int32_t* cu;     // packed sequence offsets [B + 1], or nullptr
    int64_t total;
    const int32_t* q_offsets;   // key-side block lists (block-sparse mode), or nullptr
    const int32_t* q_indices;
    int64_t nnz;
    float c;       // scale * log2(e)
    float scale;
    // Stored dS (dkdv_pair_kernel only; nullptr: not stored). Region of sequence b, query head
    // h: ds + (b * H + h) * ds_bh, a run of [128 keys, 128 query positions] bf16 tiles, one per
    // (key block, query block) pair the pass visits (numbering in dq_ds_kernel).
    uint16_t* ds;
    int64_t ds_bh;
    int nqbt;      // query blocks of the tile numbering: ceil(N / 128)
};

template <int D>
struct KVCfg {
    using C = BCfg<D>;
    // One copy of each staged tile serves both of its read patterns, the 16-byte row reads of
    // the 16x16 layout (4 lane groups x the same 16 rows) and the transposing reads (16 rows x
    // 32 bytes, two 16-lane groups served together): both are free of bank conflicts at a
    // 288-byte row stride (measured; 272 and 320 bytes each leave one of them 2-way).
    static constexpr int TS = D + 16;
    static constexpr int TE = kStep * TS;
    // stage layout: Q | dO | lse2[64] | delta[64]
    static constexpr int QR = 0, DR = TE;
    static constexpr int STATS = 2 * TE;
    static constexpr int STAGE = STATS + 2 * kStep * 2;   // in uint16 units
    static_assert((STATS * 2) % 16 == 0 && (STAGE * 2) % 16 == 0, "16-byte alignment");
};

// dK, dV: a workgroup owns 128 keys, 16 per wave (v_mfma_f32_16x16x32_bf16), 8 waves. With
// 32 keys per wave the dK, dV accumulators and the K, V operands alone take ~200 registers
// and only one wave fits a SIMD; at 16 keys a wave needs ~220 in all (two staging sets
// included), two waves share each SIMD and hide each other's latencies (at twice the LDS
// reads per product).
// Operand layout of the 16x16x32 product: lane l supplies row (A) / column (B) l % 16 and the
// 8 k-values 8*(l/16) .. 8*(l/16)+7; accumulator element r of lane l is row 4*(l/16) + r,
// column l % 16.
constexpr int kThreads16 = 512;

typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4v mfma16(bf16x8 a, bf16x8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The query steps a key block's dK/dV pass walks: 64-row query tiles, for each of the G
// query heads that read the block's K/V head in turn. Dense: the tiles from the first one
// that can see these keys (causal) or from 0 to the end. Block-sparse: both halves of every
// query block the key-side list names for this key block. Under causal masking only the
// steps of the diagonal block hold keys after queries: the first two of each query head
// (dense), or the two halves of the list's diagonal entry (block-sparse: the first entry not
// below the key block, the lists being ascending; entries before it are above-diagonal
// entries of the query-side lists, which are skipped). Those steps are numbered first, so
// the others need no element test. Out-of-range list entries (or, causal, entries above the
// diagonal) become an empty tile at row N, whose loads are zero-filled.
template <bool CAUSAL>
struct KvSteps {
    int n_all;     // steps of all query heads
    int n_mask;    // the first n_mask steps need the causal element mask
    int m_per, u_per, diag, t0, nqb, kblk, hk, G, N;
    int64_t lo;
    bool sparse;
    const int32_t* qi;

    __device__ void init(const KVParams& p, int kblk_, int hk_, int N_, int k0) {
        kblk = kblk_;
        hk = hk_;
        G = p.G;
        N = N_;
        qi = p.q_indices;
        const int nsteps = (N + kStep - 1) / kStep;
        t0 = CAUSAL ? k0 / kStep : 0;
        lo = 0;
        int64_t hi = 0;
        sparse = p.q_offsets != nullptr;
        if (sparse) {
            lo = load_uniform(p.q_offsets, kblk);
            hi = load_uniform(p.q_offsets, kblk + 1);
            lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
            hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
        }
        const int per = sparse ? (int)(2 * (hi - lo)) : nsteps - t0;
        n_all = per * G;
        nqb = (N + kKV_BK - 1) / kKV_BK;
        m_per = 0;   // masked steps per query head: 0, 2, or 1 when a head has a single step
        diag = 0;    // block-sparse: list position (from lo) of the diagonal entry
        if constexpr (CAUSAL) {
            if (sparse) {
                int64_t e = lo;
                while (e < hi && load_uniform(qi, e) < kblk) ++e;
                if (e < hi && load_uniform(qi, e) == kblk) {
                    m_per = 2;
                    diag = (int)(e - lo);
                }
            } else {
                m_per = min(2, per);
            }
        }
        n_mask = m_per * G;
        u_per = per - m_per;
    }

    // First row of step s (N past the last step or for a skipped entry); hq: its query head.
    __device__ int row(int s, int& hq) const {
        if (s >= n_all) {
            hq = hk * G;
            return N;
        }
        int gq = 0, j = 0;   // query head in the group; step within that head's sequence
        bool masked_step = false;
        if constexpr (CAUSAL) {
            if (s < n_mask) {
                gq = s / m_per;
                j = s - gq * m_per;
                masked_step = true;
            }
        }
        if (!masked_step) {
            const int u = s - n_mask;
            gq = u / u_per;
            j = u - gq * u_per;   // among the unmasked steps
        }
        hq = hk * G + gq;
        if (!sparse) return (t0 + (masked_step ? j : m_per + j)) * kStep;
        int e = j >> 1;   // list entry (from lo): the diagonal one, or the others in order
        if (masked_step) e = diag;
        else if (m_per && e >= diag) ++e;
        const int qb = load_uniform(qi, lo + e);
        if (qb < 0 || qb >= nqb || (CAUSAL && qb < kblk)) return N;
        const int r0 = qb * kKV_BK + (j & 1) * kStep;
        return r0 < N ? r0 : N;
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads16, 1) void dkdv16_kernel(KVParams p) {
    using L = KVCfg<D>;
    constexpr int KS32 = D / 32;   // 32-wide k-steps over the head dimension
    constexpr int CB16 = D / 16;   // 16-row blocks of dK^T, dV^T
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = (lane >> 4) & 3, i = lane & 15;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // Block-sparse: plain order, so that all XCDs work on the same head at once and its
    // Q/dO stay in the cache they share (key-side lists reach across the whole head).
    const int logical = p.q_offsets ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    const int bhk = logical / p.nkb, kblk = logical % p.nkb;   // ascending: longest first under causal
    const int hk = bhk / p.B, b = bhk % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int k0 = kblk * kKV_BK;
    if (k0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int kw0 = k0 + 16 * wave;
    const int key = kw0 + i;

    // K and V rows of this lane's key as B operands (column = key, k-group = g).
    bf16x8 kf[KS32], vf[KS32];
    {
        const uint16_t* kr = p.k + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn) + (int64_t)key * p.ksn + 8 * g;
        const uint16_t* vr = p.v + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn) + (int64_t)key * p.vsn + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS32; ++ks) {
            kf[ks] = as_bf16x8(load16(kr + 32 * ks, key < N));
            vf[ks] = as_bf16x8(load16(vr + 32 * ks, key < N));
        }
    }

    f32x4v dk[CB16], dv[CB16];
#pragma unroll
    for (int cb = 0; cb < CB16; ++cb) {
        dk[cb] = f32x4v{};
        dv[cb] = f32x4v{};
    }

    KvSteps<CAUSAL> steps;
    steps.init(p, kblk, hk, N, k0);
    const int n_all = steps.n_all, n_mask = steps.n_mask;
    auto step_row = [&](int s, int& hq) -> int { return steps.row(s, hq); };
    const float c = p.c;

    // Staging in two register sets: the loads of step t + 2 are issued at the start of step t
    // (into the set step t's data has just left) and stored to LDS at the end of step t + 1.
    Tile<D, kThreads16, L::TS, L::TS, 2> tq, td;
    tq.init(tid, p.qsn);
    td.init(tid, p.dsn);
    float st_stat[2] = {0.0f, 0.0f};
    auto load_step = [&](auto set, int s) {   // steps past the last one load nothing (zeros)
        constexpr int S = decltype(set)::value;
        int hq;
        const int r0 = step_row(s, hq);
        tq.template load<S>(p.q + seq_off(sp, b, hq, p.qsb, p.qsh, p.qsn), p.qsn, r0, N);
        td.template load<S>(p.dout + seq_off(sp, b, hq, p.dsb, p.dsh, p.dsn), p.dsn, r0, N);
        const int64_t so = seq_stat_off(sp, b, hq, p.H, p.N, p.total);
        // Raw LSE (wave 0) and D (wave 1), one row per lane; the LSE is converted when stored,
        // so that nothing waits for these loads before then. The branch is on a wave-uniform
        // value, so each wave loads through its own pointer.
        static_assert(kStep == 64, "one stats row per lane of waves 0 and 1");
        const int row = r0 + lane;
        if (wave_u == 0) st_stat[S] = row < N ? p.lse[so + row] : __builtin_inff();
        else if (wave_u == 1) st_stat[S] = row < N ? p.delta[so + row] : 0.0f;
    };
    auto store_step = [&](auto set, uint16_t* s) {
        constexpr int S = decltype(set)::value;
        tq.template store<S>(s + L::QR, nullptr);
        td.template store<S>(s + L::DR, nullptr);
        if (tid < kStep) {
            // exp2 domain; an LSE of -inf (a row with no allowed key) becomes +inf so that its
            // probabilities are exactly 0
            const float l = st_stat[S];
            reinterpret_cast<float*>(s + L::STATS)[tid] = (l == -__builtin_inff() ? __builtin_inff() : l) * kLog2e;
        } else if (tid < 2 * kStep) {
            reinterpret_cast<float*>(s + L::STATS)[tid] = st_stat[S];
        }
    };

    // Transposing-read lane base for a 16-wide column block: lane j of 16-lane group g addresses
    // row 4*g + j/4, column 4*(j%4); it then receives rows 4g .. 4g+3 of column i.
    const int tr_lane = (4 * g + (i >> 2)) * L::TS + 4 * (i & 3);

    // One 32-query half (m) of a step: S, dP for its two 16-query tiles, probabilities, then
    // dV^T += dO^T P and dK^T += Q^T dS. B element e of the P, dS operands is query
    // 32m + 4g + e (e < 4) or 32m + 16 + 4g + e - 4, the order two transposing reads give A.
    struct Acc { f32x4v s[2], p[2]; };
    auto sdp = [&](const uint16_t* s, int m, Acc& a) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int q0 = 32 * m + 16 * tt;   // first query of the tile within the step
            a.s[tt] = f32x4v{};
            a.p[tt] = f32x4v{};
            const uint16_t* qr = s + L::QR + (q0 + i) * L::TS + 8 * g;
            const uint16_t* dr = s + L::DR + (q0 + i) * L::TS + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS32; ++ks) {
                a.s[tt] = mfma16(*reinterpret_cast<const bf16x8*>(qr + 32 * ks), kf[ks], a.s[tt]);
                a.p[tt] = mfma16(*reinterpret_cast<const bf16x8*>(dr + 32 * ks), vf[ks], a.p[tt]);
            }
        }
    };
    auto probs = [&](bool mask, const uint16_t* s, int m, int qt0, const Acc& a, bf16x8& pb, bf16x8& db) {
        const float* sL = reinterpret_cast<const float*>(s + L::STATS);
        const float* sDel = sL + kStep;
        float pv[8], dsv[8];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int q0 = 32 * m + 16 * tt;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + q0 + 4 * g);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(sDel + q0 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pe = fast_exp2(fmaf(a.s[tt][r], c, -l4[r]));
                if (mask && key > qt0 + q0 + 4 * g + r) pe = 0.0f;
                pv[4 * tt + r] = pe;
                dsv[4 * tt + r] = pe * (a.p[tt][r] + d4[r]);   // d4 = -D
            }
        }
        pb = pack8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        db = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
    };
    auto grads = [&](const uint16_t* s, int m, const bf16x8& pb, const bf16x8& db) {
        const uint16_t* qt = s + L::QR + tr_lane + 32 * m * L::TS;
        const uint16_t* dt = s + L::DR + tr_lane + 32 * m * L::TS;
#pragma unroll
        for (int cb = 0; cb < CB16; ++cb) {
            dv[cb] = mfma16(read_tr_operand16(dt + 16 * cb, L::TS), pb, dv[cb]);
            dk[cb] = mfma16(read_tr_operand16(qt + 16 * cb, L::TS), db, dk[cb]);
        }
    };
    // A step as a pipeline inside the wave, so that each half's exponentials sit beside
    // independent matrix products: S, dP of half 0; S, dP of half 1 beside half 0's
    // probabilities; the gradient products of half 0 beside half 1's probabilities; then
    // half 1's gradient products. Scheduling-group hints alternate the two streams.
    auto step = [&](bool mask, const uint16_t* s, int qt0) {
        Acc a0, a1;
        bf16x8 pb0, db0, pb1, db1;
        sdp(s, 0, a0);
        sdp(s, 1, a1);
        probs(mask, s, 0, qt0, a0, pb0, db0);
        grads(s, 0, pb0, db0);
        probs(mask, s, 1, qt0, a1, pb1, db1);
        grads(s, 1, pb1, db1);
        // LDS reads run AHEAD ahead of the products that use them: one 16-byte read per S/dP
        // product, two transposing reads per gradient product.
        constexpr int AHEAD = 6;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
        for (int k = 0; k < 4 * KS32; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // S, dP half 0
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 4 * KS32; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // S, dP half 1
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // probabilities half 0
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 2 * CB16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // gradients half 0
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // probabilities half 1
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };

    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    if (n_all > 0) {
        load_step(Set0{}, 0);
        store_step(Set0{}, smem);
    }
    // Settle every outstanding load (the K, V rows included) so that no wait on them is left
    // inside the loop; then start the loads of step 1.
    __builtin_amdgcn_s_waitcnt(0);
    load_step(Set1{}, 1);
    __syncthreads();
    // Step t runs from LDS stage t % 2 with register set t % 2; the loops take steps in pairs
    // so that both are fixed at compile time. The masked steps are an even number except when
    // a key block sees a single step, and then every step is masked.
    int t = 0;
    auto iterate = [&](auto set, bool mask) {
        constexpr int S = decltype(set)::value;
        load_step(set, t + 2);
        int hq_unused;
        const int r0 = step_row(t, hq_unused);
        step(mask, smem + S * L::STAGE, r0);
        store_step(std::integral_constant<int, 1 - S>{}, smem + (1 - S) * L::STAGE);   // step t + 1
        __syncthreads();
        ++t;
    };
    while (t + 1 < n_mask) {
        iterate(Set0{}, true);
        iterate(Set1{}, true);
    }
    if (t < n_mask) iterate(Set0{}, true);
    while (t + 1 < n_all) {
        iterate(Set0{}, false);
        iterate(Set1{}, false);
    }
    if (t < n_all) iterate(Set0{}, false);

    if (key < N) {
        uint16_t* dkr = p.dk + seq_off(sp, b, hk, p.dksb, p.dksh, p.dksn) + (int64_t)key * p.dksn;
        uint16_t* dvr = p.dv + seq_off(sp, b, hk, p.dvsb, p.dvsh, p.dvsn) + (int64_t)key * p.dvsn;
        const float sc = p.scale;
#pragma unroll
        for (int cb = 0; cb < CB16; ++cb) {
            bf16x4 a, v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = (__bf16)(dk[cb][e] * sc);
                v[e] = (__bf16)(dv[cb][e]);
            }
            *reinterpret_cast<bf16x4*>(dkr + 16 * cb + 4 * g) = a;
            *reinterpret_cast<bf16x4*>(dvr + 16 * cb + 4 * g) = v;
        }
    }
}

// ----------------------------------------------------------------------------- dK, dV, head dimension 128
// A workgroup owns 128 keys in four groups of 32. Each group is served by a pair of waves
// that share the staged Q and dO tiles and split the group's four products:
// * the P wave (waves 0-3) computes S = Q K^T, P = exp2(S scale log2(e) - LSE log2(e)) and
//   dV^T += dO^T P, and hands P to its partner through LDS as fp16 (P <= 1; rounding to
//   nearest loses at most 2^-11 of it, a quarter of what bf16 would, so dS = P (dP - D)
//   keeps nearly the accuracy of an fp32 P, which would not fit the LDS budget);
// * the dS wave (waves 4-7) computes dP - D of a step (its accumulators start at -D), kept in
//   registers until P arrives, then dS = P o (dP - D) and dK^T += Q^T dS.
// Every product is a 32x32x16 one with the lane's key as its column: K (P wave) or V (dS
// wave) rows of the key are register B operands of S and dP, whose accumulators (rows =
// queries) turn into the B operands of the gradient products without any exchange between
// lanes; Q and dO rows (S, dP) and their transposes (dV, dK, via ds_read_b64_tr_b16) come
// from one unpadded copy of each tile whose 16-byte chunks are XOR-swizzled so that both
// read patterns are free of bank conflicts. Against 16 keys per wave on 16x16x32 products,
// this reads a quarter of the LDS bytes per product.
//
// The two kinds of wave alternate as in the forward: an iteration t has two phases, each
// with one kind of wave on the matrix cores and the other on its vector work. Phase A: the
// P waves run dV(t) (P(t) kept in registers from the previous phase) and S(t + 1), while the
// dS waves read P(t) from the single exchange buffer, form dS(t) and issue the loads of step
// t + 3. Phase B, after a barrier: the P waves form P(t + 1) and overwrite the exchange
// buffer, while the dS waves run dK(t) and dP(t + 1) (kept in registers for the next phase
// A). So every phase holds 32 products per SIMD, and the vector work of each kind of wave
// sits beside the other's products. Tiles travel from memory straight into LDS (four
// stages: steps t and t + 1 are read, t + 2 and t + 3 are loading), with the step's LSE
// (pre-converted to the exp2 domain by pre_kernel) and -D rows. Only the dS waves load, in
// phase A, where their own work is vector work: issuing the loads of a step stalls a wave
// for hundreds of cycles while the address path works through them. Product phases run at
// raised wave priority, so that they issue ahead of the neighbour's vector work. Rows past
// the sequence end read as zeros, which makes their contributions exactly 0 (zero dO rows
// for dV; dP = 0 and D = 0 for dK).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr int kPairStages = 4;
constexpr int kPairStatB = 2 * kStep * 4;                      // lse2[64], -D[64]
constexpr int kPairStageB = 2 * kLdsTileB + kPairStatB;       // Q | dO | lse2 | -D
constexpr int kPairXB = 4 * kStep * 32 * 2;                   // P of one step for four key groups, fp16

// Pointers into global memory that stay global (not generic) after passing through an
// empty asm statement, so that stores through them remain global stores.
using GlobalU16 = __attribute__((address_space(1))) uint16_t;
using GlobalU32x4 = __attribute__((address_space(1))) u32x4;

template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void dkdv_pair_kernel(KVParams p) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kPairStages * kPairStageB + kPairXB];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const bool pwave = wave_u < 4;   // uniform per wave
    const int grp = wave_u & 3;
    // Block-sparse: plain order, so that all XCDs work on the same head at once and its
    // Q/dO stay in the cache they share (key-side lists reach across the whole head).
    const int logical = p.q_offsets ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    const int bhk = logical / p.nkb, kblk = logical % p.nkb;   // ascending: longest first under causal
    const int hk = bhk / p.B, b = bhk % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int k0 = kblk * kKV_BK;
    if (k0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)
    const int key = k0 + 32 * grp + i;

    // K (P waves) or V (dS waves) of the lane's key: k-step ks holds d = 16 ks + 8 hf .. + 7.
    bf16x8 kv[D / 16];
    {
        const uint16_t* base = pwave ? p.k + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn) + (int64_t)key * p.ksn
                                     : p.v + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn) + (int64_t)key * p.vsn;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kv[ks] = as_bf16x8(load16(base + 16 * ks + 8 * hf, key < N));
    }
    f32x16 acc[D / 32];   // dV^T (P waves) or dK^T (dS waves): row = head-dimension column, column = key
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

    KvSteps<CAUSAL> steps;
    steps.init(p, kblk, hk, N, k0);
    const int n_all = steps.n_all, n_mask = steps.n_mask, m_per = steps.m_per, u_per = steps.u_per;
    const float c = p.c;

    // Per-lane LDS byte offsets within a tile: row reads (row i, chunk 2 ks + hf) and
    // transposing reads (per 32-column block cb, for the lane's row and the row 8 below it),
    // both in the kSwzBoth layout.
    uint32_t ar[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ar[ks] = (uint32_t)(i * kLdsRowB + 16 * ((2 * ks + hf) ^ swz<kSwzBoth>(i)));
    uint32_t at[D / 32][2];
    {
        const int g16 = (lane >> 4) & 1, j16 = lane & 15;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            const int row = 4 * hf + (j16 >> 2) + 8 * h8;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int chunk = 4 * cb + 2 * g16 + ((j16 & 3) >> 1);
                at[cb][h8] = (uint32_t)(row * kLdsRowB + 16 * (chunk ^ swz<kSwzBoth>(row)) + 8 * (j16 & 1));
            }
        }
    }
    const uint32_t lds0 = lds_address(smem);
    const uint32_t xbuf = lds0 + kPairStages * kPairStageB;
    // The P wave reads Q rows and dO transposes, the dS wave dO rows and Q transposes; the P
    // wave reads the lse2 row of a stage, the dS wave the -D row (16 bytes per lane group of four
    // queries: 4 hf + 32 m + 8 j).
    const uint32_t row_tile = pwave ? 0u : (uint32_t)kLdsTileB;
    const uint32_t tr_tile = pwave ? (uint32_t)kLdsTileB : 0u;
    const uint32_t stat_lane = 2 * kLdsTileB + (pwave ? 0u : (uint32_t)(kStep * 4)) + 16 * hf;
    // the lane's 16-byte slot of the exchange buffer for (group, half m, k-step st)
    const uint32_t xlane = (uint32_t)(grp * 4 * 1024 + 16 * lane);

    // Loads (dS waves only): each dS wave fetches four of the sixteen 1-KB pieces (four rows
    // each) of both the Q and the dO tile; wave 4 also the lse2 row, wave 5 the -D row. The
    // steps are walked in order with an iterator: the query head changes only at the end of a
    // run (a head's masked steps, then its unmasked ones), so the per-head bases move by one
    // add then.
    const int G = p.G;
    const int h0 = hk * G;
    const uint32_t qsn2 = (uint32_t)(2 * p.qsn), dsn2 = (uint32_t)(2 * p.dsn);   // row strides in bytes
    const unsigned char* const q_head0 = reinterpret_cast<const unsigned char*>(p.q + seq_off(sp, b, h0, p.qsb, p.qsh, p.qsn));
    const unsigned char* const d_head0 =
        reinterpret_cast<const unsigned char*>(p.dout + seq_off(sp, b, h0, p.dsb, p.dsh, p.dsn));
    const float* const st_head0 = (wave_u == 4 ? p.lse2 : p.delta) + seq_stat_off(sp, b, h0, p.H, p.N, p.total);
    const int64_t st_dh = sp.packed ? p.total : (int64_t)p.N;   // statistics stride between heads
    const unsigned char* ld_q = q_head0;
    const unsigned char* ld_d = d_head0;
    const float* ld_st = st_head0;
    uint32_t qoff[4], doff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * (4 * grp + j) + (lane >> 4), slot = lane & 15;
        const uint32_t sw = 16 * (slot ^ swz<kSwzBoth>(row));
        qoff[j] = (uint32_t)row * qsn2 + sw;
        doff[j] = (uint32_t)row * dsn2 + sw;
    }
    const uint32_t lds_piece = 4096u * (uint32_t)grp;
    const bool stat_wave = wave_u == 4 || wave_u == 5;
    const uint32_t lds_stat = 2 * kLdsTileB + (uint32_t)((wave_u - 4) * kStep * 4);
    int ld_gq = 0, ld_j = 0;
    bool ld_masked = m_per > 0;
    auto issue_next = [&](uint32_t stage) {
        // first row of the step at (ld_masked, ld_gq, ld_j); N for a skipped list entry
        int r0;
        if (!steps.sparse) {
            r0 = (steps.t0 + (ld_masked ? ld_j : m_per + ld_j)) * kStep;
        } else {
            int e = ld_j >> 1;
            if (ld_masked) e = steps.diag;
            else if (m_per && e >= steps.diag) ++e;
            const int qb = load_uniform(steps.qi, steps.lo + e);
            r0 = (qb < 0 || qb >= steps.nqb || (CAUSAL && qb < kblk)) ? N : qb * kKV_BK + (ld_j & 1) * kStep;
            r0 = r0 < N ? r0 : N;
        }
        const int rows = min(N - r0, kStep);   // rows of the tile inside the sequence (<= 0: none)
        const uint64_t qb64 = reinterpret_cast<uint64_t>(ld_q) + (uint64_t)(uint32_t)r0 * qsn2;
        const uint64_t db64 = reinterpret_cast<uint64_t>(ld_d) + (uint64_t)(uint32_t)r0 * dsn2;
        i32x4 rq, rd;
        rq[0] = (int)(uint32_t)qb64;
        rq[1] = (int)((uint32_t)(qb64 >> 32) & 0xffffu);
        rq[2] = rows > 0 ? (int)((uint32_t)(rows - 1) * qsn2 + 2 * D) : 0;
        rq[3] = 0x00020000;
        rd[0] = (int)(uint32_t)db64;
        rd[1] = (int)((uint32_t)(db64 >> 32) & 0xffffu);
        rd[2] = rows > 0 ? (int)((uint32_t)(rows - 1) * dsn2 + 2 * D) : 0;
        rd[3] = 0x00020000;
        const uint32_t piece = stage + lds_piece;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            load16_to_lds(rq, qoff[j], piece + 1024u * j);
            load16_to_lds(rd, doff[j], piece + kLdsTileB + 1024u * j);
        }
        if (stat_wave)
            load4_to_lds(rsrc_words(ld_st + r0, rows > 0 ? (uint32_t)(4 * rows) : 0u), (uint32_t)(4 * lane),
                         stage + lds_stat);
        // advance to the next step
        if (++ld_j == (ld_masked ? m_per : u_per)) {
            ld_j = 0;
            if (++ld_gq == G) {
                ld_gq = 0;
                ld_masked = false;
                ld_q = q_head0;
                ld_d = d_head0;
                ld_st = st_head0;
            } else {
                ld_q += 2 * p.qsh;
                ld_d += 2 * p.dsh;
                ld_st += st_dh;
            }
        }
    };

    // Read-ahead of the LDS operands: without the scheduling hints the compiler issues each
    // product right behind its own reads and waits for them (lgkmcnt(0)), exposing the full
    // LDS latency on every product. Row-read phase (S or dP): 16 products, one read each, six
    // ahead; gradient phase (dV or dK): 16 products, two transposing reads each, ten ahead.
    // Each product phase is fenced off (sched_barrier) so that the statistics and exchange
    // reads of the vector phases cannot take the places the hints give its reads.
    // Addresses: one add per column (hidden from the compiler, which would otherwise fold the
    // row offsets into more adds), the row offsets in the instructions' immediate fields.
    auto rows_phase_hints = [] {
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int k = 0; k < 10; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    };
    auto grad_phase_hints = [] {
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
        for (int k = 0; k < 11; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
    };
    // S (P wave) or dP (dS wave) of the stage at byte offset `so`: rows of the wave's row tile
    // times the register K or V, accumulated onto `a`.
    auto row_products = [&](uint32_t so, f32x16 (&a)[2]) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        const uint32_t rb = lds0 + so + row_tile;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            uint32_t x = ar[ks] + rb;
            asm("" : "+v"(x));
#pragma unroll
            for (int m = 0; m < 2; ++m) a[m] = mfma32(lds16(x + 32 * m * kLdsRowB), kv[ks], a[m]);
        }
        rows_phase_hints();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };
    // acc += (transposed tile)^T (P or dS): 32 transposing reads, 16 products.
    auto grad_products = [&](uint32_t so, const bf16x8 (&bop)[2][2]) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        const uint32_t tb = lds0 + so + tr_tile;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            uint32_t x0 = at[cb][0] + tb, x1 = at[cb][1] + tb;
            asm("" : "+v"(x0), "+v"(x1));
            bf16x8 op[2][2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const uint32_t ro = (32 * m + 16 * s2) * kLdsRowB;
                    const u32x2 lo = lds_tr4(x0 + ro);
                    const u32x2 hi = lds_tr4(x1 + ro);
                    u32x4 x;
                    x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
                    op[m][s2] = as_bf16x8(x);
                }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) acc[cb] = mfma32(op[m][s2], bop[m][s2], acc[cb]);
        }
        grad_phase_hints();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    // P wave, vector phase of the step at stage `so` with first row r0: P from S (masked in the
    // diagonal steps), to the exchange buffer (fp16) and as bf16 B operands.
    auto probs = [&](auto masked_c, uint32_t so, int r0, const f32x16 (&sacc)[2], bf16x8 (&pb)[2][2]) {
        constexpr bool MASKED = decltype(masked_c)::value;
        uint32_t sa = stat_lane + so + lds0;
        uint32_t xa = xlane + xbuf;
        asm("" : "+v"(sa), "+v"(xa));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            // element r: query 32 m + 8 (r / 4) + 4 hf + r % 4 of the step (acc_row)
            float pr[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 l4 = lds_f32x4(sa + 4 * (32 * m + 8 * j));
#pragma unroll
                for (int e = 0; e < 4; ++e) pr[4 * j + e] = fast_exp2(fmaf(sacc[m][4 * j + e], c, -l4[e]));
            }
            if constexpr (MASKED) {
                // keys after their query: key - r0 - 32 m - 4 hf > 8 (r / 4) + r % 4
                const int lim = key - r0 - 32 * m - 4 * hf;
#pragma unroll
                for (int r = 0; r < 16; ++r) pr[r] = 8 * (r >> 2) + (r & 3) < lim ? 0.0f : pr[r];
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                pb[m][s2] = pack8(pr[8 * s2], pr[8 * s2 + 1], pr[8 * s2 + 2], pr[8 * s2 + 3], pr[8 * s2 + 4],
                                  pr[8 * s2 + 5], pr[8 * s2 + 6], pr[8 * s2 + 7]);
                f16x8 h;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (_Float16)pr[8 * s2 + e];
                *(__attribute__((address_space(3))) f16x8*)(uintptr_t)(xa + (2 * m + s2) * 1024) = h;
            }
        }
    };

    // dS wave: dP - D of the step at stage `so` into dacc (the accumulators start at -D).
    f32x16 dacc[2];
    auto dp_products = [&](uint32_t so) {
        uint32_t sa = stat_lane + so + lds0;
        asm("" : "+v"(sa));
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 d4 = lds_f32x4(sa + 4 * (32 * m + 8 * j));
#pragma unroll
                for (int e = 0; e < 4; ++e) dacc[m][4 * j + e] = d4[e];
            }
        row_products(so, dacc);
    };
    // dS wave: dS = P (dP - D) with P from the exchange buffer and dP - D in dacc.
    auto ds_values = [&](bf16x8 (&db)[2][2]) {
        uint32_t xa = xlane + xbuf;
        asm("" : "+v"(xa));
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const f16x8 h = *(const __attribute__((address_space(3))) f16x8*)(uintptr_t)(xa + (2 * m + s2) * 1024);
                float ds[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ds[e] = (float)h[e] * dacc[m][8 * s2 + e];
                db[m][s2] = pack8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
            }
    };

    // dS wave, stored-dS mode: the step's dS as rounded for the dK product, to its tile, in
    // register-fragment order: [query half][key group grp][m][s2][lane][8 values], so that each
    // store instruction writes 1 KB of whole cache lines. Lane (hf, i) holds key 32 grp + i and,
    // per (m, s2), the 8 queries 32 m + 16 s2 + 4 hf + {0..3, 8..11} of the 64-query step (the
    // dQ pass gathers them back into rows). Keys past the sequence end store zeros (their P is
    // not masked and is finite only for bounded LSE). The steps are walked like the loads, one
    // behind the products; the stores are issued after the iteration's load wait, so that they
    // complete during the next iteration.
    int sv_gq = 0, sv_j = 0;
    bool sv_masked = m_per > 0;
    const bool tail_block = k0 + kKV_BK > N;   // uniform: some of the block's keys are past the end
    const bool key_out = key >= N;
    // The address of the step's dS tile half for this lane; advances the store iterator.
    // Computed early in the iteration, where the dS waves would otherwise wait for the P
    // waves' S products, so that only the stores remain behind the gradient products.
    auto ds_address = [&]() -> uint16_t* {
        int64_t tile;
        int half;
        if (!steps.sparse) {
            const int s = steps.t0 + (sv_masked ? sv_j : m_per + sv_j);   // the step's 64-row index
            const int qb = s >> 1;
            half = s & 1;
            tile = CAUSAL ? (int64_t)kblk * p.nqbt - (int64_t)kblk * (kblk - 1) / 2 + (qb - kblk)
                          : (int64_t)kblk * p.nqbt + qb;
        } else {
            int e = sv_j >> 1;   // list entry (from lo), as in KvSteps::row
            if (sv_masked) e = steps.diag;
            else if (m_per && e >= steps.diag) ++e;
            tile = steps.lo + e;
            half = sv_j & 1;
        }
        uint16_t* dst = p.ds + ((int64_t)b * p.H + (h0 + sv_gq)) * p.ds_bh + tile * (kKV_BK * 128) +
                        half * 8192 + grp * 2048 + lane * 8;
        if (++sv_j == (sv_masked ? m_per : u_per)) {
            sv_j = 0;
            if (++sv_gq == G) {
                sv_gq = 0;
                sv_masked = false;
            }
        }
        return dst;
    };
    auto store_ds = [&](bf16x8 (&db)[2][2], GlobalU16* dst) {
        if (tail_block) {
            asm volatile("");   // a branch, not selects on every step: only the last key block has such keys
            if (key_out) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) db[m][s2] = bf16x8{};
            }
        }
        // written once and read once by the dQ pass: non-temporal stores, whole lines
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4, db[m][s2]),
                                            reinterpret_cast<GlobalU32x4*>(dst + 512 * (2 * m + s2)));
    };

    if (!pwave) {
        if (n_all > 0) issue_next(lds0);
        if (n_all > 1) issue_next(lds0 + kPairStageB);
    }
    // Settle every outstanding load (the K/V rows and steps 0 and 1) before the loop.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Iterations t = -1 .. n_all - 1 (two phases each, see above; iteration -1 only starts
    // step 0). Stage of step s: s % 4; the loads of step t + 3 go to the stage of step t - 1,
    // last read in iteration t - 1. Each kind of wave runs its own copy of the loop (the same
    // iterations and barriers), so that neither holds the other's registers. The P waves take
    // the masked steps first, in a loop of their own, so that the others carry no element test.
    int t = -1;
    auto stage_of = [&](int s) -> uint32_t { return (uint32_t)((s & (kPairStages - 1)) * kPairStageB); };
    if (pwave) {
        bf16x8 pb[2][2];   // P(t) as bf16 B operands, from phase B of iteration t - 1 to dV(t)
        auto iterate = [&](auto masked_c) {
            const int tn = t + 1;
            if (t >= 0) grad_products(stage_of(t), pb);   // dV(t)
            f32x16 sacc[2];
            if (tn < n_all) {
                sacc[0] = f32x16{};
                sacc[1] = f32x16{};
                row_products(stage_of(tn), sacc);          // S(t + 1)
            }
            __syncthreads();   // the dS waves have read the exchange buffer
            if (tn < n_all) {
                // masked steps (the first n_mask): the diagonal block's halves, m_per per head
                const int r0 = k0 + (m_per == 2 ? (tn & 1) : 0) * kStep;
                probs(masked_c, stage_of(tn), r0, sacc, pb);
            }
            __syncthreads();
            ++t;
        };
        while (t + 1 < n_mask) iterate(std::true_type{});
        while (t < n_all) iterate(std::false_type{});
    } else {
        while (t < n_all) {
            const int tn = t + 1;
            bf16x8 db[2][2];
            if (t >= 0) ds_values(db);
            GlobalU16* ds_dst = nullptr;
            if (t >= 0 && p.ds != nullptr) {
                ds_dst = (GlobalU16*)ds_address();
                asm volatile("" : "+v"(ds_dst));   // keep the address work here, not at the stores
            }
            const bool more = t + 3 < n_all;
            if (more) issue_next(lds0 + stage_of(t + 3));
            __syncthreads();   // the exchange buffer is read; the P waves may overwrite it
            if (t >= 0) grad_products(stage_of(t), db);   // dK(t)
            if (tn < n_all) dp_products(stage_of(tn));    // dP(t + 1)
            // step t + 2 must have arrived; step t + 3's loads may stay in flight
            if (more) {
                if (stat_wave) __builtin_amdgcn_s_waitcnt(0x0F70 | 9);   // vmcnt(9)
                else __builtin_amdgcn_s_waitcnt(0x0F70 | 8);             // vmcnt(8)
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
            }
            if (t >= 0 && p.ds != nullptr) store_ds(db, ds_dst);
            __syncthreads();
            ++t;
        }
    }

    // dV (P waves) or dK (dS waves) of the wave's 32 keys, through the LDS the loop has freed
    static_assert(sizeof(smem) >= 8 * kRowStageWaveB, "every wave stages its rows in LDS");
    store_rows_staged(acc, pwave ? 1.0f : p.scale, i, hf, lane,
                      pwave ? p.dv + seq_off(sp, b, hk, p.dvsb, p.dvsh, p.dvsn)
                            : p.dk + seq_off(sp, b, hk, p.dksb, p.dksh, p.dksn),
                      pwave ? p.dvsn : p.dksn, k0 + 32 * grp, N, lds0 + (uint32_t)wave_u * kRowStageWaveB);
}

// ----------------------------------------------------------------------------- dQ
constexpr int kQ_BQ = 128;   // query rows per workgroup (32 per wave)

struct QParams {
    const uint16_t *q, *k, *v, *dout;
    const float* lse;
    const float* delta;
    uint16_t* dq;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, dsb, dsh, dsn, dqsb, dqsh, dqsn;
    int B, H, N, nqb;
    int G;
    const int32_t* cu;
    int64_t total;
    const int32_t* kv_offsets;   // query-side block lists (block-sparse mode), or nullptr
    const int32_t* kv_indices;
    int64_t nnz;
    float c;
    float scale;
};

template <int D>
struct QCfg {
    using C = BCfg<D>;
    // one stage: K rows | K (transposed reads) | V rows
    static constexpr int KR = 0, KT = C::RE, VR = C::RE + C::TE;
    static constexpr int STAGE = 2 * C::RE + C::TE;
};

// Single LDS stage (two workgroups fit on a CU): the next tile is loaded into registers
// during the current step and written after a barrier.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(QParams p) {
    using C = BCfg<D>;
    using L = QCfg<D>;
    constexpr int KSTEPS = C::KSTEPS, CB = C::CB;
    __shared__ __attribute__((aligned(16))) uint16_t smem[L::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    // Block-sparse: plain order, so that all XCDs work on the same head at once and its K/V
    // stay in the cache they share (strided lists reach back over the whole head).
    const int logical = p.kv_offsets ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical % p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int hh = bh / p.B, b = bh % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qb * kQ_BQ;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const uint16_t* kp = p.k + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const uint16_t* vp = p.v + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);
    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kQ_BQ - 1, N - 1);

    bf16x8 qf[KSTEPS], df[KSTEPS];
    {
        const uint16_t* qr = p.q + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn) + (int64_t)qrow * p.qsn + 8 * hf;
        const uint16_t* dr = p.dout + seq_off(sp, b, hh, p.dsb, p.dsh, p.dsn) + (int64_t)qrow * p.dsn + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qf[ks] = as_bf16x8(load16(qr + 16 * ks, qrow < N));
            df[ks] = as_bf16x8(load16(dr + 16 * ks, qrow < N));
        }
    }
    const int64_t so = seq_stat_off(sp, b, hh, p.H, p.N, p.total);
    float lse2 = 0.0f, dlt = 0.0f;   // dlt: -D of the row
    if (qrow < N) {
        float l = p.lse[so + qrow];
        if (l == -__builtin_inff()) l = __builtin_inff();
        lse2 = l * kLog2e;
        dlt = p.delta[so + qrow];
    }

    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    // Steps: 64-key tiles. Dense: from 0 to the end (causal: to the block's last row).
    // Block-sparse: both halves of every key block listed for this query block; entries out
    // of range (or, causal, above the diagonal) are skipped.
    int nsteps = (N + kStep - 1) / kStep;
    if (CAUSAL) nsteps = min(nsteps, qlast / kStep + 1);
    const bool sparse = p.kv_offsets != nullptr;
    int64_t lo = 0;
    if (sparse) {
        int64_t hi = load_uniform(p.kv_offsets, qb + 1);
        lo = load_uniform(p.kv_offsets, qb);
        lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
        hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
        nsteps = (int)(2 * (hi - lo));
    }
    const int nkb = (N + kQ_BQ - 1) / kQ_BQ;
    auto step_key = [&](int t) -> int {   // first key of step t, or -1 to skip it
        if (!sparse) return t * kStep;
        const int kb = load_uniform(p.kv_indices, lo + (t >> 1));
        if (kb < 0 || kb >= nkb || (CAUSAL && kb > qb)) return -1;
        const int kt0 = kb * kQ_BQ + (t & 1) * kStep;
        return (kt0 < N && (!CAUSAL || kt0 <= qlast)) ? kt0 : -1;
    };
    const float c = p.c;
    const uint16_t* kt_base = tr_lane_base(smem + L::KT, C::TS, lane);

    Tile<D> tk, tv;
    tk.init(tid, p.ksn);
    tv.init(tid, p.vsn);
    if (nsteps > 0) {
        const int kt0 = step_key(0);
        if (kt0 >= 0) {
            tk.load(kp, p.ksn, kt0, N);
            tv.load(vp, p.vsn, kt0, N);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int t = 0; t < nsteps; ++t) {
        tk.store(smem + L::KR, smem + L::KT);
        tv.store(smem + L::VR, nullptr);
        __syncthreads();
        if (t + 1 < nsteps) {
            const int ktn = step_key(t + 1);
            if (ktn >= 0) {
                tk.load(kp, p.ksn, ktn, N);
                tv.load(vp, p.vsn, ktn, N);
            }
        }
        const int kt = step_key(t);
        if (kt >= 0 && qw0 < N && (!CAUSAL || kt <= qw0 + 31)) {
            const bool masked = (kt + kStep > N) || (CAUSAL && kt + kStep - 1 > qw0);
            bf16x8 db[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sacc = {}, pacc = {};
                const uint16_t* kr = smem + L::KR + (32 * kb + i) * C::RS + 8 * hf;
                const uint16_t* vr = smem + L::VR + (32 * kb + i) * C::RS + 8 * hf;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    sacc = mfma32(*reinterpret_cast<const bf16x8*>(kr + 16 * ks), qf[ks], sacc);
                    pacc = mfma32(*reinterpret_cast<const bf16x8*>(vr + 16 * ks), df[ks], pacc);
                }
                // P from the LSE; in diagonal and tail tiles the masked keys' probabilities
                // are zeroed in one block the wave skips elsewhere (a test inside the element
                // loop became an exec-masked region per element, executed on every tile).
                float dsv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] = fast_exp2(fmaf(sacc[r], c, -lse2));
                if (masked) {
                    // key of element r: kt + 4 hf + 32 kb + 8 (r / 4) + r % 4 (acc_row)
                    int lim = N - 1 - kt - 4 * hf - 32 * kb;
                    if (CAUSAL) lim = min(lim, qrow - kt - 4 * hf - 32 * kb);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) dsv[r] = 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] *= pacc[r] + dlt;   // dlt = -D
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    db[kb][st] = pack8(dsv[8 * st], dsv[8 * st + 1], dsv[8 * st + 2], dsv[8 * st + 3],
                                       dsv[8 * st + 4], dsv[8 * st + 5], dsv[8 * st + 6], dsv[8 * st + 7]);
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        dq[cb] = mfma32(read_tr_operand(kt_base, (32 * kb + 16 * st) * C::TS + 32 * cb, C::TS),
                                        db[kb][st], dq[cb]);
        }
        __syncthreads();
    }

    if (qrow < N) {
        uint16_t* dqr = p.dq + seq_off(sp, b, hh, p.dqsb, p.dqsh, p.dqsn) + (int64_t)qrow * p.dqsn;
        const float sc = p.scale;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (__bf16)(dq[cb][4 * j + e] * sc);
                *reinterpret_cast<bf16x4*>(dqr + 32 * cb + 8 * j + 4 * hf) = a;
            }
    }
}

// dQ at head dimension 128 with the K/V tiles loaded straight into LDS: one copy of K, with
// the swizzle that serves both its row reads (S^T) and its transposing reads (dQ^T), and V;
// two 32 KB stages (two workgroups still fit on a CU). The next step's loads are issued at
// the start of a step into the other stage and waited for before the step's closing barrier.
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void dq_dma_kernel(QParams p) {
    constexpr int D = 128;
    using C = BCfg<D>;
    constexpr int KSTEPS = C::KSTEPS, CB = C::CB;
    constexpr int STAGEB = 2 * kLdsTileB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGEB];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    // Block-sparse: plain order, so that all XCDs work on the same head at once and its K/V
    // stay in the cache they share (strided lists reach back over the whole head).
    const int logical = p.kv_offsets ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical % p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int hh = bh / p.B, b = bh % p.B;   // head-major: an XCD's share spans every sequence
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qb * kQ_BQ;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const uint16_t* kp = p.k + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const uint16_t* vp = p.v + seq_off(sp, b, hk, p.vsb, p.vsh, p.vsn);
    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kQ_BQ - 1, N - 1);

    bf16x8 qf[KSTEPS], df[KSTEPS];
    {
        const uint16_t* qr = p.q + seq_off(sp, b, hh, p.qsb, p.qsh, p.qsn) + (int64_t)qrow * p.qsn + 8 * hf;
        const uint16_t* dr = p.dout + seq_off(sp, b, hh, p.dsb, p.dsh, p.dsn) + (int64_t)qrow * p.dsn + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qf[ks] = as_bf16x8(load16(qr + 16 * ks, qrow < N));
            df[ks] = as_bf16x8(load16(dr + 16 * ks, qrow < N));
        }
    }
    const int64_t so = seq_stat_off(sp, b, hh, p.H, p.N, p.total);
    float lse2 = 0.0f, dlt = 0.0f;   // dlt: -D of the row
    if (qrow < N) {
        float l = p.lse[so + qrow];
        if (l == -__builtin_inff()) l = __builtin_inff();
        lse2 = l * kLog2e;
        dlt = p.delta[so + qrow];
    }

    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    // Steps: 64-key tiles. Dense: from 0 to the end (causal: to the block's last row).
    // Block-sparse: both halves of every key block listed for this query block; entries out
    // of range (or, causal, above the diagonal) are skipped.
    int nsteps = (N + kStep - 1) / kStep;
    if (CAUSAL) nsteps = min(nsteps, qlast / kStep + 1);
    const bool sparse = p.kv_offsets != nullptr;
    int64_t lo = 0;
    if (sparse) {
        int64_t hi = load_uniform(p.kv_offsets, qb + 1);
        lo = load_uniform(p.kv_offsets, qb);
        lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
        hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
        nsteps = (int)(2 * (hi - lo));
    }
    const int nkb = (N + kQ_BQ - 1) / kQ_BQ;
    auto step_key = [&](int t) -> int {   // first key of step t, or -1 to skip it
        if (!sparse) return t * kStep;
        const int kb = load_uniform(p.kv_indices, lo + (t >> 1));
        if (kb < 0 || kb >= nkb || (CAUSAL && kb > qb)) return -1;
        const int kt0 = kb * kQ_BQ + (t & 1) * kStep;
        return (kt0 < N && (!CAUSAL || kt0 <= qlast)) ? kt0 : -1;
    };
    const float c = p.c;

    // Per-lane byte offsets within a stage: row reads of K (V: + kLdsTileB), row i and
    // logical chunk 2 * ks + hf; transposing reads of K per 32-column block cb, for the
    // lane's row and the row 8 below it.
    uint32_t ar[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) ar[ks] = (uint32_t)(i * kLdsRowB + 16 * ((2 * ks + hf) ^ swz<kSwzBoth>(i)));
    uint32_t at[CB][2];
    {
        const int g16 = (lane >> 4) & 1, j16 = lane & 15;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            const int row = 4 * hf + (j16 >> 2) + 8 * h8;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int chunk = 4 * cb + 2 * g16 + ((j16 & 3) >> 1);
                at[cb][h8] = (uint32_t)(row * kLdsRowB + 16 * (chunk ^ swz<kSwzBoth>(row)) + 8 * (j16 & 1));
            }
        }
    }

    DmaStage<kThreads / 64, kSwzBoth, kSwzBoth> st;
    st.init(wave, lane, p.ksn, p.vsn);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_address(smem);
    // Loads of the key tile starting at kt0 (< N) into the stage at LDS address `stage`: the
    // per-lane offsets of the wave's four 1-KB pieces of each tile are fixed, so per step only
    // the tile base (a 32x32->64-bit multiply and an add per tensor) and the byte count change.
    const uint32_t ksn2 = (uint32_t)(2 * p.ksn), vsn2 = (uint32_t)(2 * p.vsn);
    const uint32_t piece0 = 1024u * 4u * (uint32_t)wave_u;
    auto issue = [&](int kt0, uint32_t stage) {
        const uint32_t rows = (uint32_t)min(N - kt0, kStep);
        const uint64_t kb64 = reinterpret_cast<uint64_t>(kp) + (uint64_t)(uint32_t)kt0 * ksn2;
        const uint64_t vb64 = reinterpret_cast<uint64_t>(vp) + (uint64_t)(uint32_t)kt0 * vsn2;
        i32x4 rk, rv;
        rk[0] = (int)(uint32_t)kb64;
        rk[1] = (int)((uint32_t)(kb64 >> 32) & 0xffffu);
        rk[2] = (int)((rows - 1) * ksn2 + 2 * D);
        rk[3] = 0x00020000;
        rv[0] = (int)(uint32_t)vb64;
        rv[1] = (int)((uint32_t)(vb64 >> 32) & 0xffffu);
        rv[2] = (int)((rows - 1) * vsn2 + 2 * D);
        rv[3] = 0x00020000;
        const uint32_t piece = stage + piece0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            load16_to_lds(rk, st.koff[j], piece + 1024u * j);
            load16_to_lds(rv, st.voff[j], piece + kLdsTileB + 1024u * j);
        }
    };
    static_assert(kThreads / 64 == 4, "four waves of four pieces per tile");
    if (nsteps > 0) {
        const int kt0 = step_key(0);
        if (kt0 >= 0) issue(kt0, lds0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int cur = 0;
    for (int t = 0; t < nsteps; ++t) {
        // the other stage was last read in the previous step, which ended with a barrier
        if (t + 1 < nsteps) {
            const int ktn = step_key(t + 1);
            if (ktn >= 0) issue(ktn, lds0 + (cur ^ 1) * STAGEB);
        }
        const unsigned char* buf = smem + cur * STAGEB;
        const int kt = step_key(t);
        if (kt >= 0 && qw0 < N && (!CAUSAL || kt <= qw0 + 31)) {
            const bool masked = (kt + kStep > N) || (CAUSAL && kt + kStep - 1 > qw0);
            bf16x8 db[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sacc = {}, pacc = {};
                const unsigned char* kr = buf + 32 * kb * kLdsRowB;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    sacc = mfma32(*reinterpret_cast<const bf16x8*>(kr + ar[ks]), qf[ks], sacc);
                    pacc = mfma32(*reinterpret_cast<const bf16x8*>(kr + kLdsTileB + ar[ks]), df[ks], pacc);
                }
                // P from the LSE; in diagonal and tail tiles the masked keys' probabilities
                // are zeroed in one block the wave skips elsewhere (a test inside the element
                // loop became an exec-masked region per element, executed on every tile).
                float dsv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] = fast_exp2(fmaf(sacc[r], c, -lse2));
                if (masked) {
                    // key of element r: kt + 4 hf + 32 kb + 8 (r / 4) + r % 4 (acc_row)
                    int lim = N - 1 - kt - 4 * hf - 32 * kb;
                    if (CAUSAL) lim = min(lim, qrow - kt - 4 * hf - 32 * kb);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) dsv[r] = 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] *= pacc[r] + dlt;   // dlt = -D
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    db[kb][st] = pack8(dsv[8 * st], dsv[8 * st + 1], dsv[8 * st + 2], dsv[8 * st + 3],
                                       dsv[8 * st + 4], dsv[8 * st + 5], dsv[8 * st + 6], dsv[8 * st + 7]);
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const unsigned char* p0 = buf + (32 * kb + 16 * s2) * kLdsRowB;
                        const u32x2 lo = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + at[cb][0]));
                        const u32x2 hi = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + at[cb][1]));
                        u32x4 x;
                        x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
                        dq[cb] = mfma32(as_bf16x8(x), db[kb][s2], dq[cb]);
                    }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of the next step
        __syncthreads();
        cur ^= 1;
    }

    // the wave's 32 dQ rows, through the LDS the loop has freed
    static_assert(sizeof(smem) >= (kThreads / 64) * kRowStageWaveB, "every wave stages its rows in LDS");
    store_rows_staged(dq, p.scale, i, hf, lane, p.dq + seq_off(sp, b, hh, p.dqsb, p.dqsh, p.dqsn), p.dqsn, qw0, N,
                      lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kRowStageWaveB);
}


// ----------------------------------------------------------------------------- dQ from stored dS
// With a large enough workspace the dK/dV kernel stores the bf16 dS of every (key block,
// query block) pair it visits, and dQ = scale * dS K is one product per step instead of the
// three of dq_dma_kernel (S and dP recomputed): the rows of the tile are read back rather
// than recomputed. Tile numbering within the region of one (sequence, query head), nqb =
// ceil(N / 128) with N the longest sequence: dense non-causal kb * nqb + qb; dense causal
// (qb >= kb) kb * nqb - kb (kb - 1) / 2 + qb - kb; block-sparse: the pair's entry index in the
// key-side lists (the dQ pass finds it through `pos`, written by ds_pos_kernel).
struct DsQParams {
    const uint16_t* k;
    const uint16_t* ds;
    const int32_t* pos;          // block-sparse: key-side entry of every query-side entry, or -1
    uint16_t* dq;
    int64_t ksb, ksh, ksn, dqsb, dqsh, dqsn;
    int64_t ds_bh;
    int B, H, N, nqb, G;
    const int32_t* cu;
    int64_t total;
    const int32_t* kv_offsets;   // query-side block lists (block-sparse mode), or nullptr
    const int32_t* kv_indices;
    int64_t nnz;
    float scale;
};

// For every query-side entry e (query block qb, key block kv_indices[e]) the index of qb in
// the key block's ascending key-side list, or -1 when it is not there (or the entry is out of
// range). One wave per query block, one lane per entry (a binary search each); offsets are
// clamped, so any list content stays in bounds.
__global__ __launch_bounds__(256) void ds_pos_kernel(const int32_t* kv_off, const int32_t* kv_idx,
                                                     const int32_t* q_off, const int32_t* q_idx, int64_t nnz,
                                                     int nb, int32_t* pos) {
    const int qb = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (qb >= nb) return;
    auto clampo = [&](int64_t x) -> int64_t { return x < 0 ? 0 : (x > nnz ? nnz : x); };
    const int64_t lo = clampo(kv_off[qb]);
    int64_t hi = clampo(kv_off[qb + 1]);
    if (hi < lo) hi = lo;
    for (int64_t e = lo + (threadIdx.x & 63); e < hi; e += 64) {
        const int kb = kv_idx[e];
        int32_t r = -1;
        if (kb >= 0 && kb < nb) {
            const int64_t a0 = clampo(q_off[kb]);
            int64_t z = clampo(q_off[kb + 1]);
            if (z < a0) z = a0;
            const int64_t end = z;
            int64_t a = a0;
            while (a < z) {   // first entry not below qb
                const int64_t m = (a + z) >> 1;
                if (q_idx[m] < qb) a = m + 1;
                else z = m;
            }
            if (a < end && q_idx[a] == qb) r = (int32_t)a;
        }
        pos[e] = r;
    }
}

// Lane i of a wave's 32 query positions holds query i with bits 2 and 3 swapped (the order
// the dK/dV kernel stores a step's queries in).
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// dQ^T += K^T dS^T per 64-key step: the K rows and the dS rows of the same keys are loaded
// straight into LDS (two 32 KB stages, two workgroups per CU) in the layout of dq_dma_kernel's
// K tile, and both operands come from transposing reads of them: K^T per 32-column block of the
// head dimension (the same for every wave), dS^T for the wave's 32 query positions. A dS row
// (one key, 128 query positions; position p of a 64-query half holds query p with bits 2 and
// 3 swapped) is gathered from the stored fragments: 16 bytes per 8 positions, 64 contiguous
// bytes per 4 consecutive keys. Entries the lists or the causal mask exclude are skipped; the
// stored dS of masked elements and of keys past the sequence end are zeros, so no element
// needs a mask here.
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void dq_ds_kernel(DsQParams p) {
    constexpr int D = 128, CB = D / 32;
    constexpr int STAGEB = 2 * kLdsTileB;   // K rows | dS rows (128 query positions) of 64 keys
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGEB];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int logical = p.kv_offsets ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical % p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int hh = bh / p.B, b = bh % p.B;
    const SeqSpan sp = seq_span(p.cu, p.total, b, p.N);
    const int N = sp.len;
    const int q0 = qb * kQ_BQ;
    if (q0 >= N) return;   // past the end of a shorter packed sequence (uniform per workgroup)

    const int hk = hh / p.G;
    const uint16_t* kp = p.k + seq_off(sp, b, hk, p.ksb, p.ksh, p.ksn);
    const uint16_t* dsp = p.ds + ((int64_t)b * p.H + hh) * p.ds_bh;
    const int qw0 = q0 + 32 * wave;
    const int qlast = min(q0 + kQ_BQ - 1, N - 1);

    int nsteps = (N + kStep - 1) / kStep;
    if (CAUSAL) nsteps = min(nsteps, qlast / kStep + 1);
    const bool sparse = p.kv_offsets != nullptr;
    int64_t lo = 0;
    if (sparse) {
        int64_t hi = load_uniform(p.kv_offsets, qb + 1);
        lo = load_uniform(p.kv_offsets, qb);
        lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
        hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
        nsteps = (int)(2 * (hi - lo));
    }
    const int nkb = (N + kQ_BQ - 1) / kQ_BQ;
    // first key of step t (-1: skipped) and the element offset of its key half of the tile
    auto step_src = [&](int t, int64_t& src) -> int {
        if (!sparse) {
            const int kb = t >> 1;
            const int64_t tile = CAUSAL ? (int64_t)kb * p.nqb - (int64_t)kb * (kb - 1) / 2 + (qb - kb)
                                        : (int64_t)kb * p.nqb + qb;
            src = tile * (kQ_BQ * 128) + (t & 1) * 4096;
            return t * kStep;
        }
        const int64_t e = lo + (t >> 1);
        const int kb = load_uniform(p.kv_indices, e);
        const int ps = load_uniform(p.pos, e);
        if (kb < 0 || kb >= nkb || (CAUSAL && kb > qb) || ps < 0 || ps >= p.nnz) return -1;
        const int kt0 = kb * kQ_BQ + (t & 1) * kStep;
        if (kt0 >= N || (CAUSAL && kt0 > qlast)) return -1;
        src = (int64_t)ps * (kQ_BQ * 128) + (t & 1) * 4096;
        return kt0;
    };

    // transposing-read offsets within a tile: per 32-column block cb (K^T) and for the wave's
    // query positions (dS^T), for the lane's row and the row 8 below it
    uint32_t at[CB][2], bt[2];
    {
        const int g16 = (lane >> 4) & 1, j16 = lane & 15;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            const int row = 4 * hf + (j16 >> 2) + 8 * h8;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int chunk = 4 * cb + 2 * g16 + ((j16 & 3) >> 1);
                at[cb][h8] = (uint32_t)(row * kLdsRowB + 16 * (chunk ^ swz<kSwzBoth>(row)) + 8 * (j16 & 1));
            }
            const int chunk = 4 * wave + 2 * g16 + ((j16 & 3) >> 1);
            bt[h8] = (uint32_t)(kLdsTileB + row * kLdsRowB + 16 * (chunk ^ swz<kSwzBoth>(row)) + 8 * (j16 & 1));
        }
    }

    DmaStage<kThreads / 64, kSwzBoth, kSwzBoth> st;
    st.init(wave, lane, p.ksn, 128);
    // byte offset (from the step's key half of the tile) of the fragment that fills LDS row r,
    // physical chunk c: logical chunk c ^ swizzle = 8 positions of query half h, slot 4 m + 2 s2
    // + hf; key group r / 32 of the half, lane 32 hf + r % 32
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * (4 * wave + j) + (lane >> 4);
        const int lc = (lane & 15) ^ swz<kSwzBoth>(r);
        const int h = lc >> 3, slot = lc & 7;
        const int m = slot >> 2, s2 = (slot >> 1) & 1, f = slot & 1;
        st.voff[j] = (uint32_t)(2 * (h * 8192 + (r >> 5) * 2048 + (2 * m + s2) * 512 + (32 * f + (r & 31)) * 8));
    }
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_address(smem);
    const uint32_t ksn2 = (uint32_t)(2 * p.ksn);
    const uint32_t piece0 = 1024u * 4u * (uint32_t)wave_u;
    auto issue = [&](int kt0, int64_t src, uint32_t stage) {
        const uint32_t rows = (uint32_t)min(N - kt0, kStep);
        const uint64_t kb64 = reinterpret_cast<uint64_t>(kp) + (uint64_t)(uint32_t)kt0 * ksn2;
        const uint64_t db64 = reinterpret_cast<uint64_t>(dsp + src);
        i32x4 rk, rd;
        rk[0] = (int)(uint32_t)kb64;
        rk[1] = (int)((uint32_t)(kb64 >> 32) & 0xffffu);
        rk[2] = (int)((rows - 1) * ksn2 + 2 * D);
        rk[3] = 0x00020000;
        rd[0] = (int)(uint32_t)db64;
        rd[1] = (int)((uint32_t)(db64 >> 32) & 0xffffu);
        rd[2] = (int)(2 * (kQ_BQ * 128 - (src & 4096)));   // to the end of the tile
        rd[3] = 0x00020000;
        const uint32_t piece = stage + piece0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            load16_to_lds(rk, st.koff[j], piece + 1024u * j);
            load16_to_lds(rd, st.voff[j], piece + kLdsTileB + 1024u * j);
        }
    };
    static_assert(kThreads / 64 == 4, "four waves of four pieces per tile");

    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    int64_t src_next = 0;
    int kt_next = nsteps > 0 ? step_src(0, src_next) : -1;
    if (kt_next >= 0) issue(kt_next, src_next, lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int cur = 0;
    for (int t = 0; t < nsteps; ++t) {
        const int kt = kt_next;
        // the other stage was last read in the previous step, which ended with a barrier
        if (t + 1 < nsteps) {
            kt_next = step_src(t + 1, src_next);
            if (kt_next >= 0) issue(kt_next, src_next, lds0 + (cur ^ 1) * STAGEB);
        }
        if (kt >= 0 && qw0 < N && (!CAUSAL || kt <= qw0 + 31)) {
            const unsigned char* buf = smem + cur * STAGEB;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const unsigned char* p0 = buf + (32 * kb + 16 * s2) * kLdsRowB;
                    u32x4 y;
                    {
                        const u32x2 lo2 = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + bt[0]));
                        const u32x2 hi2 = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + bt[1]));
                        y[0] = lo2[0]; y[1] = lo2[1]; y[2] = hi2[0]; y[3] = hi2[1];
                    }
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const u32x2 lo2 = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + at[cb][0]));
                        const u32x2 hi2 = lds_read_tr4(reinterpret_cast<const uint16_t*>(p0 + at[cb][1]));
                        u32x4 x;
                        x[0] = lo2[0]; x[1] = lo2[1]; x[2] = hi2[0]; x[3] = hi2[1];
                        dq[cb] = mfma32(as_bf16x8(x), as_bf16x8(y), dq[cb]);
                    }
                }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of the next step
        __syncthreads();
        cur ^= 1;
    }

    // the wave's 32 dQ rows (lane i holds query position i, i.e. row qw0 + swap23(i)), through
    // the LDS the loop has freed
    static_assert(sizeof(smem) >= (kThreads / 64) * kRowStageWaveB, "every wave stages its rows in LDS");
    store_rows_staged(dq, p.scale, swap23(i), hf, lane, p.dq + seq_off(sp, b, hh, p.dqsb, p.dqsh, p.dqsn), p.dqsn, qw0, N,
                      lds_address(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * kRowStageWaveB);
}

template <int D, bool CAUSAL>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream) {
    const Layout& L = a.L;
    {
        // D has the LSE's layout: [B, H, N], or [H, total] for packed sequences, which is the
        // same computation over one sequence of `total` rows.
        const bool packed = L.cu != nullptr;
        const int Bp = packed ? 1 : L.B;
        const int Np = packed ? (int)L.total : L.N;
        const int64_t rows = (int64_t)Bp * L.H * Np;
        constexpr int RPB = kThreads / (D / 8);
        constexpr int64_t kMaxGrid = (int64_t)1 << 16;   // the kernel strides over the rest
        const int64_t grid = std::min((rows + RPB - 1) / RPB, kMaxGrid);
        hipLaunchKernelGGL((pre_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(a.o.p), packed ? 0 : a.o.sb, a.o.sh, a.o.sn,
                           static_cast<const uint16_t*>(a.dout.p), packed ? 0 : a.dout.sb, a.dout.sh, a.dout.sn,
                           a.lse, a.delta, a.delta + rows, L.H, Np, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const float c = a.scale * kLog2e;
    const bool store_ds = D == 128 && a.ds != nullptr;
    const int nqbt = (L.N + kQ_BQ - 1) / kQ_BQ;
    if (store_ds && a.kv_offsets) {
        hipLaunchKernelGGL(ds_pos_kernel, dim3((unsigned)((nqbt + 3) / 4)), dim3(256), 0, stream, a.kv_offsets,
                           a.kv_indices, a.q_offsets, a.q_indices, a.nnz, nqbt, a.ds_pos);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        KVParams p;
        p.q = static_cast<const uint16_t*>(a.q.p);
        p.k = static_cast<const uint16_t*>(a.k.p);
        p.v = static_cast<const uint16_t*>(a.v.p);
        p.dout = static_cast<const uint16_t*>(a.dout.p);
        p.lse = a.lse;
        p.delta = a.delta;
        p.lse2 = a.delta + (int64_t)(L.cu ? 1 : L.B) * L.H * (L.cu ? L.total : L.N);
        p.dk = static_cast<uint16_t*>(a.dk);
        p.dv = static_cast<uint16_t*>(a.dv);
        p.qsb = a.q.sb; p.qsh = a.q.sh; p.qsn = a.q.sn;
        p.ksb = a.k.sb; p.ksh = a.k.sh; p.ksn = a.k.sn;
        p.vsb = a.v.sb; p.vsh = a.v.sh; p.vsn = a.v.sn;
        p.dsb = a.dout.sb; p.dsh = a.dout.sh; p.dsn = a.dout.sn;
        p.dksb = a.dksb; p.dksh = a.dksh; p.dksn = a.dksn;
        p.dvsb = a.dvsb; p.dvsh = a.dvsh; p.dvsn = a.dvsn;
        p.B = L.B; p.H = L.H; p.Hkv = L.Hkv; p.N = L.N;
        p.G = L.H / L.Hkv;
        p.cu = L.cu;
        p.total = L.total;
        p.q_offsets = a.kv_offsets ? a.q_offsets : nullptr;
        p.q_indices = a.q_indices;
        p.nnz = a.nnz;
        p.nkb = (L.N + kKV_BK - 1) / kKV_BK;
        p.c = c;
        p.scale = a.scale;
        p.ds = store_ds ? a.ds : nullptr;
        p.ds_bh = a.ds_bh;
        p.nqbt = nqbt;
        const int64_t grid = (int64_t)L.B * L.Hkv * p.nkb;
        if constexpr (D == 128)
            hipLaunchKernelGGL((dkdv_pair_kernel<CAUSAL>), dim3((unsigned)grid), dim3(512), 0, stream, p);
        else
            hipLaunchKernelGGL((dkdv16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads16), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (store_ds) {
        DsQParams p;
        p.k = static_cast<const uint16_t*>(a.k.p);
        p.ds = a.ds;
        p.pos = a.ds_pos;
        p.dq = static_cast<uint16_t*>(a.dq);
        p.ksb = a.k.sb; p.ksh = a.k.sh; p.ksn = a.k.sn;
        p.dqsb = a.dqsb; p.dqsh = a.dqsh; p.dqsn = a.dqsn;
        p.ds_bh = a.ds_bh;
        p.B = L.B; p.H = L.H; p.N = L.N;
        p.nqb = nqbt;
        p.G = L.H / L.Hkv;
        p.cu = L.cu;
        p.total = L.total;
        p.kv_offsets = a.kv_offsets;
        p.kv_indices = a.kv_indices;
        p.nnz = a.nnz;
        p.scale = a.scale;
        const int64_t grid = (int64_t)L.B * L.H * nqbt;
        hipLaunchKernelGGL((dq_ds_kernel<CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    {
        QParams p;
        p.q = static_cast<const uint16_t*>(a.q.p);
        p.k = static_cast<const uint16_t*>(a.k.p);
        p.v = static_cast<const uint16_t*>(a.v.p);
        p.dout = static_cast<const uint16_t*>(a.dout.p);
        p.lse = a.lse;
        p.delta = a.delta;
        p.dq = static_cast<uint16_t*>(a.dq);
        p.qsb = a.q.sb; p.qsh = a.q.sh; p.qsn = a.q.sn;
        p.ksb = a.k.sb; p.ksh = a.k.sh; p.ksn = a.k.sn;
        p.vsb = a.v.sb; p.vsh = a.v.sh; p.vsn = a.v.sn;
        p.dsb = a.dout.sb; p.dsh = a.dout.sh; p.dsn = a.dout.sn;
        p.dqsb = a.dqsb; p.dqsh = a.dqsh; p.dqsn = a.dqsn;
        p.B = L.B; p.H = L.H; p.N = L.N;
        p.G = L.H / L.Hkv;
        p.cu = L.cu;
        p.total = L.total;
        p.kv_offsets = a.kv_offsets;
        p.kv_indices = a.kv_indices;
        p.nnz = a.nnz;
        p.nqb = (L.N + kQ_BQ - 1) / kQ_BQ;
        p.c = c;
        p.scale = a.scale;
        const int64_t grid = (int64_t)L.B * L.H * p.nqb;
        if constexpr (D == 128)
            hipLaunchKernelGGL((dq_dma_kernel<CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
}

}  // namespace

// Library-owned backward workspace for callers that cannot allocate: one array per GPU,
// held until the process ends. In host code `scratch` only names the array (it is not a
// device address); its address on each device comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is ever handed to a kernel.
// Every call on a GPU shares the array: calls that overlap on one GPU race on it.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_workspace(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.L.d == 64) return a.causal ? launch_all<64, true>(a, stream) : launch_all<64, false>(a, stream);
    return a.causal ? launch_all<128, true>(a, stream) : launch_all<128, false>(a, stream);
}

}  // namespace fa
