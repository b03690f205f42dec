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
// S and dP are thus computed twice (7 matrix products instead of 5) in exchange for no
// atomics and bitwise-reproducible results.
//
// LDS layouts, all free of bank conflicts for the reads they serve: the dK/dV kernel stages
// its Q and dO tiles through registers into one copy with 288-byte rows, which serves both
// its row reads and its transposing reads; dq_dma_kernel loads K and V straight into LDS as
// unpadded rows with XOR-swizzled 16-byte chunks (one K copy for both read patterns);
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

// ----------------------------------------------------------------------------- D = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(kThreads) void pre_kernel(const uint16_t* o, int64_t osb, int64_t osh, int64_t osn,
                                                       const uint16_t* dout, int64_t dsb, int64_t dsh, int64_t dsn,
                                                       float* delta, int H, int N, int64_t rows) {
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
        if (row < rows && part == 0) delta[row] = acc;
    }
}

// ----------------------------------------------------------------------------- dK, dV
constexpr int kKV_BK = 128;   // keys per workgroup (32 per wave)

struct KVParams {
    const uint16_t *q, *k, *v, *dout;
    const float* lse;
    const float* delta;
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

    // Steps: 64-row query tiles, for each of the G query heads that read this K/V head in
    // turn. Dense: the tiles from the first one that can see these keys (causal) or from 0 to
    // the end. Block-sparse: both halves of every query block the key-side list names for
    // this key block. Under causal masking only the steps of the diagonal block hold keys
    // after queries: the first two of each query head (dense), or the two halves of the
    // list's diagonal entry (block-sparse: the first entry not below the key block, the lists
    // being ascending; entries before it are above-diagonal entries of the query-side lists,
    // which are skipped). Those steps are taken first, so the others run without the element
    // test. Out-of-range list entries (or, causal, entries above the diagonal) become an empty
    // tile at row N: zero-filled loads, LSE = +inf, so their probabilities are exactly 0.
    const int nsteps = (N + kStep - 1) / kStep;
    const int t0 = CAUSAL ? k0 / kStep : 0;
    int64_t lo = 0, hi = 0;
    const bool sparse = p.q_offsets != nullptr;
    if (sparse) {
        lo = load_uniform(p.q_offsets, kblk);
        hi = load_uniform(p.q_offsets, kblk + 1);
        lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
        hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
    }
    const int per = sparse ? (int)(2 * (hi - lo)) : nsteps - t0;
    const int n_all = per * p.G;
    const int nqb = (N + kKV_BK - 1) / kKV_BK;
    int m_per = 0;      // masked steps per query head: 0, 2, or 1 when a head has a single step
    int diag = 0;       // block-sparse: list position (from lo) of the diagonal entry
    if constexpr (CAUSAL) {
        if (sparse) {
            int64_t e = lo;
            while (e < hi && load_uniform(p.q_indices, e) < kblk) ++e;
            if (e < hi && load_uniform(p.q_indices, e) == kblk) {
                m_per = 2;
                diag = (int)(e - lo);
            }
        } else {
            m_per = min(2, per);
        }
    }
    const int n_mask = m_per * p.G;
    const int u_per = per - m_per;
    auto step_row = [&](int s, int& hq) -> int {   // first row of step s; N past the last step
        if (s >= n_all) {
            hq = hk * p.G;
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
        hq = hk * p.G + gq;
        if (!sparse) return (t0 + (masked_step ? j : m_per + j)) * kStep;
        int e = j >> 1;   // list entry (from lo): the diagonal one, or the others in order
        if (masked_step) e = diag;
        else if (m_per && e >= diag) ++e;
        const int qb = load_uniform(p.q_indices, lo + e);
        if (qb < 0 || qb >= nqb || (CAUSAL && qb < kblk)) return N;
        const int r0 = qb * kKV_BK + (j & 1) * kStep;
        return r0 < N ? r0 : N;
    };
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
                dsv[4 * tt + r] = pe * (a.p[tt][r] - d4[r]);
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
    float lse2 = 0.0f, dlt = 0.0f;
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
                for (int r = 0; r < 16; ++r) dsv[r] *= pacc[r] - dlt;
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
    float lse2 = 0.0f, dlt = 0.0f;
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
    if (nsteps > 0) {
        const int kt0 = step_key(0);
        if (kt0 >= 0) st.issue(kp, vp, p.ksn, p.vsn, kt0, N, lds0, wave_u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int cur = 0;
    for (int t = 0; t < nsteps; ++t) {
        // the other stage was last read in the previous step, which ended with a barrier
        if (t + 1 < nsteps) {
            const int ktn = step_key(t + 1);
            if (ktn >= 0) st.issue(kp, vp, p.ksn, p.vsn, ktn, N, lds0 + (cur ^ 1) * STAGEB, wave_u);
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
                for (int r = 0; r < 16; ++r) dsv[r] *= pacc[r] - dlt;
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
                           a.delta, L.H, Np, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const float c = a.scale * kLog2e;
    {
        KVParams p;
        p.q = static_cast<const uint16_t*>(a.q.p);
        p.k = static_cast<const uint16_t*>(a.k.p);
        p.v = static_cast<const uint16_t*>(a.v.p);
        p.dout = static_cast<const uint16_t*>(a.dout.p);
        p.lse = a.lse;
        p.delta = a.delta;
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
        const int64_t grid = (int64_t)L.B * L.Hkv * p.nkb;
        hipLaunchKernelGGL((dkdv16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads16), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
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
