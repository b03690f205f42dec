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
// 2. dkdv_kernel: a workgroup owns 128 keys (32 per wave, one key per lane column) and
//    walks the query tiles that can see them. K and V of the wave's keys stay in
//    registers; Q and dO tiles are staged in LDS row-major (MFMA A operands of S and dP)
//    and transposed (A operands of dK^T and dV^T). dK^T, dV^T accumulate in fp32.
// 3. dq_kernel: a workgroup owns 128 query rows, as in the forward, and walks the key
//    tiles: S^T = K Q^T and dP^T = V dO^T with Q and dO in registers, then
//    dQ^T += K^T dS^T with K staged transposed in LDS.
// S and dP are thus computed twice (7 matrix products instead of 5) in exchange for no
// atomics and bitwise-reproducible results.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// Rows [r0, r0 + R) of a row-major [N, D] bf16 matrix (row stride sn elements), held in
// registers as 4-row x 8-column blocks and written to LDS row-major (stride D + 8)
// and/or transposed (stride R + 8). Rows at or past N read as zeros.
template <int D, int R>
struct TileStage {
    static constexpr int CR = D / 8;
    static constexpr int NBLK = (R / 4) * CR;
    static constexpr int PER = (NBLK + kThreads - 1) / kThreads;
    static constexpr int RS = D + 8;   // row-major LDS stride
    static constexpr int TS = R + 8;   // transposed LDS stride
    u32x4 r[PER][4];

    __device__ __forceinline__ void load(const uint16_t* base, int64_t sn, int r0, int N, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int blk = tid + p * kThreads;
            const int cg = blk % CR, rg = blk / CR;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = r0 + 4 * rg + j;
                r[p][j] = load16(base + (int64_t)row * sn + 8 * cg, blk < NBLK && row < N);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* rowmajor, uint16_t* transposed, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int blk = tid + p * kThreads;
            if (blk >= NBLK) continue;
            const int cg = blk % CR, rg = blk / CR;
            if (rowmajor) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4*>(rowmajor + (4 * rg + j) * RS + 8 * cg) = r[p][j];
            }
            if (transposed)
                store_transposed_4x8(transposed + (8 * cg) * TS + 4 * rg, TS, r[p][0], r[p][1], r[p][2], r[p][3]);
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
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
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

// ----------------------------------------------------------------------------- dK, dV
constexpr int kKV_BK = 128;   // keys per workgroup (32 per wave)
constexpr int kKV_BQ = 64;    // query rows per pipeline step

struct KVParams {
    const uint16_t *q, *k, *v, *dout;
    const float* lse;
    const float* delta;
    uint16_t *dk, *dv;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, dsb, dsh, dsn;
    int64_t dksb, dksh, dksn, dvsb, dvsh, dvsn;
    int B, H, N, nkb;
    float c;       // scale * log2(e)
    float scale;
};

template <int D>
struct KVCfg {
    using T = TileStage<D, kKV_BQ>;
    static constexpr int RS = T::RS, TS = T::TS;
    static constexpr int ROWEL = kKV_BQ * RS;          // a row-major tile
    static constexpr int TREL = D * TS;                // a transposed tile
    // stage layout: Q | Q^T | dO | dO^T | lse2[64] | delta[64] (floats at the end)
    static constexpr int STAGE_U16 = 2 * ROWEL + 2 * TREL + 2 * kKV_BQ * 2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(KVParams p) {
    using C = KVCfg<D>;
    using T = typename C::T;
    constexpr int KSTEPS = D / 16, CB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE_U16];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nkb, kblk = logical % p.nkb;   // ascending: longest first under causal
    const int b = bh / p.H, hh = bh % p.H;
    const int N = p.N;

    const uint16_t* qp = p.q + b * p.qsb + hh * p.qsh;
    const uint16_t* dp = p.dout + b * p.dsb + hh * p.dsh;
    const float* lsep = p.lse + (int64_t)bh * N;
    const float* delp = p.delta + (int64_t)bh * N;

    const int k0 = kblk * kKV_BK;
    const int kw0 = k0 + 32 * wave;
    const int key = kw0 + i;

    // K and V rows of this lane's key as B operands (column = key, k-group = half).
    bf16x8 kf[KSTEPS], vf[KSTEPS];
    {
        const uint16_t* kr = p.k + b * p.ksb + hh * p.ksh + (int64_t)key * p.ksn + 8 * hf;
        const uint16_t* vr = p.v + b * p.vsb + hh * p.vsh + (int64_t)key * p.vsn + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            kf[ks] = as_bf16x8(load16(kr + 16 * ks, key < N));
            vf[ks] = as_bf16x8(load16(vr + 16 * ks, key < N));
        }
    }

    f32x16 dk[CB], dv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        dk[cb] = f32x16{};
        dv[cb] = f32x16{};
    }

    const int nsteps = (N + kKV_BQ - 1) / kKV_BQ;
    int t = CAUSAL ? k0 / kKV_BQ : 0;
    const float c = p.c;

    T sq, sd;
    float st_lse = 0.0f, st_del = 0.0f;
    auto load_step = [&](int tt) {
        const int r0 = tt * kKV_BQ;
        sq.load(qp, p.qsn, r0, N, tid);
        sd.load(dp, p.dsn, r0, N, tid);
        if (tid < kKV_BQ) {
            const int row = r0 + tid;
            // Rows past N get LSE = +inf, so their recomputed probabilities are exactly 0.
            float l = row < N ? lsep[row] : __builtin_inff();
            if (l == -__builtin_inff()) l = __builtin_inff();   // a row that saw no key
            st_lse = l * kLog2e;
        } else if (tid < 2 * kKV_BQ) {
            const int row = r0 + tid - kKV_BQ;
            st_del = row < N ? delp[row] : 0.0f;
        }
    };
    auto store_step = [&](uint16_t* s) {
        sq.store(s, s + C::ROWEL, tid);
        sd.store(s + C::ROWEL + C::TREL, s + 2 * C::ROWEL + C::TREL, tid);
        float* f = reinterpret_cast<float*>(s + 2 * C::ROWEL + 2 * C::TREL);
        if (tid < kKV_BQ) f[tid] = st_lse;
        else if (tid < 2 * kKV_BQ) f[tid] = st_del;
    };

    if (t < nsteps) {
        load_step(t);
        store_step(smem);
    }
    __syncthreads();
    int cur = 0;
    for (; t < nsteps; ++t) {
        const bool has_next = t + 1 < nsteps;
        if (has_next) load_step(t + 1);

        const uint16_t* s = smem + cur * C::STAGE_U16;
        const uint16_t* sQ = s;
        const uint16_t* sQT = s + C::ROWEL;
        const uint16_t* sD = s + C::ROWEL + C::TREL;
        const uint16_t* sDT = s + 2 * C::ROWEL + C::TREL;
        const float* sL = reinterpret_cast<const float*>(s + 2 * C::ROWEL + 2 * C::TREL);
        const float* sDel = sL + kKV_BQ;
        const int qt0 = t * kKV_BQ;
        const bool active = key - i < N && (!CAUSAL || qt0 + kKV_BQ - 1 >= kw0);
        if (active) {
#pragma unroll
            for (int qb = 0; qb < kKV_BQ / 32; ++qb) {
                if (CAUSAL && qt0 + 32 * qb + 31 < kw0) continue;   // every query before every key
                // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys. A-operand
                // row i holds query swz(i), so the accumulator hands out 8 consecutive queries
                // per lane and k-step below.
                f32x16 sacc = {}, pacc = {};
                const uint16_t* qr = sQ + (32 * qb + swz(i)) * C::RS + 8 * hf;
                const uint16_t* dr = sD + (32 * qb + swz(i)) * C::RS + 8 * hf;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    sacc = mfma32(*reinterpret_cast<const bf16x8*>(qr + 16 * ks), kf[ks], sacc);
                    pacc = mfma32(*reinterpret_cast<const bf16x8*>(dr + 16 * ks), vf[ks], pacc);
                }
                const bool masked = CAUSAL && qt0 + 32 * qb < kw0 + 31;
                bf16x8 pb[2], db[2];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int q8 = 32 * qb + 16 * st + 8 * hf;   // first of this lane's 8 queries
                    const f32x4 l0 = *reinterpret_cast<const f32x4*>(sL + q8);
                    const f32x4 l1 = *reinterpret_cast<const f32x4*>(sL + q8 + 4);
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(sDel + q8);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(sDel + q8 + 4);
                    float pv[8], dsv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float lq = e < 4 ? l0[e] : l1[e - 4];
                        const float dq = e < 4 ? d0[e] : d1[e - 4];
                        float pe = fast_exp2(fmaf(sacc[8 * st + e], c, -lq));
                        if (masked && key > qt0 + q8 + e) pe = 0.0f;
                        pv[e] = pe;
                        dsv[e] = pe * (pacc[8 * st + e] - dq);
                    }
                    pb[st] = pack8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
                    db[st] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
                }
                // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries.
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const uint16_t* dtr = sDT + (32 * cb + i) * C::TS + 32 * qb + 8 * hf;
                    const uint16_t* qtr = sQT + (32 * cb + i) * C::TS + 32 * qb + 8 * hf;
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        dv[cb] = mfma32(*reinterpret_cast<const bf16x8*>(dtr + 16 * st), pb[st], dv[cb]);
                        dk[cb] = mfma32(*reinterpret_cast<const bf16x8*>(qtr + 16 * st), db[st], dk[cb]);
                    }
                }
            }
        }
        if (has_next) store_step(smem + (cur ^ 1) * C::STAGE_U16);
        __syncthreads();
        cur ^= 1;
    }

    if (key < N) {
        uint16_t* dkr = p.dk + b * p.dksb + hh * p.dksh + (int64_t)key * p.dksn;
        uint16_t* dvr = p.dv + b * p.dvsb + hh * p.dvsh + (int64_t)key * p.dvsn;
        const float sc = p.scale;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 a, v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = (__bf16)(dk[cb][4 * j + e] * sc);
                    v[e] = (__bf16)(dv[cb][4 * j + e]);
                }
                *reinterpret_cast<bf16x4*>(dkr + 32 * cb + 8 * j + 4 * hf) = a;
                *reinterpret_cast<bf16x4*>(dvr + 32 * cb + 8 * j + 4 * hf) = v;
            }
    }
}

// ----------------------------------------------------------------------------- dQ
constexpr int kQ_BQ = 128;   // query rows per workgroup (32 per wave)
constexpr int kQ_BK = 64;    // keys per pipeline step

struct QParams {
    const uint16_t *q, *k, *v, *dout;
    const float* lse;
    const float* delta;
    uint16_t* dq;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, dsb, dsh, dsn, dqsb, dqsh, dqsn;
    int B, H, N, nqb;
    float c;
    float scale;
};

template <int D>
struct QCfg {
    using T = TileStage<D, kQ_BK>;
    static constexpr int RS = T::RS, TS = T::TS;
    static constexpr int ROWEL = kQ_BK * RS;
    static constexpr int TREL = D * TS;
    // stage layout: K | K^T | V
    static constexpr int STAGE_U16 = 2 * ROWEL + TREL;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(QParams p) {
    using C = QCfg<D>;
    using T = typename C::T;
    constexpr int KSTEPS = D / 16, CB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE_U16];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical % p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int b = bh / p.H, hh = bh % p.H;
    const int N = p.N;

    const uint16_t* kp = p.k + b * p.ksb + hh * p.ksh;
    const uint16_t* vp = p.v + b * p.vsb + hh * p.vsh;
    const int q0 = qb * kQ_BQ;
    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kQ_BQ - 1, N - 1);

    bf16x8 qf[KSTEPS], df[KSTEPS];
    {
        const uint16_t* qr = p.q + b * p.qsb + hh * p.qsh + (int64_t)qrow * p.qsn + 8 * hf;
        const uint16_t* dr = p.dout + b * p.dsb + hh * p.dsh + (int64_t)qrow * p.dsn + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qf[ks] = as_bf16x8(load16(qr + 16 * ks, qrow < N));
            df[ks] = as_bf16x8(load16(dr + 16 * ks, qrow < N));
        }
    }
    float lse2 = 0.0f, dlt = 0.0f;
    if (qrow < N) {
        float l = p.lse[(int64_t)bh * N + qrow];
        if (l == -__builtin_inff()) l = __builtin_inff();
        lse2 = l * kLog2e;
        dlt = p.delta[(int64_t)bh * N + qrow];
    }

    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    int nsteps = (N + kQ_BK - 1) / kQ_BK;
    if (CAUSAL) nsteps = min(nsteps, qlast / kQ_BK + 1);
    const float c = p.c;

    T sk, sv;
    if (nsteps > 0) {
        sk.load(kp, p.ksn, 0, N, tid);
        sv.load(vp, p.vsn, 0, N, tid);
        sk.store(smem, smem + C::ROWEL, tid);
        sv.store(smem + C::ROWEL + C::TREL, nullptr, tid);
    }
    __syncthreads();
    int cur = 0;
    for (int t = 0; t < nsteps; ++t) {
        const bool has_next = t + 1 < nsteps;
        if (has_next) {
            sk.load(kp, p.ksn, (t + 1) * kQ_BK, N, tid);
            sv.load(vp, p.vsn, (t + 1) * kQ_BK, N, tid);
        }
        const uint16_t* s = smem + cur * C::STAGE_U16;
        const uint16_t* sK = s;
        const uint16_t* sKT = s + C::ROWEL;
        const uint16_t* sV = s + C::ROWEL + C::TREL;
        const int kt = t * kQ_BK;
        const bool active = qw0 < N && (!CAUSAL || kt <= qw0 + 31);
        if (active) {
            const bool masked = (kt + kQ_BK > N) || (CAUSAL && kt + kQ_BK - 1 > qw0);
            bf16x8 db[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sacc = {}, pacc = {};
                const uint16_t* kr = sK + (32 * kb + swz(i)) * C::RS + 8 * hf;
                const uint16_t* vr = sV + (32 * kb + swz(i)) * C::RS + 8 * hf;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    sacc = mfma32(*reinterpret_cast<const bf16x8*>(kr + 16 * ks), qf[ks], sacc);
                    pacc = mfma32(*reinterpret_cast<const bf16x8*>(vr + 16 * ks), df[ks], pacc);
                }
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    float dsv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float pe = fast_exp2(fmaf(sacc[8 * st + e], c, -lse2));
                        if (masked) {
                            const int kk = kt + 32 * kb + 16 * st + 8 * hf + e;
                            if (kk >= N || (CAUSAL && kk > qrow)) pe = 0.0f;
                        }
                        dsv[e] = pe * (pacc[8 * st + e] - dlt);
                    }
                    db[kb][st] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
                }
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint16_t* ktr = sKT + (32 * cb + i) * C::TS + 8 * hf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        dq[cb] = mfma32(*reinterpret_cast<const bf16x8*>(ktr + 32 * kb + 16 * st), db[kb][st], dq[cb]);
            }
        }
        if (has_next) {
            uint16_t* n = smem + (cur ^ 1) * C::STAGE_U16;
            sk.store(n, n + C::ROWEL, tid);
            sv.store(n + C::ROWEL + C::TREL, nullptr, tid);
        }
        __syncthreads();
        cur ^= 1;
    }

    if (qrow < N) {
        uint16_t* dqr = p.dq + b * p.dqsb + hh * p.dqsh + (int64_t)qrow * p.dqsn;
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
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    constexpr int RPB = kThreads / (D / 8);
    {
        const int64_t grid = (rows + RPB - 1) / RPB;
        hipLaunchKernelGGL((pre_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(a.o.p), a.o.sb, a.o.sh, a.o.sn,
                           static_cast<const uint16_t*>(a.dout.p), a.dout.sb, a.dout.sh, a.dout.sn, a.delta, a.H,
                           a.N, rows);
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
        p.B = a.B; p.H = a.H; p.N = a.N;
        p.nkb = (a.N + kKV_BK - 1) / kKV_BK;
        p.c = c;
        p.scale = a.scale;
        const int64_t grid = (int64_t)a.B * a.H * p.nkb;
        hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
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
        p.B = a.B; p.H = a.H; p.N = a.N;
        p.nqb = (a.N + kQ_BQ - 1) / kQ_BQ;
        p.c = c;
        p.scale = a.scale;
        const int64_t grid = (int64_t)a.B * a.H * p.nqb;
        hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return a.causal ? launch_all<64, true>(a, stream) : launch_all<64, false>(a, stream);
    return a.causal ? launch_all<128, true>(a, stream) : launch_all<128, false>(a, stream);
}

}  // namespace fa
