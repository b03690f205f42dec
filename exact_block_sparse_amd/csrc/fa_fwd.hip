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
// * a workgroup is 4 wave64s; each wave owns QB blocks of 32 query rows (QB = 1: 128 rows
//   per workgroup, two workgroups per CU; QB = 2: 256 rows, one workgroup per CU, and every
//   K/V operand read from LDS feeds two MFMAs);
// * key/value tiles of 64 keys are staged through LDS, double-buffered, with raw buffer
//   loads whose hardware range check zero-fills rows past the sequence end; K and V are
//   both stored row-major; P.V reads its V^T operands with the transposing LDS read
//   ds_read_b64_tr_b16; row paddings keep reads and writes free of bank conflicts;
// * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so the 32
//   scores of a query over a 32-key block sit in one lane and its partner lane 32 away: the
//   row max needs one cross-half exchange (v_permlane32_swap), the row sum none until the end;
// * the running max is raised only when a tile's max exceeds it by more than 2^8 (in the
//   exp2 domain): probabilities then stay below 256 and the O rescale becomes rare. The
//   result is the same function; only the reference point of the exponentials moves;
// * O^T = V^T P^T accumulates in fp32 registers; P is rounded to bf16 only as an MFMA
//   operand; exp is computed as exp2 with scale*log2(e) folded into one FMA;
// * the LSE is written in natural log, O as bf16.
#include <cstdlib>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;            // keys per pipeline step
constexpr int kSparseBlock = 128;
constexpr float kRescaleSlack = 8.0f;   // log2 of the largest probability allowed before a rescale

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;             // K tile row stride in LDS (elements)
    static constexpr int VS = D + 32;            // V tile row stride in LDS (elements)
    static constexpr int KEL = kBK * KS;
    static constexpr int VEL = kBK * VS;
    static constexpr int BUF = KEL + VEL;        // elements per pipeline stage
    static constexpr int CR = D / 8;             // 16-byte chunks per row
    static constexpr int KCH = kBK * CR / kThreads;
    static constexpr int KSTEPS = D / 16;        // MFMA k-steps over the head dimension
    static constexpr int CB = D / 32;            // 32-wide head-dimension blocks of O
    static_assert((BUF * 2) % 16 == 0, "stage size must keep 16-byte alignment");
};

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, osb, osh, osn;
    int B, H, N;
    int nqb;          // query blocks (of the workgroup's row count) per head
    float c;          // scale * log2(e)
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    int64_t nnz;
};

// Per-thread staging of one K/V step: 16-byte row chunks of K and V.
template <int D>
struct Stage {
    using C = Cfg<D>;
    u32x4 k[C::KCH];
    u32x4 v[C::KCH];
    uint32_t koff[C::KCH];   // byte offsets (relative to the step's first row), fixed per thread
    uint32_t voff[C::KCH];
    int klds[C::KCH];        // LDS element offsets of the chunks
    int vlds[C::KCH];

    __device__ void init(int tid, int64_t ksn, int64_t vsn) {
#pragma unroll
        for (int j = 0; j < C::KCH; ++j) {
            const int id = tid + j * kThreads;
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
        for (int j = 0; j < C::KCH; ++j) k[j] = buf_load16(kr, koff[j], 0);
#pragma unroll
        for (int j = 0; j < C::KCH; ++j) v[j] = buf_load16(vr, voff[j], 0);
    }
    __device__ void store(uint16_t* buf) const {
#pragma unroll
        for (int j = 0; j < C::KCH; ++j) *reinterpret_cast<u32x4*>(buf + klds[j]) = k[j];
#pragma unroll
        for (int j = 0; j < C::KCH; ++j) *reinterpret_cast<u32x4*>(buf + vlds[j]) = v[j];
    }
};

// One 64-key step for one wave: scores for QB query blocks, masks (diagonal or tail tiles
// only), online softmax update, P.V. `masked[qb]` is uniform across the wave.
template <int D, int QB, bool CAUSAL>
__device__ __forceinline__ void tile_step(const uint16_t* buf, const bf16x8 (&qf)[QB][Cfg<D>::KSTEPS],
                                          f32x16 (&o)[QB][Cfg<D>::CB], float (&m_run)[QB], float (&l_part)[QB],
                                          const bool (&masked)[QB], int kt0, int qw0, int N, float c, bool cpos,
                                          int i, int hf) {
    using C = Cfg<D>;
    f32x16 s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        s[qb][0] = f32x16{};
        s[qb][1] = f32x16{};
    }
    // S^T = K Q^T. Row i of each 32-key block; the two blocks' chains alternate.
    const uint16_t* kr = buf + i * C::KS + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 32 * kb * C::KS + 16 * ks);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qf[qb][ks], s[qb][kb]);
        }
    }

    bf16x8 pb[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw0 + 32 * qb + i;
        // In masked tiles the scores are scaled here and masked keys (past the sequence end,
        // or after the query under causal masking) become -inf; the exponent below then uses
        // a unit multiplier. Elsewhere the scale is folded into the exponent's FMA.
        float ce = c;
        if (masked[qb]) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt0 + 32 * kb + acc_row(r, hf);
                    const bool ok = key < N && (!CAUSAL || key <= qrow);
                    s[qb][kb][r] = ok ? s[qb][kb][r] * c : kNegInf;
                }
            ce = 1.0f;
        }
        float mt;
        if (masked[qb] || cpos) {
            mt = fmaxf(s[qb][0][0], s[qb][1][0]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[qb][kb][r]);
            mt = pair_max(mt);
        } else {   // negative scale: the largest scaled score comes from the smallest raw one
            mt = fminf(s[qb][0][0], s[qb][1][0]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 1; r < 16; ++r) mt = fminf(mt, s[qb][kb][r]);
            mt = pair_min(mt);
        }
        mt *= ce;

        // Raise the running max only when the tile would push a probability above 2^8.
        const bool need = mt > m_run[qb] + kRescaleSlack;
        if (__any(need)) {
            const float m_new = need ? mt : m_run[qb];
            const float alpha = need ? fast_exp2(m_run[qb] - m_new) : 1.0f;
            m_run[qb] = m_new;
            l_part[qb] *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[qb][cb][r] *= alpha;
        }
        const float m_use = (m_run[qb] == kNegInf) ? 0.0f : m_run[qb];

        // The row sum is taken in fp32 over the unrounded probabilities (the LSE contract
        // needs it); P is rounded to bf16 only as the MFMA operand.
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[qb][kb][r], ce, -m_use));
                s[qb][kb][r] = p;
                psum += p;
            }
        l_part[qb] += psum;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
                pb[qb][kb][st] = pack8(s[qb][kb][8 * st + 0], s[qb][kb][8 * st + 1], s[qb][kb][8 * st + 2],
                                       s[qb][kb][8 * st + 3], s[qb][kb][8 * st + 4], s[qb][kb][8 * st + 5],
                                       s[qb][kb][8 * st + 6], s[qb][kb][8 * st + 7]);
    }

    // O^T += V^T P^T. B element e of k-step st in half hf is key 16*st + 8*(e/4) + 4*hf + e%4
    // of the 32-key block (the accumulator row order). The A operand (V^T: row = head-dim
    // column, k = key) comes from the row-major V tile through two transposing reads: lane j
    // of each 16-lane group addresses V[key0 + j/4][col0 + 4*(j%4)] and receives the 4 keys
    // of column col0 + j.
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
                u32x4 w;
                w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
                a[kb][st] = as_bf16x8(w);
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][cb] = mfma32(a[kb][st], pb[qb][kb][st], o[qb][cb]);
    }
}

template <int D, int QB, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads, QB == 1 ? 2 : 1) void fwd_kernel(Params p) {
    using C = Cfg<D>;
    constexpr int BQ = 128 * QB;
    static_assert(!SPARSE || QB == 1, "a sparse workgroup covers exactly one 128-row block");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qblk = logical % p.nqb;
    if (CAUSAL || SPARSE) qblk = p.nqb - 1 - qblk;   // longest query blocks first
    const int b = bh / p.H, hh = bh % p.H;
    const int N = p.N;

    const uint16_t* qp = p.q + b * p.qsb + hh * p.qsh;
    const uint16_t* kp = p.k + b * p.ksb + hh * p.ksh;
    const uint16_t* vp = p.v + b * p.vsb + hh * p.vsh;

    const int q0 = qblk * BQ;
    const int qw0 = q0 + 32 * QB * wave;
    const int qlast = min(q0 + BQ - 1, N - 1);

    bf16x8 qf[QB][C::KSTEPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw0 + 32 * qb + i;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            qf[qb][ks] = as_bf16x8(load16(qp + (int64_t)qrow * p.qsn + 16 * ks + 8 * hf, qrow < N));
    }

    // Pipeline steps. Dense: step t covers keys [64t, 64t+64). Sparse: step t covers half
    // (t & 1) of the listed key block kv_indices[t >> 1].
    int t_end;
    int t = 0;
    const int nkb = (N + kSparseBlock - 1) / kSparseBlock;
    if constexpr (SPARSE) {
        int64_t lo = p.kv_offsets[qblk], hi = p.kv_offsets[qblk + 1];
        lo = lo < 0 ? 0 : (lo > p.nnz ? p.nnz : lo);
        hi = hi < lo ? lo : (hi > p.nnz ? p.nnz : hi);
        t = (int)(2 * lo);
        t_end = (int)(2 * hi);
    } else {
        t_end = (N + kBK - 1) / kBK;
        if (CAUSAL) t_end = min(t_end, qlast / kBK + 1);
    }
    auto step_key = [&](int tt) -> int {   // first key of step tt, or -1 to skip it
        if constexpr (SPARSE) {
            const int kblk = p.kv_indices[tt >> 1];
            if (kblk < 0 || kblk >= nkb || (CAUSAL && kblk > qblk)) return -1;
            const int kt0 = kblk * kSparseBlock + (tt & 1) * kBK;
            if (kt0 >= N || (CAUSAL && kt0 > qlast)) return -1;
            return kt0;
        } else {
            return tt * kBK;
        }
    };

    int kt = -1;
    while (t < t_end && (kt = step_key(t)) < 0) ++t;

    f32x16 o[QB][C::CB];
    float m_run[QB], l_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) o[qb][cb] = f32x16{};
        m_run[qb] = kNegInf;
        l_part[qb] = 0.0f;
    }
    const float c = p.c;
    const bool cpos = c >= 0.0f;

    Stage<D> st;
    st.init(tid, p.ksn, p.vsn);
    if (t < t_end) {
        st.load(kp, vp, p.ksn, p.vsn, kt, N);
        st.store(smem);
    }
    // Settle every outstanding load (the Q fragments included) before the loop, so that no
    // wait on them is left inside it.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    int cur = 0;
    while (t < t_end) {
        int tn = t + 1, ktn = -1;
        while (tn < t_end && (ktn = step_key(tn)) < 0) ++tn;
        const bool has_next = tn < t_end;
        if (has_next) st.load(kp, vp, p.ksn, p.vsn, ktn, N);

        const uint16_t* buf = smem + cur * C::BUF;
        bool active = false;
        bool masked[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qs = qw0 + 32 * qb;
            active |= qs < N && (!CAUSAL || kt <= qs + 31);
            masked[qb] = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qs);
        }
        if (active) tile_step<D, QB, CAUSAL>(buf, qf, o, m_run, l_part, masked, kt, qw0, N, c, cpos, i, hf);
        if (has_next) st.store(smem + (cur ^ 1) * C::BUF);
        __syncthreads();
        cur ^= 1;
        t = tn;
        kt = ktn;
    }

    // Epilogue: O = O^T / l as bf16; LSE = (m + log2 l) * ln 2.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw0 + 32 * qb + i;
        const float l_tot = pair_sum(l_part[qb]);
        if (qrow < N) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            uint16_t* orow = p.o + b * p.osb + hh * p.osh + (int64_t)qrow * p.osn;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 val;
                    val[0] = (__bf16)(o[qb][cb][4 * j + 0] * inv);
                    val[1] = (__bf16)(o[qb][cb][4 * j + 1] * inv);
                    val[2] = (__bf16)(o[qb][cb][4 * j + 2] * inv);
                    val[3] = (__bf16)(o[qb][cb][4 * j + 3] * inv);
                    *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * j + 4 * hf) = val;
                }
            if (hf == 0)
                p.lse[(int64_t)bh * N + qrow] = l_tot > 0.0f ? (m_run[qb] + log2f(l_tot)) * kLn2 : kNegInf;
        }
    }
}

template <int D, int QB, bool CAUSAL, bool SPARSE>
hipError_t launch(Params p, hipStream_t stream) {
    p.nqb = (p.N + 128 * QB - 1) / (128 * QB);
    const int64_t grid = (int64_t)p.B * p.H * p.nqb;
    hipLaunchKernelGGL((fwd_kernel<D, QB, CAUSAL, SPARSE>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// Rows per wave for the dense kernels: 1 -> 32, 2 -> 64 (FA_FWD_QB overrides, for tuning).
int dense_qb() {
    static const int qb = [] {
        const char* e = std::getenv("FA_FWD_QB");
        return (e && e[0] == '2') ? 2 : 1;
    }();
    return qb;
}

template <int D>
hipError_t dispatch(const Params& p, bool causal, bool sparse, hipStream_t stream) {
    if (sparse) return causal ? launch<D, 1, true, true>(p, stream) : launch<D, 1, false, true>(p, stream);
    if (dense_qb() == 2)
        return causal ? launch<D, 2, true, false>(p, stream) : launch<D, 2, false, false>(p, stream);
    return causal ? launch<D, 1, true, false>(p, stream) : launch<D, 1, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const uint16_t*>(a.q.p);
    p.k = static_cast<const uint16_t*>(a.k.p);
    p.v = static_cast<const uint16_t*>(a.v.p);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.qsb = a.q.sb; p.qsh = a.q.sh; p.qsn = a.q.sn;
    p.ksb = a.k.sb; p.ksh = a.k.sh; p.ksn = a.k.sn;
    p.vsb = a.v.sb; p.vsh = a.v.sh; p.vsn = a.v.sn;
    p.osb = a.osb; p.osh = a.osh; p.osn = a.osn;
    p.B = a.B; p.H = a.H; p.N = a.N;
    p.nqb = 0;
    p.c = a.scale * kLog2e;
    p.kv_offsets = a.kv_offsets;
    p.kv_indices = a.kv_indices;
    p.nnz = a.nnz;
    const bool sparse = a.kv_offsets != nullptr;
    if (a.d == 64) return dispatch<64>(p, a.causal != 0, sparse, stream);
    return dispatch<128>(p, a.causal != 0, sparse, stream);
}

}  // namespace fa
