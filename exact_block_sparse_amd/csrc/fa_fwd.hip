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
// * a workgroup is 4 wave64s and owns 128 query rows; each wave owns 32 rows;
// * key/value tiles of 64 keys are staged through LDS, double-buffered: K row-major,
//   V transposed on the way in so that P.V reads 16-byte operands;
// * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so the
//   32 scores of a query over a 32-key block sit in one lane and its partner lane 32
//   away: row max and row sum need one cross-half exchange (v_permlane32_swap);
// * O^T = V^T P^T accumulates in fp32 registers; P is rounded to bf16 only as an MFMA
//   operand; exp is computed as exp2 with scale*log2(e) folded into one FMA;
// * the LSE is written in natural log, O as bf16.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBQ = 128;   // query rows per workgroup
constexpr int kBK = 64;    // keys per pipeline step
constexpr int kSparseBlock = 128;

template <int D>
struct Cfg {
    static constexpr int KS = D + 8;             // K tile row stride in LDS (elements)
    static constexpr int VS = kBK + 8;           // V^T tile row stride in LDS (elements)
    static constexpr int KEL = kBK * KS;
    static constexpr int VEL = D * VS;
    static constexpr int BUF = KEL + VEL;        // elements per pipeline stage
    static constexpr int CR = D / 8;             // 16-byte chunks per row
    static constexpr int KCH = kBK * CR / kThreads;
    static constexpr int VGROUPS = (kBK / 4) * CR;
    static constexpr int KSTEPS = D / 16;        // MFMA k-steps over the head dimension
    static constexpr int CB = D / 32;            // 32-wide head-dimension blocks of O
};

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, osb, osh, osn;
    int B, H, N;
    int nqb;          // query blocks of kBQ rows per head
    float c;          // scale * log2(e)
    const int32_t* kv_offsets;
    const int32_t* kv_indices;
    int64_t nnz;
};

template <int D>
struct Stage {
    u32x4 k[Cfg<D>::KCH];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_stage(Stage<D>& st, const uint16_t* kb, const uint16_t* vb,
                                           int64_t ksn, int64_t vsn, int kt0, int N, int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
        const int id = tid + j * kThreads;
        const int row = id / C::CR, ch = id % C::CR;
        const int key = kt0 + row;
        st.k[j] = load16(kb + (int64_t)key * ksn + ch * 8, key < N);
    }
    if (tid < C::VGROUPS) {
        const int cg = tid % C::CR, kg = tid / C::CR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kt0 + 4 * kg + r;
            st.v[r] = load16(vb + (int64_t)key * vsn + cg * 8, key < N);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_stage(const Stage<D>& st, uint16_t* buf, int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
        const int id = tid + j * kThreads;
        const int row = id / C::CR, ch = id % C::CR;
        *reinterpret_cast<u32x4*>(buf + row * C::KS + ch * 8) = st.k[j];
    }
    if (tid < C::VGROUPS) {
        const int cg = tid % C::CR, kg = tid / C::CR;
        store_transposed_4x8(buf + C::KEL + (8 * cg) * C::VS + 4 * kg, C::VS, st.v[0], st.v[1], st.v[2],
                             st.v[3]);
    }
}

// One 64-key step for one wave: scores, mask (diagonal or tail tiles only), online
// softmax update and P.V. `masked` is uniform across the wave.
template <int D, bool CAUSAL>
__device__ __forceinline__ void tile_step(const uint16_t* buf, const bf16x8* qf, f32x16* o, float& m_run,
                                          float& l_part, int kt0, int qrow, int N, float c, bool cpos,
                                          bool masked, int i, int hf) {
    using C = Cfg<D>;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        f32x16 acc = {};
        const uint16_t* kr = buf + (32 * kb + swz(i)) * C::KS + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
            acc = mfma32(a, qf[ks], acc);
        }
        s[kb] = acc;
    }

    // In masked tiles the scores are scaled here and masked keys (past the sequence end,
    // or after the query under causal masking) become -inf; the exponent below then uses
    // a unit multiplier. Elsewhere the scale is folded into the exponent's FMA.
    float ce = c;
    if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt0 + 32 * kb + swz(acc_row(r, hf));
                const bool ok = key < N && (!CAUSAL || key <= qrow);
                s[kb][r] = ok ? s[kb][r] * c : kNegInf;
            }
        ce = 1.0f;
    }
    float mt = s[0][0];
    if (masked || cpos) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
        mt = pair_max(mt);
    } else {   // negative scale: the largest scaled score comes from the smallest raw one
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fminf(mt, s[kb][r]);
        mt = pair_min(mt);
    }
    mt *= ce;

    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[kb][r], ce, -m_use));
            s[kb][r] = p;
            psum += p;
        }
    }
    l_part = alpha * l_part + psum;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
            pb[kb][st] = pack8(s[kb][8 * st + 0], s[kb][8 * st + 1], s[kb][8 * st + 2], s[kb][8 * st + 3],
                               s[kb][8 * st + 4], s[kb][8 * st + 5], s[kb][8 * st + 6], s[kb][8 * st + 7]);

    const uint16_t* vt = buf + C::KEL;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
        const uint16_t* vr = vt + (32 * cb + i) * C::VS + 8 * hf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vr + 32 * kb + 16 * st);
                o[cb] = mfma32(a, pb[kb][st], o[cb]);
            }
    }
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(Params p) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, i = lane & 31;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical % p.nqb;
    if (CAUSAL || SPARSE) qb = p.nqb - 1 - qb;   // longest query blocks first
    const int b = bh / p.H, hh = bh % p.H;
    const int N = p.N;

    const uint16_t* qp = p.q + b * p.qsb + hh * p.qsh;
    const uint16_t* kp = p.k + b * p.ksb + hh * p.ksh;
    const uint16_t* vp = p.v + b * p.vsb + hh * p.vsh;

    const int q0 = qb * kBQ;
    const int qw0 = q0 + 32 * wave;
    const int qrow = qw0 + i;
    const int qlast = min(q0 + kBQ - 1, N - 1);

    bf16x8 qf[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
        qf[ks] = as_bf16x8(load16(qp + (int64_t)qrow * p.qsn + 16 * ks + 8 * hf, qrow < N));

    // Pipeline steps. Dense: step t covers keys [64t, 64t+64). Sparse: step t covers half
    // (t & 1) of the listed key block kv_indices[t >> 1].
    int t_end;
    int t = 0;
    const int nkb = (N + kSparseBlock - 1) / kSparseBlock;
    if constexpr (SPARSE) {
        int64_t lo = p.kv_offsets[qb], hi = p.kv_offsets[qb + 1];
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
            if (kblk < 0 || kblk >= nkb || (CAUSAL && kblk > qb)) return -1;
            const int kt0 = kblk * kSparseBlock + (tt & 1) * kBK;
            if (kt0 >= N || (CAUSAL && kt0 > qlast)) return -1;
            return kt0;
        } else {
            return tt * kBK;
        }
    };

    int kt = -1;
    while (t < t_end && (kt = step_key(t)) < 0) ++t;

    f32x16 o[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) o[cb] = f32x16{};
    float m_run = kNegInf, l_part = 0.0f;
    const float c = p.c;
    const bool cpos = c >= 0.0f;

    Stage<D> st;
    if (t < t_end) {
        load_stage<D>(st, kp, vp, p.ksn, p.vsn, kt, N, tid);
        store_stage<D>(st, smem, tid);
    }
    __syncthreads();

    int cur = 0;
    while (t < t_end) {
        int tn = t + 1, ktn = -1;
        while (tn < t_end && (ktn = step_key(tn)) < 0) ++tn;
        const bool has_next = tn < t_end;
        if (has_next) load_stage<D>(st, kp, vp, p.ksn, p.vsn, ktn, N, tid);

        const uint16_t* buf = smem + cur * C::BUF;
        const bool active = qw0 < N && (!CAUSAL || kt <= qw0 + 31);
        if (active) {
            const bool masked = (kt + kBK > N) || (CAUSAL && kt + kBK - 1 > qw0);
            tile_step<D, CAUSAL>(buf, qf, o, m_run, l_part, kt, qrow, N, c, cpos, masked, i, hf);
        }
        if (has_next) store_stage<D>(st, smem + (cur ^ 1) * C::BUF, tid);
        __syncthreads();
        cur ^= 1;
        t = tn;
        kt = ktn;
    }

    // Epilogue: O = O^T / l as bf16; LSE = (m + log2 l) * ln 2.
    const float l_tot = pair_sum(l_part);
    if (qrow < N) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = p.o + b * p.osb + hh * p.osh + (int64_t)qrow * p.osn;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 val;
                val[0] = (__bf16)(o[cb][4 * j + 0] * inv);
                val[1] = (__bf16)(o[cb][4 * j + 1] * inv);
                val[2] = (__bf16)(o[cb][4 * j + 2] * inv);
                val[3] = (__bf16)(o[cb][4 * j + 3] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * j + 4 * hf) = val;
            }
        if (hf == 0)
            p.lse[(int64_t)bh * N + qrow] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch(const Params& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.B * p.H * p.nqb;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, SPARSE>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch(const Params& p, bool causal, bool sparse, hipStream_t stream) {
    if (sparse) return causal ? launch<D, true, true>(p, stream) : launch<D, false, true>(p, stream);
    return causal ? launch<D, true, false>(p, stream) : launch<D, false, false>(p, stream);
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
    p.nqb = (a.N + kBQ - 1) / kBQ;
    p.c = a.scale * kLog2e;
    p.kv_offsets = a.kv_offsets;
    p.kv_indices = a.kv_indices;
    p.nnz = a.nnz;
    const bool sparse = a.kv_offsets != nullptr;
    if (a.d == 64) return dispatch<64>(p, a.causal != 0, sparse, stream);
    return dispatch<128>(p, a.causal != 0, sparse, stream);
}

}  // namespace fa
