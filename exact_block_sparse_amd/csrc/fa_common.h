// Device-side building blocks shared by the forward and backward kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16), one wave64.
// Operand layout used throughout: lane l supplies row (A) / column (B) l % 32 and the
// 8 k-values of k-group l / 32; the accumulator element r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in element r by a lane of half `hf` (= lane / 32).
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Combine a value with the one held by the lane 32 positions away (the other half of the
// wave), with a symmetric op: the two halves hold complementary keys of the same query.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Element of a table that stays unchanged while the kernel runs (the block lists), read
// with a wave-uniform index. Through the constant address space the read can be a scalar
// load, which does not make the wave wait for its vector loads still in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* table, int64_t idx) {
    return ((const __attribute__((address_space(4))) int32_t*)table)[idx];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// 16-byte global load that yields zeros when `ok` is false (no access is made then).
__device__ __forceinline__ u32x4 load16(const uint16_t* p, bool ok) {
    u32x4 z = {0u, 0u, 0u, 0u};
    return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// Pack eight fp32 values into an MFMA bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// Workgroups are handed to the 8 XCDs round-robin. Map the hardware id so that the
// logical ids an XCD receives are consecutive: neighbouring query blocks of one head then
// run on the same XCD and share its L2 for the K/V stream.
__device__ __forceinline__ int xcd_remap(int w, int G) {
    constexpr int X = 8;
    const int x = w % X, slot = w / X;
    const int per = G / X, rem = G % X;
    return x * per + (x < rem ? x : rem) + slot;
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes return 0
// without touching memory (the hardware range check), which gives zero-filled tails.
// Word 3 is the gfx9-family raw-buffer format (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// Bytes of rows [r0, n) of a matrix with row stride `sn` elements and `d` columns of `es`
// bytes (2: bf16, 1: fp8), capped to `rows` rows; the cap keeps the value well inside 32 bits.
__device__ __forceinline__ uint32_t rows_bytes(int r0, int n, int64_t sn, int d, int rows, int es = 2) {
    int last = n - 1 - r0;
    if (last >= rows) last = rows - 1;
    if (last < 0) return 0u;
    return (uint32_t)(((int64_t)last * sn + d) * es);
}

// 16-byte global load from a byte address that yields zeros when `ok` is false.
__device__ __forceinline__ u32x4 load16b(const uint8_t* p, bool ok) {
    u32x4 z = {0u, 0u, 0u, 0u};
    return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// fp8 (OCP e4m3) operands: 32 values per lane. D(32x32 fp32) += A(32x64) * B(64x32) with
// v_mfma_f32_32x32x64_f8f6f4, twice the bf16 rate. Operand layout (measured): lane l supplies
// row (A) / column (B) l % 32 and the 32 consecutive k-values 32*(l/32) .. 32*(l/32)+31; the
// accumulator layout is the one of mfma32.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ i32x8 join8(const u32x4& lo, const u32x4& hi) {
    i32x8 r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}
// Sixteen fp8 (e4m3) values to sixteen bf16, exactly (every e4m3 value is a bf16 value):
// word w of `x` holds values 4w .. 4w+3; the result's word j holds values 2j, 2j+1.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& x, u32x4& lo, u32x4& hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t out[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true);
        out[2 * w] = __builtin_bit_cast(uint32_t, a);
        out[2 * w + 1] = __builtin_bit_cast(uint32_t, b);
    }
    lo[0] = out[0]; lo[1] = out[1]; lo[2] = out[2]; lo[3] = out[3];
    hi[0] = out[4]; hi[1] = out[5]; hi[2] = out[6]; hi[3] = out[7];
}

// Where one sequence lives. Fixed length (cu == nullptr): sequence b is the b-th [N, d]
// slab of each tensor. Packed variable length: rows cu[b] .. cu[b+1]-1 of the packed
// tensors, clamped to [0, total) and to at most N rows, so that no access leaves the
// tensors whatever the offsets hold.
struct SeqSpan {
    int64_t tok0;   // first packed row (packed mode)
    int len;        // rows of this sequence
    bool packed;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int64_t total, int b, int N) {
    SeqSpan s{0, N, false};
    if (cu) {
        int64_t lo = cu[b], hi = cu[b + 1];
        lo = lo < 0 ? 0 : (lo > total ? total : lo);
        hi = hi < lo ? lo : (hi > total ? total : hi);
        const int64_t n = hi - lo;
        s.tok0 = lo;
        s.len = (int)(n < N ? n : N);
        s.packed = true;
    }
    return s;
}
// Element offset of row 0 of sequence b, head h, in a tensor with strides (sb, sh, sn).
__device__ __forceinline__ int64_t seq_off(const SeqSpan& s, int b, int h, int64_t sb, int64_t sh, int64_t sn) {
    return (s.packed ? s.tok0 * sn : (int64_t)b * sb) + (int64_t)h * sh;
}
// Offset of the first per-row statistic (LSE, D) of sequence b, head h: [B, H, N] for fixed
// length, [H, total] when packed.
__device__ __forceinline__ int64_t seq_stat_off(const SeqSpan& s, int b, int h, int H, int N, int64_t total) {
    return s.packed ? (int64_t)h * total + s.tok0 : ((int64_t)b * H + h) * N;
}

// ds_read_b64_tr_b16 (gfx950): each lane supplies the LDS address of 4 consecutive bf16.
// Within every group of 16 lanes, lane i receives element (i % 4) of the chunks addressed
// by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4. So if lane j of a group addresses
// M[k0 + j/4][c0 + 4*(j%4)] of a row-major matrix, lane i receives M[k0 .. k0+3][c0 + i]:
// a column, i.e. the transposed operand, without a transposing store.
__device__ __forceinline__ u32x2 lds_read_tr4(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// A operand of a 32x32x16 MFMA holding M^T (row = column of M, k = 8 rows of M), read from
// a row-major bf16 tile M with two transposing reads. `lane_base` is the per-lane address
//   M + (4*hf + j/4) * stride + 16*g + 4*(j%4)      (j = lane % 16, g = (lane / 16) % 2),
// and `off` = r0 * stride + c0 selects rows r0 .. r0 + 15 and columns c0 .. c0 + 31: element
// e of the lane with row c (= lane % 32) is M[r0 + 8*(e/4) + 4*hf + e%4][c0 + c], the order
// in which a 32x32 accumulator hands its rows to a B operand.
__device__ __forceinline__ bf16x8 read_tr_operand(const uint16_t* lane_base, int off, int stride) {
    const u32x2 lo = lds_read_tr4(lane_base + off);
    const u32x2 hi = lds_read_tr4(lane_base + off + 8 * stride);
    u32x4 x;
    x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
    return as_bf16x8(x);
}
// A operand of a 16x16x32 MFMA holding M^T (row = column of M, k = 8 rows of M), read from
// a row-major bf16 tile (row stride `stride`) with two transposing reads; `p` is the lane's
// address for rows 4*g .. 4*g+3 (g = lane / 16). Element e is row 4*g + e (e < 4) or
// 16 + 4*g + e - 4 of M.
__device__ __forceinline__ bf16x8 read_tr_operand16(const uint16_t* p, int stride) {
    const u32x2 lo = lds_read_tr4(p);
    const u32x2 hi = lds_read_tr4(p + 16 * stride);
    u32x4 x;
    x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
    return as_bf16x8(x);
}
__device__ __forceinline__ const uint16_t* tr_lane_base(const uint16_t* tile, int stride, int lane) {
    const int hf = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
    return tile + (4 * hf + (j >> 2)) * stride + 16 * g + 4 * (j & 3);
}


// ----------------------------------------------------------------------------- loads into LDS
// bf16 tiles of 64 rows at head dimension 128 loaded from memory straight into LDS
// (`buffer_load_dwordx4 ... lds`: lane L's 16 bytes land at M0 + 16 * L, so one wave
// instruction fills 1 KB, four whole 256-byte rows). The tiles are unpadded; bank conflicts
// are avoided by keeping 16-byte chunk c of row r at chunk slot c ^ swz(r), and each lane
// loads the chunk that belongs at its slot, so every instruction still reads whole rows.
// Swizzles (all depend on r & 15 only, so 16-row offsets move no chunk):
// * kSwzRow  = r & 15: 16-byte reads of one chunk by 16 consecutive rows;
// * kSwzTr   = 4 (r & 3): transposing reads of four consecutive rows x four chunks;
// * kSwzBoth = 4 (r & 3) | ((r >> 2) & 3): both patterns (a bijection on 16 rows whose bits
//   2-3 differ between four consecutive rows).
// The loads are issued from inline assembly so that the compiler does not count them as
// pending LDS stores (it would make every barrier wait for all of them); callers wait with
// s_waitcnt vmcnt before the barrier that precedes the first read of a stage.
constexpr int kLdsRowB = 256;                   // bytes per bf16 row at head dimension 128
constexpr int kLdsTileB = 64 * kLdsRowB;        // one 64-row tile
enum { kSwzRow = 0, kSwzTr = 1, kSwzBoth = 2 };

template <int S>
__device__ __forceinline__ int swz(int row) {
    if constexpr (S == kSwzRow) return row & 15;
    else if constexpr (S == kSwzTr) return 4 * (row & 3);
    else return (4 * (row & 3)) | ((row >> 2) & 3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words over [base, base + bytes) (as make_rsrc), for inline assembly.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from the buffer at byte offset `voff` into LDS at `lds` + 16 * lane
// (`lds` wave-uniform). No register receives data, so nothing is left for the compiler to
// reuse while the load is in flight.
// The block sets M0 itself and the load reads it at once. M0 is a register the compiler
// reserves: it does not honour it in a clobber list (so none is given), and the block is
// correct only because nothing the compiler emits in these kernels keeps a value in M0
// across it. The library build checks that on the generated assembly: every M0 reference
// and every load into LDS must sit inside one of these blocks, and nothing else may use
// M0 implicitly (relative register moves, messages, GWS or ordered-count operations).
__device__ __forceinline__ void load16_to_lds(i32x4 r, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(lds)
                 : "memory");
}

// 4 bytes per lane from the buffer at byte offset `voff` into LDS at `lds` + 4 * lane: one
// wave instruction fills 256 bytes (a row of 64 fp32 statistics). Same M0 contract as above.
// The descriptor and the LDS address must be wave-uniform; they are read from the first lane
// so that they sit in scalar registers even where the compiler cannot prove them uniform.
__device__ __forceinline__ void load4_to_lds(i32x4 r, uint32_t voff, uint32_t lds) {
    i32x4 u;
    u[0] = __builtin_amdgcn_readfirstlane(r[0]);
    u[1] = __builtin_amdgcn_readfirstlane(r[1]);
    u[2] = __builtin_amdgcn_readfirstlane(r[2]);
    u[3] = __builtin_amdgcn_readfirstlane(r[3]);
    const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(u), "s"(l)
                 : "memory");
}

// 16-byte row read and 8-byte transposing read at an LDS byte address.
__device__ __forceinline__ bf16x8 lds16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}
__device__ __forceinline__ u32x2 lds_tr4(uint32_t addr) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr));
}
__device__ __forceinline__ f32x4 lds_f32x4(uint32_t addr) {
    return *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)addr;
}

// Per-thread part of one step's K and V loads: a 64-row tile is 16 pieces of 1 KB; each of
// the NW waves loads 16 / NW consecutive pieces of K and as many of V. A stage holds the K
// tile (swizzle SK) and then the V tile (swizzle SV). Rows past the end read as zeros (the
// buffer range check).
template <int NW, int SK, int SV>
struct DmaStage {
    static constexpr int P = 16 / NW;
    static_assert(P * NW == 16, "the waves must split the tile evenly");
    uint32_t koff[P], voff[P];   // global byte offsets relative to the step's first row

    __device__ void init(int wave, int lane, int64_t ksn, int64_t vsn) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int row = 4 * (P * wave + j) + (lane >> 4), slot = lane & 15;
            koff[j] = (uint32_t)((int64_t)row * ksn * 2 + 16 * (slot ^ swz<SK>(row)));
            voff[j] = (uint32_t)((int64_t)row * vsn * 2 + 16 * (slot ^ swz<SV>(row)));
        }
    }
    // `stage` (LDS byte address) and `wave` must be wave-uniform: the loads take M0.
    __device__ void issue(const uint16_t* kbase, const uint16_t* vbase, int64_t ksn, int64_t vsn, int r0, int N,
                          uint32_t stage, int wave) const {
        const i32x4 rk = rsrc_words(kbase + (int64_t)r0 * ksn, rows_bytes(r0, N, ksn, 128, 64));
        const i32x4 rv = rsrc_words(vbase + (int64_t)r0 * vsn, rows_bytes(r0, N, vsn, 128, 64));
        const uint32_t piece = stage + 1024u * P * (uint32_t)wave;
#pragma unroll
        for (int j = 0; j < P; ++j) load16_to_lds(rk, koff[j], piece + 1024u * j);
#pragma unroll
        for (int j = 0; j < P; ++j) load16_to_lds(rv, voff[j], piece + kLdsTileB + 1024u * j);
    }
};

// LDS byte address of a __shared__ object, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// Output of one wave at head dimension 128: 32 rows held in accumulator order (lane (i, hf),
// block cb, group j: columns 32 cb + 8 j + 4 hf .. + 3 of local row `lrow`), scaled by `sc`
// and written as bf16 to rows row0 + r (r < 32, row0 + r < nrows) of a row-major tensor
// (`base`: row 0, `rs`: row stride in elements, both 16-byte aligned). Stored directly, each
// store instruction would write 64 scattered 8-byte pieces; staged through the wave's own LDS
// area (32 rows of kRowStagePitch bytes at `lds_wave`, not in use by any wave when called)
// whole rows go out, 16 lanes per row, 16 bytes each, non-temporal. The wave reads back only
// what it wrote, so no barrier is needed.
constexpr uint32_t kRowStagePitch = 2 * 128 + 16;   // the pad spreads a wave's row writes evenly over the banks
constexpr uint32_t kRowStageWaveB = 32 * kRowStagePitch;
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[4], float sc, int lrow, int hf, int lane,
                                                  uint16_t* base, int64_t rs, int row0, int nrows, uint32_t lds_wave) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = (__bf16)(acc[cb][4 * j + e] * sc);
            *(__attribute__((address_space(3))) bf16x4*)(uintptr_t)(lds_wave + lrow * kRowStagePitch +
                                                                  2 * (32 * cb + 8 * j + 4 * hf)) = a;
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    const int ch = lane & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4);
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(lds_wave + r * kRowStagePitch + 16 * ch);
        if (row0 + r < nrows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + (int64_t)(row0 + r) * rs + 8 * ch));
    }
}

}  // namespace fa
