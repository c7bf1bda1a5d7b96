// Device-side building blocks shared by the KDA kernels (gfx950, wave64).
//
// Matrix-core fragments.  Every contraction in the chunked prefill is issued
// as 16x16 output tiles over 32-wide slabs of the contraction index:
//   bf16: one v_mfma_f32_16x16x32_bf16 per slab;
//   fp32: eight v_mfma_f32_16x16x4_f32 per slab (exact fp32 products).
// Lane l = 16*g + i (i = l % 16, g = l / 16) of a wave holds, for a slab:
//   A operand (16 x 32): row i, eight contraction indices kk(g, 0..7);
//   B operand (32 x 16): column i, the same eight contraction indices;
//   C/D (16 x 16):       column i, rows 4g + 0..3.
// The contraction index order inside a slab is free as long as A and B agree,
// so all operands use kk(g, e) = 4g + (e & 3) + 16 (e >> 2).  With this order
// two stacked 16x16 accumulator tiles (rows 0..15 and 16..31 of a slab) are
// already a B operand lane for lane, which lets the state and the corrected
// values stay in registers between contractions with no shuffles.
// Swapping the A and B registers of a product yields its transpose, with lane
// (i, g) holding D[i][4g + r]; that layout is the A operand of a later
// product, which is how the intra-chunk kernel writes w in the scan's order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;      // rows per chunk
constexpr int kSub = 16;        // rows per sub-block / MFMA tile edge
constexpr int kSlab = 32;       // contraction slab
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int kk_of(int g, int e) { return 4 * g + (e & 3) + 16 * (e >> 2); }

// Eight-element operand fragment in the io element type.
template <typename E> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 x;
    __device__ __forceinline__ void set(int e, float v) { x[e] = (bf16)v; }
    __device__ __forceinline__ float get(int e) const { return (float)x[e]; }
};
template <> struct Frag<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void set(int e, float v) {
        if (e < 4) lo[e] = v; else hi[e - 4] = v;
    }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x, b.x, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

// Two stacked C tiles (slab rows 0..15 in t0, 16..31 in t1) as a B operand.
template <typename E>
__device__ __forceinline__ Frag<E> frag_from_tiles(const f32x4 &t0, const f32x4 &t1) {
    Frag<E> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) { f.set(r, t0[r]); f.set(4 + r, t1[r]); }
    return f;
}

// A fragment from two runs of four consecutive elements (e < 4 from p0,
// e >= 4 from p1), e.g. two 8-byte LDS reads for bf16.
template <typename E>
__device__ __forceinline__ Frag<E> frag_from_runs(const E *p0, const E *p1);
template <>
__device__ __forceinline__ Frag<bf16> frag_from_runs<bf16>(const bf16 *p0, const bf16 *p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
    Frag<bf16> f;
    f.x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_from_runs<float>(const float *p0, const float *p1) {
    Frag<float> f;
    f.lo = *reinterpret_cast<const f32x4 *>(p0);
    f.hi = *reinterpret_cast<const f32x4 *>(p1);
    return f;
}

// B-operand fragment of a row-major LDS tile M (pitch P elements): lane
// (i, g) receives M[k0 + kk(g, e)][n0 + i], i.e. column n0 + i with the
// contraction running down the rows.  For bf16 this is two transposing LDS
// reads (ds_read_b64_tr_b16).  Within each group of 16 lanes that read hands
// lane l element (l & 3) of the 8-byte runs addressed by lanes (l >> 2) + 4j,
// j = 0..3; so lane m of group g addresses row k0 + 4g + (m >> 2), columns
// n0 + 4 (m & 3) .. + 3, and a second read 16 rows further down supplies
// elements 4..7.  Rows of M must be 8-byte aligned (P, n0 multiples of 4).
typedef short v4i16 __attribute__((ext_vector_type(4)));
template <typename E>
__device__ __forceinline__ Frag<E> frag_cols(const E *M, int P, int k0, int n0, int lane);
template <>
__device__ __forceinline__ Frag<bf16> frag_cols<bf16>(const bf16 *M, int P, int k0, int n0, int lane) {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int m = lane & 15, g = lane >> 4;
    bf16 *p = const_cast<bf16 *>(M) + (k0 + 4 * g + (m >> 2)) * P + n0 + 4 * (m & 3);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 16 * P));
    Frag<bf16> f;
    f.x = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_cols<float>(const float *M, int P, int k0, int n0, int lane) {
    const int i = lane & 15, g = lane >> 4;
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.set(e, M[(k0 + kk_of(g, e)) * P + n0 + i]);
    return f;
}

// Global fragment load/store: one fragment is 64 lanes x 8 elements,
// contiguous per lane, so a wave moves 1 KiB (bf16) or 2 KiB (fp32) with
// perfectly coalesced 16-byte accesses.
template <typename E>
__device__ __forceinline__ Frag<E> load_frag(const E *base, int lane);
template <>
__device__ __forceinline__ Frag<bf16> load_frag<bf16>(const bf16 *base, int lane) {
    Frag<bf16> f;
    f.x = *reinterpret_cast<const bf16x8 *>(base + 8 * lane);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag<float>(const float *base, int lane) {
    Frag<float> f;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(base + 8 * lane);
    f.lo = p[0];
    f.hi = p[1];
    return f;
}
template <typename E>
__device__ __forceinline__ void store_frag(E *base, int lane, const Frag<E> &f);
template <>
__device__ __forceinline__ void store_frag<bf16>(bf16 *base, int lane, const Frag<bf16> &f) {
    *reinterpret_cast<bf16x8 *>(base + 8 * lane) = f.x;
}
template <>
__device__ __forceinline__ void store_frag<float>(float *base, int lane, const Frag<float> &f) {
    f32x4 *p = reinterpret_cast<f32x4 *>(base + 8 * lane);
    p[0] = f.lo;
    p[1] = f.hi;
}

// Four consecutive io elements <-> float4.
template <typename E> __device__ __forceinline__ f32x4 load4(const E *p);
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16 *p) {
    bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <> __device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <typename E> __device__ __forceinline__ void store4(E *p, const f32x4 &v);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, const f32x4 &v) {
    bf16x4 x;
    x[0] = (bf16)v[0]; x[1] = (bf16)v[1]; x[2] = (bf16)v[2]; x[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4 *>(p) = x;
}
template <> __device__ __forceinline__ void store4<float>(float *p, const f32x4 &v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw io vectors of four elements, kept unconverted while loads are in flight.
template <typename E> struct Raw4Of { typedef f32x4 type; };
template <> struct Raw4Of<bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 raw_to_f32(const f32x4 &x) { return x; }
__device__ __forceinline__ f32x4 raw_to_f32(const bf16x4 &x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// Varlen bookkeeping shared by the prefill kernels.  Sequence n starts at
// row clamp(cu[n], 0, T) and ends at clamp(cu[n+1], start, T).  Its chunks
// take the ids floor(start / 64) + n + j, j = 0 .. ceil(len / 64) - 1; these
// ranges are disjoint across sequences, so every chunk has a workspace record
// without any prefix sum over sequences.  The last id of sequence n is at most
// floor((start + len - 1) / 64) + n <= floor((T - 1) / 64) + N - 1, whatever
// the offsets, so chunk_id_count ids cover every chunk (at T = 8192, N = 1
// that is 128 ids, a whole number of 64-chunk windows).
__host__ __device__ constexpr int chunk_id_count(int T, int N) { return T > 0 ? (T - 1) / kChunk + N : N; }
struct SeqSpan {
    int start, len, first_chunk;
};
__device__ __forceinline__ int clamp_row(int x, int T) { return x < 0 ? 0 : (x > T ? T : x); }
__device__ __forceinline__ SeqSpan seq_span(const int32_t *cu, int n, int T) {
    SeqSpan s;
    s.start = clamp_row(cu[n], T);
    int end = clamp_row(cu[n + 1], T);
    s.len = end > s.start ? end - s.start : 0;
    s.first_chunk = s.start / kChunk + n;
    return s;
}

// Index of the lower-triangular fragment (row tile m, 32-row slab s <= m/2)
// of a 64x64 lower-triangular matrix: 0, 1, (2, 3), (4, 5).
__device__ __forceinline__ constexpr int tri_frag(int m, int s) { return m < 2 ? m : 2 * m - 2 + s; }

// Workspace record layout: one record per (chunk id, head), all fragments in
// the scan's lane order.  Offsets are in elements of type E except `dec`.
template <typename E, int DK, int DV> struct WsLayout {
    static constexpr int kWElems = kChunk * DK;           // w:    4 x (DK/32) frags
    static constexpr int kQElems = kChunk * DK;           // q*exp(Gamma): same
    static constexpr int kKElems = DK * kChunk;           // K~^T: (DK/16) x 2 frags
    static constexpr int kAElems = 6 * 512;               // A_qk: the 6 lower frags
    static constexpr int kUElems = kChunk * DV;           // u: (DV/16) tiles x 4 row tiles x 64 lanes x 4
    static constexpr int kRecElems = kWElems + kQElems + kKElems + kAElems + kUElems;
};

// Short conv front end (shared by the prefill pass and the fused decode).
// Each head's channels [q | k | v] are convolved per sequence with 4 taps:
// y_t = w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t, the three older inputs
// coming from the sequence's window at its start, then an optional SiLU;
// the result is rounded to the io dtype, as the layer before would emit it.
constexpr int kConvWindow = 3;
constexpr int kConvTaps = kConvWindow + 1;

__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float xm3,
                                       float xm2, float xm1, float x0) {
#pragma clang fp contract(off)
    return __builtin_fmaf(w3, x0, __builtin_fmaf(w2, xm1, __builtin_fmaf(w1, xm2, w0 * xm3)));
}

// SiLU y / (1 + e^-y) with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float conv_act(float y, int silu) {
#pragma clang fp contract(off)
    return silu ? y * __builtin_amdgcn_rcpf(1.f + fast_exp2(-y * kLog2e)) : y;
}

template <typename E> __device__ __forceinline__ float round_io(float x) { return (float)(E)x; }

}  // namespace kda
