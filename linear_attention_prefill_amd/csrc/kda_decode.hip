// KDA single-token decode step for gfx950: a streaming read-modify-write of
// the state pool (the KDA step of the kern-k3-pp-prefill page, section
// "D: TP8 / EP8 / DCP8"; padded rows with an out-of-range slot are skipped,
// as its section "D inside SGLang" describes for slot -1).
//
// For one (sequence, head) with the pool row j holding column j of S
// (the [slot][head][v][k] layout), one token does
//   s' = exp(g) * S[:, j]                    decay per key channel
//   d_j = beta (v_j - s'.k)                  delta-rule correction
//   S[:, j] = s' + d_j k                     write back in place
//   o_j = scale (s'.q + d_j (k.q))           = scale S_new[:, j].q
// so each 4 * d_k-byte row is read once and written once.  A workgroup of 256
// threads covers 64 rows of one (sequence, head); d_k / 4 lanes share a row,
// each lane holding four key channels, and the two dot products are reduced
// across those lanes with cross-lane shuffles.  Every lane issues all of its
// row loads before any arithmetic, so each workgroup keeps 64 rows
// (16-32 KiB) in flight.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kDecodeRows = 64;

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *pool,
    const int32_t *__restrict__ slots, E *__restrict__ o, int N, int H, int num_slots,
    float scale) {
    constexpr int PARTS = DV / kDecodeRows;
    constexpr int LPR = DK / 4;          // lanes per state row
    constexpr int RPI = 256 / LPR;       // rows covered by one pass of the workgroup
    constexpr int P = kDecodeRows / RPI; // passes
    const int tid = threadIdx.x;
    const int part = blockIdx.x % PARTS;
    const int nh = blockIdx.x / PARTS;
    const int n = nh / H, h = nh % H;
    if (n >= N) return;
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) return;   // padded row: touch nothing
    const int c4 = tid % LPR, rr = tid / LPR;
    const size_t tok = (size_t)n * H + h;

    const f32x4 k4 = load4<E>(k + tok * DK + 4 * c4);
    const f32x4 q4 = load4<E>(q + tok * DK + 4 * c4);
    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(g + tok * DK + 4 * c4);
    const float bt = beta[tok];
    float *S = pool + ((size_t)slot * H + h) * (size_t)DV * DK;

    f32x4 s[P];
    float vv[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kDecodeRows + p * RPI + rr;
        s[p] = *reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * c4);
        vv[p] = (float)v[tok * DV + row];
    }

    f32x4 a4;
#pragma unroll
    for (int r = 0; r < 4; ++r) a4[r] = fast_exp2(g4[r] * kLog2e);
    float kq = k4[0] * q4[0] + k4[1] * q4[1] + k4[2] * q4[2] + k4[3] * q4[3];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) kq += __shfl_xor(kq, m);

#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kDecodeRows + p * RPI + rr;
        const f32x4 sp = s[p] * a4;
        float dk = sp[0] * k4[0] + sp[1] * k4[1] + sp[2] * k4[2] + sp[3] * k4[3];
        float dq = sp[0] * q4[0] + sp[1] * q4[1] + sp[2] * q4[2] + sp[3] * q4[3];
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) {
            dk += __shfl_xor(dk, m);
            dq += __shfl_xor(dq, m);
        }
        const float d = bt * (vv[p] - dk);
        *reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * c4) = sp + d * k4;
        if (c4 == 0) o[tok * DV + row] = (E)(scale * (dq + d * kq));
    }
}

template <typename E, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    const int nblocks = a.N * a.H * (DV / kDecodeRows);
    kda_decode_kernel<E, DK, DV><<<dim3(nblocks), dim3(256), 0, stream>>>(
        static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
        a.g, a.beta, a.pool, a.slots, static_cast<E *>(a.o), a.N, a.H, a.num_slots, a.scale);
    return hipGetLastError();
}

#define KDA_INST(E, DK, DV) \
    template hipError_t launch_decode<E, DK, DV>(const DecodeArgs &, hipStream_t);
KDA_INST(bf16, 64, 64)
KDA_INST(bf16, 64, 128)
KDA_INST(bf16, 128, 64)
KDA_INST(bf16, 128, 128)
KDA_INST(float, 64, 64)
KDA_INST(float, 64, 128)
KDA_INST(float, 128, 64)
KDA_INST(float, 128, 128)
#undef KDA_INST

}  // namespace kda
