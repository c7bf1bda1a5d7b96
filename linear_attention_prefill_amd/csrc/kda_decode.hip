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
// threads covers 64 rows of one (sequence, head); a row is spread over the 16
// lanes of a DPP row, each lane holding d_k / 16 key channels, and the two dot
// products are summed across those lanes with four row rotations.  Every lane
// issues all of its row loads before any arithmetic, so each workgroup keeps
// 64 rows (16-32 KiB) in flight.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kDecodeRows = 64;

// Sum over the 16 lanes of a DPP row, left in every lane (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row_allreduce(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
    return x;
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *pool,
    const int32_t *__restrict__ slots, E *__restrict__ o, int N, int H, int num_slots,
    float scale, int64_t slot_stride, int64_t head_stride) {
    constexpr int PARTS = DV / kDecodeRows;
    constexpr int CPL = DK / 16;         // key channels per lane
    constexpr int V4 = CPL / 4;          // float4 per lane and row
    constexpr int RPI = 256 / 16;        // rows covered by one pass of the workgroup
    constexpr int P = kDecodeRows / RPI; // passes
    const int tid = threadIdx.x;
    const int part = blockIdx.x % PARTS;
    const int nh = blockIdx.x / PARTS;
    const int n = nh / H, h = nh % H;
    if (n >= N) return;
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) return;   // padded row: touch nothing
    const int c = tid & 15, rr = tid >> 4;
    const size_t tok = (size_t)n * H + h;

    // lane c holds key channels 4 (c + 16 x) .. + 3, x < V4, so that a row's
    // lanes read consecutive 16-byte pieces
    f32x4 k4[V4], q4[V4], a4[V4];
#pragma unroll
    for (int x = 0; x < V4; ++x) {
        const int ch = 4 * (c + 16 * x);
        k4[x] = load4<E>(k + tok * DK + ch);
        q4[x] = load4<E>(q + tok * DK + ch);
        a4[x] = *reinterpret_cast<const f32x4 *>(g + tok * DK + ch);
    }
    const float bt = beta[tok];
    float *S = pool + slot * slot_stride + h * head_stride;

    f32x4 s[P][V4];
    float vv[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kDecodeRows + p * RPI + rr;
#pragma unroll
        for (int x = 0; x < V4; ++x)
            s[p][x] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
        vv[p] = (float)v[tok * DV + row];
    }

    float kq = 0.f;
#pragma unroll
    for (int x = 0; x < V4; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            a4[x][r] = fast_exp2(a4[x][r] * kLog2e);
            kq += k4[x][r] * q4[x][r];
        }
    }
    kq = row_allreduce(kq);

#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kDecodeRows + p * RPI + rr;
        f32x4 sp[V4];
        float dk = 0.f, dq = 0.f;
#pragma unroll
        for (int x = 0; x < V4; ++x) {
            sp[x] = s[p][x] * a4[x];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dk += sp[x][r] * k4[x][r];
                dq += sp[x][r] * q4[x][r];
            }
        }
        dk = row_allreduce(dk);
        dq = row_allreduce(dq);
        const float d = bt * (vv[p] - dk);
#pragma unroll
        for (int x = 0; x < V4; ++x)
            __builtin_nontemporal_store(sp[x] + d * k4[x],
                                        reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
        if (c == 0) o[tok * DV + row] = (E)(scale * (dq + d * kq));
    }
}

template <typename E, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    const int nblocks = a.N * a.H * (DV / kDecodeRows);
    kda_decode_kernel<E, DK, DV><<<dim3(nblocks), dim3(256), 0, stream>>>(
        static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
        a.g, a.beta, a.pool, a.slots, static_cast<E *>(a.o), a.N, a.H, a.num_slots, a.scale,
        a.slot_stride, a.head_stride);
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
