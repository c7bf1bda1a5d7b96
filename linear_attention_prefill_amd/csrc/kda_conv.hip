// Short conv front end of the prefill for gfx950.
//
// On the prefill side of the kern-k3-pp-prefill page every sequence carries
// a conv window next to its recurrent state (section "P: the packed prefill"); SGLang keeps the
// window as [slot][tap][q | k | v] bf16 (section "D inside SGLang").  Each
// head's channels [q | k | v] are convolved per sequence with 4 taps, the
// three inputs before a sequence's first row coming from its window, and the
// window is left holding the sequence's last three raw inputs.
//
// kda_conv_kernel writes the convolved q, k, v (io dtype) for the intra-chunk
// kernel to read in place of the raw inputs.  A workgroup covers 64 rows of
// one head, heads varying fastest across the grid: 4 groups of 16 rows times
// (2 d_k + d_v) / 8 channel octets (quads for fp32), one thread each.  A
// thread loads its 16 rows and the 3 before them up front (indices clamped, so
// no load is conditional) and rolls the taps along the rows when all of them
// lie in one sequence; the few groups that touch a
// sequence start or end go row by row, reading the window where the three
// earlier inputs fall before the start.
//
// kda_conv_window_kernel then stores each live sequence's new window.  It
// runs after the conv kernel in stream order, so no workgroup can still be
// reading a window it overwrites.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kConvRows = 16;       // rows per thread
constexpr int kConvGroups = 4;      // row groups per 64-row block

// 16 bytes of io values: every load and store of the conv pass moves whole
// 16-byte pieces per lane (narrower bf16 stores reach L2 as partial lines).
template <typename E> struct Io16;
template <> struct Io16<bf16> {
    static constexpr int kN = 8;
    typedef bf16x8 raw;
    __device__ static float get(const raw &r, int e) { return (float)r[e]; }
    __device__ static void put(raw &r, int e, float x) { r[e] = (bf16)x; }
};
template <> struct Io16<float> {
    static constexpr int kN = 4;
    typedef f32x4 raw;
    __device__ static float get(const raw &r, int e) { return r[e]; }
    __device__ static void put(raw &r, int e, float x) { r[e] = x; }
};

template <typename E, int DK, int DV>
constexpr int conv_threads() { return kConvGroups * (2 * DK + DV) / Io16<E>::kN; }

template <typename E, int DK, int DV, int SILU>
__global__ __launch_bounds__((conv_threads<E, DK, DV>())) void kda_conv_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    E *__restrict__ qc, E *__restrict__ kc, E *__restrict__ vc,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots,
    const float *__restrict__ weight, const E *__restrict__ window, ConvWin win, int T, int N,
    int H, int num_slots) {
    using IO = Io16<E>;
    using Raw = typename IO::raw;
    constexpr int V = IO::kN;            // channels per thread
    constexpr int C = 2 * DK + DV;
    constexpr int CG = C / V;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    // heads vary fastest across the grid, so the workgroups in flight read
    // whole rows of q, k and v rather than one head's slice of many rows
    // (which would fall on a few HBM channels)
    const int h = blockIdx.x % H;
    const int r0 = (blockIdx.x / H) * kChunk + rg * kConvRows;
    if (r0 >= T) return;
    const int ch = V * cg;
    const int part = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
    const int pc = ch - part * DK;
    const E *src = part == 0 ? q : (part == 1 ? k : v);
    E *dst = part == 0 ? qc : (part == 1 ? kc : vc);
    const int D = part == 2 ? DV : DK;

    Raw x[kConvRows + kConvWindow];      // raw io values, converted at use
#pragma unroll
    for (int i = 0; i < kConvRows + kConvWindow; ++i) {
        int row = r0 - kConvWindow + i;
        row = row < 0 ? 0 : (row > T - 1 ? T - 1 : row);
        x[i] = *reinterpret_cast<const Raw *>(src + ((size_t)row * H + h) * D + pc);
    }
    float w[kConvTaps][V];
#pragma unroll
    for (int j = 0; j < kConvTaps; ++j) {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(
                weight + ((size_t)h * kConvTaps + j) * C + ch + e);
            w[j][e] = t[0]; w[j][e + 1] = t[1]; w[j][e + 2] = t[2]; w[j][e + 3] = t[3];
        }
    }

    // the sequence holding row r0: the last n with cu[n] <= r0
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (clamp_row(cu[mid], T) <= r0) lo = mid; else hi = mid - 1;
    }
    int n = lo;
    int start = clamp_row(cu[n], T), end = clamp_row(cu[n + 1], T);
    const int r1 = min(r0 + kConvRows, T);

    if (start <= r0 - kConvWindow && end >= r1) {
        // every row of the group and the three before it lie in sequence n
#pragma unroll
        for (int i = 0; i < kConvRows; ++i) {
            if (r0 + i < r1) {
                Raw y;
#pragma unroll
                for (int e = 0; e < V; ++e)
                    IO::put(y, e, conv_act(conv4(w[0][e], w[1][e], w[2][e], w[3][e],
                                                 IO::get(x[i], e), IO::get(x[i + 1], e),
                                                 IO::get(x[i + 2], e), IO::get(x[i + 3], e)),
                                           SILU));
                *reinterpret_cast<Raw *>(dst + ((size_t)(r0 + i) * H + h) * D + pc) = y;
            }
        }
        return;
    }
    // rows near a sequence start or end, one at a time from memory
#pragma unroll 1
    for (int r = r0; r < r1; ++r) {
        while (r >= end && n < N - 1) {
            ++n;
            start = clamp_row(cu[n], T);
            end = clamp_row(cu[n + 1], T);
        }
        if (r < start || r >= end) continue;     // not in any sequence
        const int slot = slots ? slots[n] : n;
        const bool live = slot >= 0 && slot < num_slots;
        Raw t[kConvTaps];
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) {
            const int rr = r - kConvWindow + j;
            if (rr >= start) {
                t[j] = *reinterpret_cast<const Raw *>(src + ((size_t)rr * H + h) * D + pc);
            } else if (live) {
                t[j] = *reinterpret_cast<const Raw *>(
                    window + win.at(slot, h, kConvWindow - (start - rr), part, pc));
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) IO::put(t[j], e, 0.f);
            }
        }
        Raw y;
#pragma unroll
        for (int e = 0; e < V; ++e)
            IO::put(y, e, conv_act(conv4(w[0][e], w[1][e], w[2][e], w[3][e], IO::get(t[0], e),
                                         IO::get(t[1], e), IO::get(t[2], e), IO::get(t[3], e)),
                                   SILU));
        *reinterpret_cast<Raw *>(dst + ((size_t)r * H + h) * D + pc) = y;
    }
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__((2 * DK + DV) / 4) void kda_conv_window_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots, E *window, ConvWin win,
    int T, int N, int H, int num_slots) {
    const int n = blockIdx.x, h = blockIdx.y;
    const int slot = slots ? slots[n] : n;
    if (slot < 0 || slot >= num_slots) return;
    const int start = clamp_row(cu[n], T);
    const int end = clamp_row(cu[n + 1], T);
    const int L = end - start;
    if (L <= 0) return;                          // the window stays as it is
    const int ch = 4 * threadIdx.x;
    const int part = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
    const int pc = ch - part * DK;
    const E *src = part == 0 ? q : (part == 1 ? k : v);
    const int D = part == 2 ? DV : DK;
    f32x4 old[kConvWindow], fresh[kConvWindow];
#pragma unroll
    for (int i = 0; i < kConvWindow; ++i) {
        old[i] = load4<E>(window + win.at(slot, h, i, part, pc));
        int row = end - kConvWindow + i;
        row = row < start ? start : row;
        fresh[i] = load4<E>(src + ((size_t)row * H + h) * D + pc);
    }
#pragma unroll
    for (int i = 0; i < kConvWindow; ++i) {
        // new row i is input end - 3 + i, or old row i + L (1 or 2) when the
        // sequence is shorter than the window
        f32x4 val = fresh[i];
        if (i + L < kConvWindow) val = (i + L == 1) ? old[1] : old[2];
        store4<E>(window + win.at(slot, h, i, part, pc), val);
    }
}

template <typename E, int DK, int DV>
hipError_t launch_conv_front(const ConvArgs &a, hipStream_t stream) {
    constexpr int C = 2 * DK + DV;
    if (a.T > 0) {
        const dim3 grid(((a.T + kChunk - 1) / kChunk) * a.H);
        auto kern = a.silu ? kda_conv_kernel<E, DK, DV, 1> : kda_conv_kernel<E, DK, DV, 0>;
        kern<<<grid, dim3(conv_threads<E, DK, DV>()), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            static_cast<E *>(a.qc), static_cast<E *>(a.kc), static_cast<E *>(a.vc), a.cu_seqlens,
            a.slots, a.weight, static_cast<const E *>(a.window), a.win, a.T, a.N, a.H,
            a.num_slots);
        kda_conv_window_kernel<E, DK, DV><<<dim3(a.N, a.H), dim3(C / 4), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            a.cu_seqlens, a.slots, static_cast<E *>(a.window), a.win, a.T, a.N, a.H, a.num_slots);
    }
    return hipGetLastError();
}

#define KDA_INST(E, DK, DV) \
    template hipError_t launch_conv_front<E, DK, DV>(const ConvArgs &, hipStream_t);
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
