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

constexpr int kConvRows = 8;        // rows per thread
constexpr int kConvGroups = 8;      // row groups per 64-row block
constexpr int kConvWgPerCu = 2;     // resident workgroups per CU the grid is sized for

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

// Persistent over the 64-row blocks of one head: workgroup b takes head
// b % H and blocks b / H, b / H + RB, ...  The next block's rows are fetched
// into a second register set while the current one is convolved, so a wave
// computes (the SiLU's two transcendentals per element dominate) while its
// next loads are in flight; one-shot workgroups left all the waves of a CU
// waiting on their loads together, then computing together.
template <typename E, int DK, int DV, int SILU>
__global__ __launch_bounds__((conv_threads<E, DK, DV>())) void kda_conv_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    E *__restrict__ qc, E *__restrict__ kc, E *__restrict__ vc,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots,
    const float *__restrict__ weight, const E *__restrict__ window, ConvWin win, int T, int N,
    int H, int num_slots, int RB) {
    using IO = Io16<E>;
    using Raw = typename IO::raw;
    constexpr int V = IO::kN;            // channels per thread
    constexpr int C = 2 * DK + DV;
    constexpr int CG = C / V;
    constexpr int NX = kConvRows + kConvWindow;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int h = blockIdx.x % H;
    const int nblk = (T + kChunk - 1) / kChunk;
    int rb = blockIdx.x / H;
    if (rb >= nblk) return;
    const int ch = V * cg;
    const int part = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
    const int pc = ch - part * DK;
    const E *src = part == 0 ? q : (part == 1 ? k : v);
    E *dst = part == 0 ? qc : (part == 1 ? kc : vc);
    const int D = part == 2 ? DV : DK;

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
    // raw io rows r0 - 3 .. r0 + kConvRows - 1 of a block (indices clamped,
    // so no load is conditional), converted at use
    auto fetch = [&](Raw (&x)[NX], int b) {
        const int r0 = b * kChunk + rg * kConvRows;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            int row = r0 - kConvWindow + i;
            row = row < 0 ? 0 : (row > T - 1 ? T - 1 : row);
            x[i] = *reinterpret_cast<const Raw *>(src + ((size_t)row * H + h) * D + pc);
        }
    };
    auto out = [&](int r, const float (&y)[V]) {
        Raw o;
#pragma unroll
        for (int e = 0; e < V; ++e) IO::put(o, e, conv_act(y[e], SILU));
        *reinterpret_cast<Raw *>(dst + ((size_t)r * H + h) * D + pc) = o;
    };
    // the sequence holding a row: carried from block to block (blocks only
    // move forward), found by a binary search the first time
    int n = 0, start = 0, end = 0;
    {
        const int r0 = rb * kChunk + rg * kConvRows;
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (clamp_row(cu[mid], T) <= r0) lo = mid; else hi = mid - 1;
        }
        n = lo;
        start = clamp_row(cu[n], T);
        end = clamp_row(cu[n + 1], T);
    }
    auto apply = [&](const Raw (&x)[NX], int b) {
        const int r0 = b * kChunk + rg * kConvRows;
        if (r0 >= T) return;
        const int r1 = min(r0 + kConvRows, T);
        while (r0 >= end && n < N - 1) {
            ++n;
            start = clamp_row(cu[n], T);
            end = clamp_row(cu[n + 1], T);
        }
        if (start <= r0 - kConvWindow && end >= r1) {
            // every row of the group and the three before it lie in sequence
            // n: roll the taps along the rows, each input converted once
            float xm3[V], xm2[V], xm1[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                xm3[e] = IO::get(x[0], e);
                xm2[e] = IO::get(x[1], e);
                xm1[e] = IO::get(x[2], e);
            }
#pragma unroll
            for (int i = 0; i < kConvRows; ++i) {
                float x0[V], y[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    x0[e] = IO::get(x[i + kConvWindow], e);
                    y[e] = conv4(w[0][e], w[1][e], w[2][e], w[3][e], xm3[e], xm2[e], xm1[e], x0[e]);
                }
                if (r0 + i < r1) out(r0 + i, y);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    xm3[e] = xm2[e];
                    xm2[e] = xm1[e];
                    xm1[e] = x0[e];
                }
            }
            return;
        }
        // rows near a sequence start or end, one at a time from memory
        int sn = n, ss = start, se = end;
#pragma unroll 1
        for (int r = r0; r < r1; ++r) {
            while (r >= se && sn < N - 1) {
                ++sn;
                ss = clamp_row(cu[sn], T);
                se = clamp_row(cu[sn + 1], T);
            }
            if (r < ss || r >= se) continue;     // not in any sequence
            const int slot = slots ? slots[sn] : sn;
            const bool live = slot >= 0 && slot < num_slots;
            Raw t[kConvTaps];
#pragma unroll
            for (int j = 0; j < kConvTaps; ++j) {
                const int rr = r - kConvWindow + j;
                if (rr >= ss) {
                    t[j] = *reinterpret_cast<const Raw *>(src + ((size_t)rr * H + h) * D + pc);
                } else if (live) {
                    t[j] = *reinterpret_cast<const Raw *>(
                        window + win.at(slot, h, kConvWindow - (ss - rr), part, pc));
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e) IO::put(t[j], e, 0.f);
                }
            }
            float y[V];
#pragma unroll
            for (int e = 0; e < V; ++e)
                y[e] = conv4(w[0][e], w[1][e], w[2][e], w[3][e], IO::get(t[0], e), IO::get(t[1], e),
                             IO::get(t[2], e), IO::get(t[3], e));
            out(r, y);
        }
    };

    // two register sets, alternating by block: the next block's loads are
    // issued before the current block is convolved
    Raw xa[NX], xb[NX];
    fetch(xa, rb);
    for (;;) {
        const int nb = rb + RB;
        fetch(xb, nb < nblk ? nb : nblk - 1);
        apply(xa, rb);
        if (nb >= nblk) break;
        rb = nb;
        const int nb2 = rb + RB;
        fetch(xa, nb2 < nblk ? nb2 : nblk - 1);
        apply(xb, rb);
        if (nb2 >= nblk) break;
        rb = nb2;
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
        // RB blocks of rows in flight per head: about kConvWgPerCu workgroups
        // per CU over all heads, each then walking nblk / RB blocks
        const int nblk = (a.T + kChunk - 1) / kChunk;
        const int want = kConvWgPerCu * (a.num_cus > 0 ? a.num_cus : 256);
        int RB = (want + a.H - 1) / a.H;
        RB = RB < 1 ? 1 : (RB > nblk ? nblk : RB);
        const dim3 grid(RB * a.H);
        auto kern = a.silu ? kda_conv_kernel<E, DK, DV, 1> : kda_conv_kernel<E, DK, DV, 0>;
        kern<<<grid, dim3(conv_threads<E, DK, DV>()), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            static_cast<E *>(a.qc), static_cast<E *>(a.kc), static_cast<E *>(a.vc), a.cu_seqlens,
            a.slots, a.weight, static_cast<const E *>(a.window), a.win, a.T, a.N, a.H,
            a.num_slots, RB);
        kda_conv_window_kernel<E, DK, DV><<<dim3(a.N, a.H), dim3(C / 4), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            a.cu_seqlens, a.slots, static_cast<E *>(a.window), a.win, a.T, a.N, a.H, a.num_slots);
    }
    return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_conv_window(const ConvArgs &a, hipStream_t stream) {
    constexpr int C = 2 * DK + DV;
    if (a.T > 0)
        kda_conv_window_kernel<E, DK, DV><<<dim3(a.N, a.H), dim3(C / 4), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            a.cu_seqlens, a.slots, static_cast<E *>(a.window), a.win, a.T, a.N, a.H, a.num_slots);
    return hipGetLastError();
}

#define KDA_INST(E, DK, DV) \
    template hipError_t launch_conv_front<E, DK, DV>(const ConvArgs &, hipStream_t); \
    template hipError_t launch_conv_window<E, DK, DV>(const ConvArgs &, hipStream_t);
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
