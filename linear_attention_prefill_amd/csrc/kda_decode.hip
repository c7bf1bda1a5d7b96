// KDA decode for gfx950: streaming read-modify-writes of the state pool.
//
// kda_decode_kernel is the single-token step (the KDA step of the
// kern-k3-pp-prefill page, section "D: TP8 / EP8 / DCP8"; padded rows with an
// out-of-range slot are skipped, as its section "D inside SGLang" describes
// for slot -1).  kda_decode_tokens_kernel runs T tokens per sequence against
// the same state, for multi-token decode and speculative verify (the
// conv-MTP decode kernel and the ReplaySSM exact-fold commit that the prhub
// report on SGLang PR #32890 lists under "关键文件"): outputs for every token,
// and the state written back after the first c tokens or not at all.
//
// For one (sequence, head) with the pool row j holding column j of S
// (the [slot][head][v][k] layout), one token does
//   s' = exp(g) * S[:, j]                    decay per key channel
//   d_j = beta (v_j - s'.k)                  delta-rule correction
//   S[:, j] = s' + d_j k                     write back in place
//   o_j = scale (s'.q + d_j (k.q))           = scale S_new[:, j].q
// Rows are independent, so a workgroup of 256 threads covers a slice of the
// rows of one (sequence, head); a row is spread over the 16 lanes of a DPP
// row, each lane holding d_k / 16 key channels, and the dot products are
// summed across those lanes with four row rotations.  Every lane issues all
// of its row loads before any arithmetic.  The single-token step gives each
// workgroup 16 rows (one pass of its 256 threads, 4-8 KiB of state): many
// small workgroups keep more of HBM busy than fewer large ones (measured, 64
// sequences at H = 32, d = 128: 16 rows 45 us, 32 rows 46 us, 64 rows 47 us,
// 128 rows 49 us).  The multi-token kernel gives each workgroup 32 rows,
// since each of its workgroups stages every token's k, q and decay once
// (64 sequences x 4 tokens, verify and commit in one call: 64 rows 51.4 us,
// 32 rows 49.5 us, 16 rows 55.3 us; a verify alone is 1 us slower at 32).
//
// Both kernels do a token's arithmetic through the same helpers, with every
// multiply-add written out and contraction switched off, so T tokens in one
// call give the state and outputs of T single steps bit for bit.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kDecodeRows = 32;    // state rows per workgroup, multi-token kernel
constexpr int kStepRows = 16;      // state rows per workgroup, single-token step (one pass)
// Threads of the step with the conv, whose workgroup owns all d_v rows of a
// (sequence, head): more waves per workgroup keep more state loads in flight
// (64 sequences at H = 32, d = 128 with SiLU: 256 threads 51.2-51.3 us, 512
// threads 52.0 us, 1024 threads 48.8-49.0 us, on two boxes).
constexpr int kConvStepThreads = 1024;

// Sum over the 16 lanes of a DPP row, left in every lane (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row_allreduce(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
    return x;
}

// Decay of one key channel, e^g.
__device__ __forceinline__ float decay_factor(float g) {
#pragma clang fp contract(off)
    return fast_exp2(g * kLog2e);
}

// The k.q product of a token, from the lane's key channels summed over the
// row's 16 lanes.
template <int V4>
__device__ __forceinline__ float token_kq(const f32x4 (&k)[V4], const f32x4 (&q)[V4]) {
#pragma clang fp contract(off)
    float kq = 0.f;
#pragma unroll
    for (int x = 0; x < V4; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) kq = __builtin_fmaf(k[x][r], q[x][r], kq);
    }
    return row_allreduce(kq);
}

// One token's update of one state row s (its lanes' key channels): s is
// decayed and corrected in place; returns the correction d and leaves the
// row-summed s'.q in dq.
template <int V4>
__device__ __forceinline__ float row_update(f32x4 (&s)[V4], const f32x4 (&a)[V4],
                                            const f32x4 (&k)[V4], const f32x4 (&q)[V4], float bt,
                                            float vj, float &dq) {
#pragma clang fp contract(off)
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int x = 0; x < V4; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sp = s[x][r] * a[x][r];
            s[x][r] = sp;
            sk = __builtin_fmaf(sp, k[x][r], sk);
            sq = __builtin_fmaf(sp, q[x][r], sq);
        }
    }
    sk = row_allreduce(sk);
    dq = row_allreduce(sq);
    const float d = bt * (vj - sk);
#pragma unroll
    for (int x = 0; x < V4; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[x][r] = __builtin_fmaf(d, k[x][r], s[x][r]);
    }
    return d;
}

__device__ __forceinline__ float row_output(float d, float kq, float dq, float scale) {
#pragma clang fp contract(off)
    return scale * __builtin_fmaf(d, kq, dq);
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *pool,
    const int32_t *__restrict__ slots, E *__restrict__ o, int N, int H, int num_slots,
    float scale, int64_t slot_stride, int64_t head_stride) {
    constexpr int PARTS = DV / kStepRows;
    constexpr int CPL = DK / 16;         // key channels per lane
    constexpr int V4 = CPL / 4;          // float4 per lane and row
    constexpr int RPI = 256 / 16;        // rows covered by one pass of the workgroup
    constexpr int P = kStepRows / RPI;   // passes
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
        const int row = part * kStepRows + p * RPI + rr;
#pragma unroll
        for (int x = 0; x < V4; ++x)
            s[p][x] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
        vv[p] = (float)v[tok * DV + row];
    }

#pragma unroll
    for (int x = 0; x < V4; ++x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) a4[x][r] = decay_factor(a4[x][r]);
    }
    const float kq = token_kq<V4>(k4, q4);
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kStepRows + p * RPI + rr;
        float dq;
        const float d = row_update<V4>(s[p], a4, k4, q4, bt, vv[p], dq);
#pragma unroll
        for (int x = 0; x < V4; ++x)
            __builtin_nontemporal_store(s[p][x], reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
        if (c == 0) o[tok * DV + row] = (E)row_output(d, kq, dq, scale);
    }
}

// The decode step with the short conv fused in (the KDA_CONV build of the
// kern-k3-pp-prefill page, section "D: TP8 / EP8 / DCP8", which reads the
// window in SGLang's tap-major layout in its CONV_TAP_MAJOR variant, section
// "D inside SGLang"; here any layout the window strides describe).  One
// workgroup owns all d_v rows of a (sequence, head), so it alone reads and
// rewrites that window: each of the 2 d_k + d_v channels is convolved once
// (thread t takes channel t), rounded to the io dtype as the prefill pass does,
// and staged in LDS; the window shifts by one row; then the state rows are
// updated as in the plain step, reading k, q and v from LDS.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kConvStepThreads) void kda_decode_conv_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *pool,
    const int32_t *__restrict__ slots, E *__restrict__ o, int N, int H, int num_slots,
    float scale, int64_t slot_stride, int64_t head_stride, const float *__restrict__ weight,
    E *window, ConvWin win, int silu) {
    constexpr int C = 2 * DK + DV;
    constexpr int NT = kConvStepThreads;
    constexpr int CPT = (C + NT - 1) / NT;       // channels per thread
    constexpr int V4 = DK / 64;
    constexpr int RPI = NT / 16;
    constexpr int P = DV / RPI;                  // passes over all d_v rows
    static_assert(P >= 1 && DV % RPI == 0, "whole passes over the d_v rows");
    __shared__ float sX[C];
    const int tid = threadIdx.x;
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    if (n >= N) return;
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) return;   // padded row: touch nothing
    const int c = tid & 15, rr = tid >> 4;
    const size_t tok = (size_t)n * H + h;

    // token channels, window rows and taps (unconditional, clamped loads)
    E xr[CPT], wo[CPT][kConvWindow];
    float wt[CPT][kConvTaps];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = min(tid + NT * u, C - 1);
        const int part = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
        const int pc = ch - part * DK;
        xr[u] = part == 0 ? q[tok * DK + pc] : (part == 1 ? k[tok * DK + pc] : v[tok * DV + pc]);
#pragma unroll
        for (int i = 0; i < kConvWindow; ++i) wo[u][i] = window[win.at(slot, h, i, part, pc)];
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) wt[u][j] = weight[((size_t)h * kConvTaps + j) * C + ch];
    }
    f32x4 a4[V4];
#pragma unroll
    for (int x = 0; x < V4; ++x)
        a4[x] = *reinterpret_cast<const f32x4 *>(g + tok * DK + 4 * (c + 16 * x));
    const float bt = beta[tok];
    float *S = pool + slot * slot_stride + h * head_stride;
    f32x4 s[P][V4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = p * RPI + rr;
#pragma unroll
        for (int x = 0; x < V4; ++x)
            s[p][x] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
    }

#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = tid + NT * u;
        if (ch < C) {
            const int part = ch < DK ? 0 : (ch < 2 * DK ? 1 : 2);
            const int pc = ch - part * DK;
            sX[ch] = round_io<E>(conv_act(conv4(wt[u][0], wt[u][1], wt[u][2], wt[u][3],
                                                (float)wo[u][0], (float)wo[u][1], (float)wo[u][2],
                                                (float)xr[u]), silu));
            window[win.at(slot, h, 0, part, pc)] = wo[u][1];
            window[win.at(slot, h, 1, part, pc)] = wo[u][2];
            window[win.at(slot, h, 2, part, pc)] = xr[u];
        }
    }
    __syncthreads();

    f32x4 k4[V4], q4[V4];
#pragma unroll
    for (int x = 0; x < V4; ++x) {
        k4[x] = *reinterpret_cast<const f32x4 *>(&sX[DK + 4 * (c + 16 * x)]);
        q4[x] = *reinterpret_cast<const f32x4 *>(&sX[4 * (c + 16 * x)]);
        a4[x] = f32x4{decay_factor(a4[x][0]), decay_factor(a4[x][1]), decay_factor(a4[x][2]),
                      decay_factor(a4[x][3])};
    }
    const float kq = token_kq<V4>(k4, q4);
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = p * RPI + rr;
        float dq;
        const float d = row_update<V4>(s[p], a4, k4, q4, bt, sX[2 * DK + row], dq);
#pragma unroll
        for (int x = 0; x < V4; ++x)
            __builtin_nontemporal_store(s[p][x], reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
        if (c == 0) o[tok * DV + row] = (E)row_output(d, kq, dq, scale);
    }
}

// T tokens per sequence; token t of sequence n is row n T + t of q, k, v, g,
// beta and o.  The workgroup keeps its 64 state rows in registers for all T
// tokens; the tokens' k, q, decays e^g (taken once per element here, not
// once per lane) and beta and this part's v columns are staged once in LDS
// (fp32), and outputs are gathered in LDS and written as whole rows at the
// end.  With commit, the state after the first c tokens is
// written back (c = accept[n] clamped to [0, T], or T without accept; c = 0
// writes nothing).  o may be NULL (a commit that needs no outputs, q unused).
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_tokens_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *pool,
    const int32_t *__restrict__ slots, E *__restrict__ o, const int32_t *__restrict__ accept,
    int N, int T, int H, int num_slots, float scale, int commit, int64_t slot_stride,
    int64_t head_stride) {
    constexpr int PARTS = DV / kDecodeRows;
    constexpr int CPL = DK / 16;
    constexpr int V4 = CPL / 4;
    constexpr int RPI = 256 / 16;
    constexpr int P = kDecodeRows / RPI;
    constexpr int K4 = DK / 4;           // float4 per token row of k, q or g
    // dynamic LDS sized by T (decode_tokens_lds_bytes): k, q, decay rows,
    // then v columns, outputs and beta
    extern __shared__ f32x4 lds_tok[];
    f32x4 *__restrict__ sK = lds_tok;
    f32x4 *__restrict__ sQ = sK + T * K4;
    f32x4 *__restrict__ sG = sQ + T * K4;
    float *__restrict__ sV = reinterpret_cast<float *>(sG + T * K4);
    float *__restrict__ sO = sV + T * kDecodeRows;
    float *__restrict__ sB = sO + T * kDecodeRows;

    const int tid = threadIdx.x;
    const int part = blockIdx.x % PARTS;
    const int nh = blockIdx.x / PARTS;
    const int n = nh / H, h = nh % H;
    if (n >= N) return;
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) return;   // padded row: touch nothing
    int cn = 0;
    if (commit) {
        cn = accept ? accept[n] : T;
        cn = cn < 0 ? 0 : (cn > T ? T : cn);
    }
    const bool out = o != nullptr;
    if (!out && cn == 0) return;                 // nothing to compute or write
    const int c = tid & 15, rr = tid >> 4;
    float *S = pool + slot * slot_stride + h * head_stride;

    // The tokens' loads go out first, into registers, and the state's after
    // them: loads complete in order, so the LDS writes below wait only for
    // the token data while the state is still in flight.  The loads are
    // unconditional (indices clamped to the last element, q replaced by k
    // when there are no outputs) and keep the raw io values, so no branch or
    // conversion stands between them.
    using Raw4 = typename Raw4Of<E>::type;
    constexpr int ITK = (kMaxDecodeTokens * K4 + 255) / 256;
    constexpr int ITV = (kMaxDecodeTokens * kDecodeRows + 255) / 256;
    const size_t tok0 = (size_t)n * T;           // first row of this sequence
    const E *qs = out ? q : k;
    Raw4 rk[ITK], rq[ITK];
    f32x4 rg[ITK];
    E rv[ITV];
#pragma unroll
    for (int j = 0; j < ITK; ++j) {
        const int i = min(tid + 256 * j, T * K4 - 1);
        const int t = i / K4, c4 = i - t * K4;
        const size_t off = ((tok0 + t) * H + h) * DK + 4 * c4;
        rk[j] = *reinterpret_cast<const Raw4 *>(k + off);
        rq[j] = *reinterpret_cast<const Raw4 *>(qs + off);
        rg[j] = *reinterpret_cast<const f32x4 *>(g + off);
    }
#pragma unroll
    for (int j = 0; j < ITV; ++j) {
        const int i = min(tid + 256 * j, T * kDecodeRows - 1);
        const int t = i / kDecodeRows, r = i - t * kDecodeRows;
        rv[j] = v[((tok0 + t) * H + h) * DV + part * kDecodeRows + r];
    }
    const float rb = beta[(tok0 + min(tid, T - 1)) * H + h];

    f32x4 s[P][V4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int row = part * kDecodeRows + p * RPI + rr;
#pragma unroll
        for (int x = 0; x < V4; ++x)
            s[p][x] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
    }

#pragma unroll
    for (int j = 0; j < ITK; ++j) {
        const int i = tid + 256 * j;
        if (i < T * K4) {
            sK[i] = raw_to_f32(rk[j]);
            sQ[i] = out ? raw_to_f32(rq[j]) : f32x4{0.f, 0.f, 0.f, 0.f};
            sG[i] = f32x4{decay_factor(rg[j][0]), decay_factor(rg[j][1]),
                          decay_factor(rg[j][2]), decay_factor(rg[j][3])};
        }
    }
#pragma unroll
    for (int j = 0; j < ITV; ++j) {
        const int i = tid + 256 * j;
        if (i < T * kDecodeRows) sV[i] = (float)rv[j];
    }
    if (tid < T) sB[tid] = rb;
    __syncthreads();

    for (int t = 0; t < T; ++t) {
        f32x4 k4[V4], q4[V4], a4[V4];
        float vt[P], ot[P];
#pragma unroll
        for (int x = 0; x < V4; ++x) {
            k4[x] = sK[t * K4 + c + 16 * x];
            q4[x] = sQ[t * K4 + c + 16 * x];
            a4[x] = sG[t * K4 + c + 16 * x];
        }
#pragma unroll
        for (int p = 0; p < P; ++p) vt[p] = sV[t * kDecodeRows + p * RPI + rr];
        const float bt = sB[t];
        const float kq = token_kq<V4>(k4, q4);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float dq;
            const float d = row_update<V4>(s[p], a4, k4, q4, bt, vt[p], dq);
            ot[p] = row_output(d, kq, dq, scale);
        }
        if (c == 0) {
#pragma unroll
            for (int p = 0; p < P; ++p) sO[t * kDecodeRows + p * RPI + rr] = ot[p];
        }
        if (t + 1 == cn) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int row = part * kDecodeRows + p * RPI + rr;
#pragma unroll
                for (int x = 0; x < V4; ++x)
                    __builtin_nontemporal_store(s[p][x], reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * (c + 16 * x)));
            }
            if (!out) return;
        }
    }
    if (!out) return;
    __syncthreads();
    for (int i = tid; i < T * kDecodeRows; i += 256) {
        const int t = i / kDecodeRows, r = i - t * kDecodeRows;
        o[((tok0 + t) * H + h) * DV + part * kDecodeRows + r] = (E)sO[i];
    }
}

template <typename E, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    const int nblocks = a.N * a.H * (DV / kStepRows);
    kda_decode_kernel<E, DK, DV><<<dim3(nblocks), dim3(256), 0, stream>>>(
        static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
        a.g, a.beta, a.pool, a.slots, static_cast<E *>(a.o), a.N, a.H, a.num_slots, a.scale,
        a.slot_stride, a.head_stride);
    return hipGetLastError();
}

// LDS of the multi-token kernel for T tokens: k, q and decay rows (fp32),
// v columns and outputs of one 64-row part, beta.
constexpr size_t decode_tokens_lds_bytes(int T, int DK) {
    return (size_t)T * (3 * DK + 2 * kDecodeRows + 1) * sizeof(float);
}

template <typename E, int DK, int DV>
hipError_t launch_decode_tokens(const DecodeArgs &a, hipStream_t stream) {
    const int nblocks = a.N * a.H * (DV / kDecodeRows);
    const size_t lds = decode_tokens_lds_bytes(a.T, DK);
    kda_decode_tokens_kernel<E, DK, DV><<<dim3(nblocks), dim3(256), lds, stream>>>(
        static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
        a.g, a.beta, a.pool, a.slots, static_cast<E *>(a.o), a.accept, a.N, a.T, a.H,
        a.num_slots, a.scale, a.commit, a.slot_stride, a.head_stride);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_decode_conv(const DecodeArgs &a, const ConvArgs &c, hipStream_t stream) {
    kda_decode_conv_kernel<E, DK, DV><<<dim3(a.N * a.H), dim3(kConvStepThreads), 0, stream>>>(
        static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
        a.g, a.beta, a.pool, a.slots, static_cast<E *>(a.o), a.N, a.H, a.num_slots, a.scale,
        a.slot_stride, a.head_stride, c.weight, static_cast<E *>(c.window), c.win, c.silu);
    return hipGetLastError();
}

#define KDA_INST(E, DK, DV)                                                           \
    template hipError_t launch_decode<E, DK, DV>(const DecodeArgs &, hipStream_t);    \
    template hipError_t launch_decode_tokens<E, DK, DV>(const DecodeArgs &, hipStream_t); \
    template hipError_t launch_decode_conv<E, DK, DV>(const DecodeArgs &, const ConvArgs &, \
                                                      hipStream_t);
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
