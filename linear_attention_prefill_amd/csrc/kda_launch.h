// Internal launch interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    const float *state_in;
    float *state_out;
    void *o;
    const int32_t *slots;
    void *workspace;
    int T, N, H, num_slots;
    float scale;
    int64_t slot_stride, head_stride;   // state addressing, fp32 elements (resolved)
    int num_cus;            // compute units of the device (persistent grids)
    int window_chunks = 0;  // chunk ids per window; 0 = the default policy
    int fuse_chunks = 0;    // fused prefill for sequences of <= this many chunks; 0 = default, < 0 none
    // optional timing events: [0] before the first kernel, then one after
    // each kernel launch (intra and scan of each window in turn)
    const hipEvent_t *events = nullptr;
    int num_events = 0;
    // the short conv folded into the intra-chunk kernel (bf16, d_k = d_v,
    // no fused prefill): q, k, v are the raw inputs; the windows are updated
    // after the intra-chunk launches
    const struct ConvArgs *conv = nullptr;
};

// How a prefill call splits into windows of chunk ids and lays out its
// workspace: window_chunks x H records (w, Q e^Gam, K~^T, A_qk, u in the io
// type), then the decay factors e^{Gam_C} (fp32), then, when there is more
// than one window, the states carried between windows ([N][H][d_v][d_k]
// fp32).
struct PrefillPlan {
    int chunk_ids;          // chunk_id_count(T, N): (T - 1) / 64 + N
    int windows;
    int window_chunks;
    size_t dec_offset, carry_offset, bytes;
};
PrefillPlan prefill_plan(int T, int N, int H, int dk, int dv, bool bf16, int window_chunks);
// Most chunks of a sequence the fused prefill takes (-1: none).
int prefill_fuse_max(int T, int N, int H, bool bf16, int fuse_chunks);

// Most tokens a multi-token decode call may carry per sequence.
constexpr int kMaxDecodeTokens = 16;

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *pool;
    const int32_t *slots;
    void *o;
    int N, H, num_slots;
    float scale;
    int64_t slot_stride, head_stride;   // state addressing, fp32 elements (resolved)
    int T = 1;                          // tokens per sequence (multi-token decode)
    const int32_t *accept = nullptr;    // tokens to commit per sequence, or NULL = T
    int commit = 1;                     // 0: state is only read
};

// Conv window addressing: row i of (slot, head), part p (0 q, 1 k, 2 v),
// channel c is element slot*ss + head*hs + i*ts + p*ps + c of the window
// pool (io dtype elements).
struct ConvWin {
    int64_t ss, hs, ts, ps;
    __host__ __device__ __forceinline__ int64_t at(int slot, int h, int i, int p, int c) const {
        return (int64_t)slot * ss + (int64_t)h * hs + (int64_t)i * ts + (int64_t)p * ps + c;
    }
};

// Short conv front end: raw q, k, v in, convolved q, k, v out (prefill).
struct ConvArgs {
    const void *q, *k, *v;          // raw inputs
    void *qc, *kc, *vc;             // convolved outputs (prefill)
    const int32_t *cu_seqlens;
    const int32_t *slots;
    const float *weight;            // [H][4][2 d_k + d_v]
    void *window;
    ConvWin win;
    int T, N, H, num_slots;
    int silu;
    int num_cus = 0;                // compute units of the device (persistent grid)
};

template <typename E, int DK, int DV>
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_conv_front(const ConvArgs &a, hipStream_t stream);

// Only the window update of the conv front end (the conv itself folded into
// the intra-chunk kernel).
template <typename E, int DK, int DV>
hipError_t launch_conv_window(const ConvArgs &a, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_decode_conv(const DecodeArgs &a, const ConvArgs &c, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_decode_tokens(const DecodeArgs &a, hipStream_t stream);

// Opt-in check of the prefill's device data (kda_prefill_check): clears
// *flags, then ORs in a KDA_CHECK_* bit per violated precondition.
constexpr int kCheckMaxPairsSeqs = 4096;   // duplicate slots looked for up to this N
hipError_t launch_prefill_check(const float *g, const int32_t *cu, const int32_t *slots, int T,
                                int N, int H, int dk, int num_slots, int32_t *flags,
                                hipStream_t stream);

// Phase clocks of the intra-chunk, fused and scan kernels (kda_phase_clocks):
// workgroup 0's waves record the core clock counter at each phase boundary
// of their first kClockItems items (scan: steps), in a library built with
// KDA_PHASE_CLOCKS; other builds return hipErrorNotSupported.
constexpr int kClockKernels = 3, kClockWaves = 8, kClockItems = 64, kClockMarks = 16;
hipError_t phase_clocks_copy(int kernel, unsigned long long *host, size_t count, bool clear);

// Streaming bandwidth probe (kda_stream_probe): mode 0 reads src (dst: a
// sink of 4 grid bytes), 1 copies src to dst, 2 scales dst in place.
hipError_t launch_stream_probe(int mode, const void *src, void *dst, size_t bytes, int grid,
                               hipStream_t stream);
// One workgroup of 4 waves issuing bf16 16x16x32 products on `chains`
// (1, 2, 4 or 8) independent accumulators, `iters` rounds; out: 12 words.
hipError_t launch_mfma_probe(int chains, int iters, unsigned long long *out, hipStream_t stream);

// Device address of the static scratch that backs kda_chunk_prefill_static
// on the device `stream` runs on (looked up on the first call per device).
hipError_t static_scratch(hipStream_t stream, void **ptr);

size_t prefill_workspace_bytes(int T, int N, int H, int dk, int dv, bool bf16, int window_chunks);

// Workspace bytes of the convolved q, k, v (placed after the records).
size_t conv_workspace_bytes(int T, int H, int dk, int dv, bool bf16);

}  // namespace kda
