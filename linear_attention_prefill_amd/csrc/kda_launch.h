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
    hipEvent_t events[3];   // optional: before intra, between, after scan
};

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

template <typename E, int DK, int DV>
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

template <typename E, int DK, int DV>
hipError_t launch_decode_tokens(const DecodeArgs &a, hipStream_t stream);

size_t prefill_workspace_bytes(int T, int N, int H, int dk, int dv, bool bf16);

}  // namespace kda
