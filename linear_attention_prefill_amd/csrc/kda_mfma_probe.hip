// Matrix-core issue probe: how fast one wave issues bf16 16x16x32 products
// back to back on this chip, with 1, 2, 4 or 8 independent accumulators.
// With one accumulator every product waits for the one before (the
// dependent latency); with enough of them the rate is the matrix core's
// throughput.  The prefill kernels' products are held against these rates.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kProbeThreads = 256;   // one wave per SIMD

template <int CHAINS>
__global__ __launch_bounds__(kProbeThreads) void kda_mfma_probe_kernel(unsigned long long *__restrict__ out,
                                                                       int iters) {
    const int tid = threadIdx.x, wave = tid >> 6;
    // operands from the thread index and the trip count, so that nothing
    // folds; the products stay because their sum can reach the store below
    Frag<bf16> a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a.set(i, 1e-3f * (float)(tid + i));
        b.set(i, 1e-3f * (float)(iters + i));
    }
    f32x4 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) mma(acc[c], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if ((tid & 63) == 0) {
        out[2 * wave] = t1 - t0;
        out[2 * wave + 1] = r1 - r0;
    }
    if (s == 1234.5f) out[8 + wave] = 1;       // never, for data this small
}

}  // namespace

hipError_t launch_mfma_probe(int chains, int iters, unsigned long long *out, hipStream_t stream) {
    const dim3 g(1), b(kProbeThreads);
    if (chains == 1) kda_mfma_probe_kernel<1><<<g, b, 0, stream>>>(out, iters);
    else if (chains == 2) kda_mfma_probe_kernel<2><<<g, b, 0, stream>>>(out, iters);
    else if (chains == 4) kda_mfma_probe_kernel<4><<<g, b, 0, stream>>>(out, iters);
    else kda_mfma_probe_kernel<8><<<g, b, 0, stream>>>(out, iters);
    return hipGetLastError();
}

}  // namespace kda
