// Plain streaming kernels: the bandwidth a read, a copy or an in-place update
// of a large buffer reaches on this chip, the practical ceiling that the
// prefill and decode kernels' HBM rates are held against.  Grid-stride loops
// over 16-byte nontemporal accesses, four in flight per thread.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

// mode 0: read src (XOR-folded, written to sink only if it hits a value the
// caller's data never folds to, so the loads stay); 1: copy src -> dst;
// 2: dst *= 1.0001 in place (fp32)
template <int MODE>
__global__ __launch_bounds__(kStreamThreads) void kda_stream_kernel(const u32x4v *__restrict__ src,
                                                                    u32x4v *__restrict__ dst, size_t n,
                                                                    uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kStreamThreads;
    size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    u32x4v acc = {0u, 0u, 0u, 0u};
    for (; i + (kStreamUnroll - 1) * stride < n; i += kStreamUnroll * stride) {
        u32x4v x[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            x[u] = __builtin_nontemporal_load(MODE == 2 ? dst + i + u * stride : src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            if constexpr (MODE == 0) {
                acc ^= x[u];
            } else if constexpr (MODE == 1) {
                __builtin_nontemporal_store(x[u], dst + i + u * stride);
            } else {
                const f32x4v y = __builtin_bit_cast(f32x4v, x[u]) * 1.0001f;
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, y), dst + i + u * stride);
            }
        }
    }
    for (; i < n; i += stride) {
        const u32x4v x = __builtin_nontemporal_load(MODE == 2 ? dst + i : src + i);
        if constexpr (MODE == 0) {
            acc ^= x;
        } else if constexpr (MODE == 1) {
            __builtin_nontemporal_store(x, dst + i);
        } else {
            const f32x4v y = __builtin_bit_cast(f32x4v, x) * 1.0001f;
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, y), dst + i);
        }
    }
    if constexpr (MODE == 0) {
        const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
        if (f == 0x9e3779b9u) sink[blockIdx.x] = f;
    }
}

}  // namespace

hipError_t launch_stream_probe(int mode, const void *src, void *dst, size_t bytes, int grid,
                               hipStream_t stream) {
    const size_t n = bytes / 16;
    const dim3 g(grid), b(kStreamThreads);
    auto *s = static_cast<const u32x4v *>(src);
    auto *d = static_cast<u32x4v *>(dst);
    if (mode == 0)
        kda_stream_kernel<0><<<g, b, 0, stream>>>(s, nullptr, n, static_cast<uint32_t *>(dst));
    else if (mode == 1)
        kda_stream_kernel<1><<<g, b, 0, stream>>>(s, d, n, nullptr);
    else
        kda_stream_kernel<2><<<g, b, 0, stream>>>(nullptr, d, n, nullptr);
    return hipGetLastError();
}

}  // namespace kda
