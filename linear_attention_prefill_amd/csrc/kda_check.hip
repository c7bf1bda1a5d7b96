// Opt-in check of the prefill's device-side preconditions.
//
// The prefill validates everything the host can see before it launches, but
// not the contents of device buffers: that would need a host sync, which the
// varlen path avoids (the prhub report on SGLang PR #32890, section
// "关键文件": the varlen inputs are prepared on the GPU to remove a GPU->CPU
// stall).  The "kern" page, section "The manifest", rejects a call outside its
// bounds before it launches; this check gives a caller the same guarantee for
// the device data, when it is willing to pay a pass over g and a read-back.
// It reads only inside the buffers the descriptor sizes, so malformed data is
// reported, never acted on.
#include "kda.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

__global__ void kda_check_clear_kernel(int32_t *flags) {
    if (threadIdx.x == 0) *flags = 0;
}

// Grid-stride over the g elements (four at a time; g is 16-byte aligned and
// d_k a multiple of 4), the cu_seqlens entries and the pairs of sequences.
__global__ __launch_bounds__(256) void kda_check_kernel(const float *__restrict__ g,
                                                        const int32_t *__restrict__ cu,
                                                        const int32_t *__restrict__ slots, int T,
                                                        int N, int H, int dk, int num_slots,
                                                        int32_t *flags) {
    int bits = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t ng4 = (size_t)T * H * dk / 4;
    for (size_t i = t0; i < ng4; i += stride) {
        const f32x4 x = reinterpret_cast<const f32x4 *>(g)[i];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (!(x[r] <= 0.f)) bits |= KDA_CHECK_G;      // positive or NaN
    }
    for (size_t i = t0; i <= (size_t)N; i += stride) {
        const int c = cu[i];
        if (i == 0 && c != 0) bits |= KDA_CHECK_CU_SEQLENS;
        if (i == (size_t)N && c != T) bits |= KDA_CHECK_CU_SEQLENS;
        if (i > 0 && c < cu[i - 1]) bits |= KDA_CHECK_CU_SEQLENS;
    }
    if (slots && N <= kCheckMaxPairsSeqs) {
        for (size_t p = t0; p < (size_t)N * N; p += stride) {
            const int a = (int)(p / N), b = (int)(p % N);
            if (a < b) {
                const int sa = slots[a];
                if (sa >= 0 && sa < num_slots && sa == slots[b]) bits |= KDA_CHECK_SLOTS;
            }
        }
    }
    if (bits) atomicOr(flags, bits);
}

hipError_t launch_prefill_check(const float *g, const int32_t *cu, const int32_t *slots, int T,
                                int N, int H, int dk, int num_slots, int32_t *flags,
                                hipStream_t stream) {
    kda_check_clear_kernel<<<dim3(1), dim3(64), 0, stream>>>(flags);
    const size_t pairs = N <= kCheckMaxPairsSeqs ? (size_t)N * N : 0;
    const size_t work = (size_t)T * H * dk / 4 + pairs + N + 1;
    const size_t blocks = (work + 255) / 256;
    const int grid = (int)(blocks < 4096 ? blocks : 4096);
    kda_check_kernel<<<dim3(grid), dim3(256), 0, stream>>>(g, cu, slots, T, N, H, dk, num_slots,
                                                           flags);
    return hipGetLastError();
}

}  // namespace kda
