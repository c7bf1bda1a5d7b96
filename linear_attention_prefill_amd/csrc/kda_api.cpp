// C ABI of libkda.so: host-side validation, workspace sizing and dispatch.
// Nothing here touches device memory or synchronises; every error is
// returned before the first launch.
#include "kda.h"
#include "kda_launch.h"

#ifndef KDA_CONV_FOLD
#define KDA_CONV_FOLD 1
#endif

#include <limits.h>

#include <atomic>

namespace {

using bf16 = __bf16;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_supported(int dk, int dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

template <typename E>
hipError_t dispatch_prefill(const kda::PrefillArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64 && dv == 64) return kda::launch_prefill<E, 64, 64>(a, s);
    if (dk == 64 && dv == 128) return kda::launch_prefill<E, 64, 128>(a, s);
    if (dk == 128 && dv == 64) return kda::launch_prefill<E, 128, 64>(a, s);
    return kda::launch_prefill<E, 128, 128>(a, s);
}

template <typename E>
hipError_t dispatch_decode(const kda::DecodeArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64 && dv == 64) return kda::launch_decode<E, 64, 64>(a, s);
    if (dk == 64 && dv == 128) return kda::launch_decode<E, 64, 128>(a, s);
    if (dk == 128 && dv == 64) return kda::launch_decode<E, 128, 64>(a, s);
    return kda::launch_decode<E, 128, 128>(a, s);
}

template <typename E>
hipError_t dispatch_decode_tokens(const kda::DecodeArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64 && dv == 64) return kda::launch_decode_tokens<E, 64, 64>(a, s);
    if (dk == 64 && dv == 128) return kda::launch_decode_tokens<E, 64, 128>(a, s);
    if (dk == 128 && dv == 64) return kda::launch_decode_tokens<E, 128, 64>(a, s);
    return kda::launch_decode_tokens<E, 128, 128>(a, s);
}

template <typename E>
hipError_t dispatch_conv_front(const kda::ConvArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64 && dv == 64) return kda::launch_conv_front<E, 64, 64>(a, s);
    if (dk == 64 && dv == 128) return kda::launch_conv_front<E, 64, 128>(a, s);
    if (dk == 128 && dv == 64) return kda::launch_conv_front<E, 128, 64>(a, s);
    return kda::launch_conv_front<E, 128, 128>(a, s);
}

template <typename E>
hipError_t dispatch_decode_conv(const kda::DecodeArgs &a, const kda::ConvArgs &c, int dk, int dv,
                                hipStream_t s) {
    if (dk == 64 && dv == 64) return kda::launch_decode_conv<E, 64, 64>(a, c, s);
    if (dk == 64 && dv == 128) return kda::launch_decode_conv<E, 64, 128>(a, c, s);
    if (dk == 128 && dv == 64) return kda::launch_decode_conv<E, 128, 64>(a, c, s);
    return kda::launch_decode_conv<E, 128, 128>(a, c, s);
}

// Compute units of the device a stream runs on (persistent grids are sized
// by it), queried once per device id.  The cache is the library's only
// process-wide state; it holds a hardware constant, so concurrent first calls
// store the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus(hipStream_t s) {
    int dev = 0;
    if (!s || hipStreamGetDevice(s, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) return 256;
    }
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 256;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Shape checks shared by the workspace query and the call.
kda_status_t check_desc(const kda_prefill_desc_t *d) {
    if (!d) return KDA_ERR_NULL;
    if (d->io_dtype != KDA_F32 && d->io_dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (!dims_supported(d->d_k, d->d_v)) return KDA_ERR_UNSUPPORTED;
    if (d->total_rows < 0 || d->num_seqs < 1 || d->num_heads < 1 || d->num_slots < 0)
        return KDA_ERR_SHAPE;
    if (d->conv_mode < KDA_CONV_NONE || d->conv_mode > KDA_CONV_SILU) return KDA_ERR_SHAPE;
    if (d->window_chunks < 0) return KDA_ERR_SHAPE;
    if (d->num_heads > 65535) return KDA_ERR_SHAPE;                       // grid.y of the window kernel
    const long long chunks = (long long)d->total_rows / 64 + d->num_seqs;
    if (chunks > INT_MAX) return KDA_ERR_SHAPE;
    if ((long long)d->num_seqs * d->num_heads * (d->d_v / 16) > INT_MAX) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Resolves the state strides (fp32 elements; 0 = dense) and checks the line
// rules of kda.h: multiples of 4 (16-byte rows), blocks of one line and lines
// of different slots never overlap.
bool resolve_strides(int64_t slot_stride, int64_t head_stride, int H, int dk, int dv,
                     int64_t *ss, int64_t *hs) {
    const int64_t block = (int64_t)dk * dv;
    *hs = head_stride ? head_stride : block;
    *ss = slot_stride ? slot_stride : (int64_t)H * *hs;
    if (*hs < block || *hs % 4) return false;
    if (*ss % 4 || *ss < (int64_t)(H - 1) * *hs + block) return false;
    return true;
}

// Resolves the conv window strides (io elements; 0 = dense head-major) and
// checks the rules of kda.h: multiples of 4 (8- or 16-byte rows), non-negative,
// q and k parts of a row apart by at least d_k.
bool resolve_conv(const kda_conv_t *c, int H, int dk, int dv, kda::ConvWin *w) {
    const int64_t C = 2 * (int64_t)dk + dv;
    w->ps = c->part_stride ? c->part_stride : dk;
    w->ts = c->row_stride ? c->row_stride : C;
    w->hs = c->head_stride ? c->head_stride : 3 * C;
    w->ss = c->slot_stride ? c->slot_stride : (int64_t)H * w->hs;
    const int64_t v[] = {w->ps, w->ts, w->hs, w->ss};
    for (int64_t x : v)
        if (x < 0 || x % 4) return false;
    return w->ps >= dk;
}

// Host checks shared by the conv entry points; fills the conv arguments that
// do not depend on the call's buffers.
kda_status_t check_conv(int mode, const kda_conv_t *conv, int H, int dk, int dv,
                        kda::ConvArgs *c) {
    if (mode < KDA_CONV_LINEAR || mode > KDA_CONV_SILU) return KDA_ERR_SHAPE;
    if (!conv || !conv->weight || !conv->window) return KDA_ERR_NULL;
    if (!aligned16(conv->weight) || !aligned16(conv->window)) return KDA_ERR_ALIGN;
    if (!resolve_conv(conv, H, dk, dv, &c->win)) return KDA_ERR_SHAPE;
    c->weight = conv->weight;
    c->window = conv->window;
    c->silu = mode == KDA_CONV_SILU;
    return KDA_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The conv runs folded into the intra-chunk kernel's loads for bf16 with
// d_k = d_v when no sequence is fused, else as a pass of its own that writes
// the convolved q, k, v into the workspace.
bool conv_folded(const kda_prefill_desc_t &d) {
    return d.conv_mode != KDA_CONV_NONE && d.io_dtype == KDA_BF16 && d.d_k == d.d_v && KDA_CONV_FOLD &&
           kda::prefill_fuse_max(d.total_rows, d.num_seqs, d.num_heads, true, d.fuse_chunks) < 0;
}

// workspace bytes of a valid desc: the records, and the convolved q, k, v
// when the conv runs as a pass of its own
size_t prefill_need(const kda_prefill_desc_t &d) {
    const bool bf = d.io_dtype == KDA_BF16;
    size_t n = kda::prefill_workspace_bytes(d.total_rows, d.num_seqs, d.num_heads, d.d_k, d.d_v, bf,
                                            d.window_chunks);
    if (d.conv_mode != KDA_CONV_NONE && !conv_folded(d))
        n += kda::conv_workspace_bytes(d.total_rows, d.num_heads, d.d_k, d.d_v, bf);
    return n;
}

kda_status_t prefill_impl(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const int32_t *cu_seqlens, const float *state_in,
                          float *state_out, void *o, const int32_t *slots,
                          const kda_prefill_desc_t *desc, const kda_conv_t *conv, bool with_conv,
                          void *workspace, size_t ws_bytes, void *stream, void *const *events,
                          int32_t num_events, bool static_ws = false) {
    const kda_status_t st = check_desc(desc);
    if (st != KDA_OK) return st;
    const kda_prefill_desc_t d = *desc;
    if (!with_conv && d.conv_mode != KDA_CONV_NONE) return KDA_ERR_NULL;
    if (with_conv && d.conv_mode == KDA_CONV_NONE) return KDA_ERR_SHAPE;
    if (!slots && (state_in || state_out) && d.num_slots < d.num_seqs) return KDA_ERR_SHAPE;
    // with no rows, no row input or output is touched
    if (!cu_seqlens) return KDA_ERR_NULL;
    if (d.total_rows > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    const bool bf = d.io_dtype == KDA_BF16;
    const size_t rec_bytes = kda::prefill_workspace_bytes(d.total_rows, d.num_seqs, d.num_heads,
                                                          d.d_k, d.d_v, bf, d.window_chunks);
    const size_t need = prefill_need(d);
    if (static_ws && need > KDA_STATIC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    if (need > 0 && !workspace && !static_ws) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, cu_seqlens, state_in, state_out, o, slots, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    kda::ConvArgs c{};
    if (with_conv) {
        const kda_status_t cs = check_conv(d.conv_mode, conv, d.num_heads, d.d_k, d.d_v, &c);
        if (cs != KDA_OK) return cs;
        if (((long long)d.total_rows / 64 + 1) * d.num_heads > INT_MAX) return KDA_ERR_SHAPE;
    }
    if (!static_ws && ws_bytes < need) return KDA_ERR_WORKSPACE;
    int64_t ss = 0, hs = 0;
    if (!resolve_strides(d.state_slot_stride, d.state_head_stride, d.num_heads, d.d_k, d.d_v, &ss, &hs))
        return KDA_ERR_SHAPE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (static_ws && need > 0 && kda::static_scratch(s, &workspace) != hipSuccess)
        return KDA_ERR_HIP;
    (void)hipGetLastError();       // an earlier call's error is not this call's
    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.cu_seqlens = cu_seqlens;
    const bool fold = with_conv && conv_folded(d);
    if (with_conv) {
        c.q = q; c.k = k; c.v = v;
        c.cu_seqlens = cu_seqlens; c.slots = slots;
        c.T = d.total_rows; c.N = d.num_seqs; c.H = d.num_heads; c.num_slots = d.num_slots;
        c.num_cus = device_cus(s);
    }
    if (fold) {
        a.conv = &c;
    } else if (with_conv) {
        const size_t es = bf ? 2 : 4;
        char *base = static_cast<char *>(workspace) + align256(rec_bytes);
        const size_t nq = align256((size_t)d.total_rows * d.num_heads * d.d_k * es);
        c.qc = base; c.kc = base + nq; c.vc = base + 2 * nq;
        const hipError_t e = bf ? dispatch_conv_front<bf16>(c, d.d_k, d.d_v, s)
                                : dispatch_conv_front<float>(c, d.d_k, d.d_v, s);
        if (e != hipSuccess) return KDA_ERR_HIP;
        a.q = c.qc; a.k = c.kc; a.v = c.vc;
    }
    a.state_in = state_in; a.state_out = state_out; a.o = o; a.slots = slots;
    a.workspace = workspace;
    a.T = d.total_rows; a.N = d.num_seqs; a.H = d.num_heads; a.num_slots = d.num_slots;
    a.scale = d.scale;
    a.slot_stride = ss;
    a.head_stride = hs;
    a.events = reinterpret_cast<const hipEvent_t *>(events);
    a.num_events = events ? num_events : 0;
    a.num_cus = device_cus(s);
    a.window_chunks = d.window_chunks;
    a.fuse_chunks = d.fuse_chunks;
    const hipError_t e = bf ? dispatch_prefill<bf16>(a, d.d_k, d.d_v, s)
                            : dispatch_prefill<float>(a, d.d_k, d.d_v, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t decode_impl(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state_pool, const int32_t *slots, void *o,
                         int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v,
                         int32_t num_slots, int32_t io_dtype, float scale,
                         int64_t state_slot_stride, int64_t state_head_stride, int32_t conv_mode,
                         const kda_conv_t *conv, void *stream) {
    if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (!dims_supported(d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 1 || num_heads < 1 || num_slots < 1) return KDA_ERR_SHAPE;
    if ((long long)num_seqs * num_heads * (d_v / 16) > INT_MAX) return KDA_ERR_SHAPE;   // grid of the step
    if (!q || !k || !v || !g || !beta || !state_pool || !slots || !o) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, state_pool, slots, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    kda::ConvArgs c{};
    if (conv_mode != KDA_CONV_NONE) {
        const kda_status_t cs = check_conv(conv_mode, conv, num_heads, d_k, d_v, &c);
        if (cs != KDA_OK) return cs;
    }
    int64_t ss = 0, hs = 0;
    if (!resolve_strides(state_slot_stride, state_head_stride, num_heads, d_k, d_v, &ss, &hs))
        return KDA_ERR_SHAPE;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.pool = state_pool; a.slots = slots;
    a.o = o; a.N = num_seqs; a.H = num_heads; a.num_slots = num_slots; a.scale = scale;
    a.slot_stride = ss;
    a.head_stride = hs;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = io_dtype == KDA_BF16;
    (void)hipGetLastError();       // an earlier call's error is not this call's
    hipError_t e;
    if (conv_mode != KDA_CONV_NONE)
        e = bf ? dispatch_decode_conv<bf16>(a, c, d_k, d_v, s)
               : dispatch_decode_conv<float>(a, c, d_k, d_v, s);
    else
        e = bf ? dispatch_decode<bf16>(a, d_k, d_v, s) : dispatch_decode<float>(a, d_k, d_v, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t kda_prefill_windows(const kda_prefill_desc_t *desc) {
    if (check_desc(desc) != KDA_OK) return 0;
    const int fm = kda::prefill_fuse_max(desc->total_rows, desc->num_seqs, desc->num_heads,
                                         desc->io_dtype == KDA_BF16, desc->fuse_chunks);
    if (fm >= 0 && (long long)fm * 64 >= desc->total_rows) return 0;   // every sequence fused
    return kda::prefill_plan(desc->total_rows, desc->num_seqs, desc->num_heads, desc->d_k,
                             desc->d_v, desc->io_dtype == KDA_BF16, desc->window_chunks).windows;
}

int32_t kda_prefill_fuse_chunks(const kda_prefill_desc_t *desc) {
    if (check_desc(desc) != KDA_OK) return -1;
    return kda::prefill_fuse_max(desc->total_rows, desc->num_seqs, desc->num_heads,
                                 desc->io_dtype == KDA_BF16, desc->fuse_chunks);
}

size_t kda_prefill_workspace_size(const kda_prefill_desc_t *desc) {
    if (check_desc(desc) != KDA_OK) return 0;
    return prefill_need(*desc);
}

kda_status_t kda_chunk_prefill_timed(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta,
                                     const int32_t *cu_seqlens, const float *state_in,
                                     float *state_out, void *o, const int32_t *slots,
                                     const kda_prefill_desc_t *desc, void *workspace,
                                     size_t ws_bytes, void *stream, void *const *events,
                                     int32_t num_events) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, slots, desc, nullptr,
                        false, workspace, ws_bytes, stream, events, num_events);
}

kda_status_t kda_chunk_prefill_conv(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const int32_t *cu_seqlens,
                                    const float *state_in, float *state_out, void *o,
                                    const int32_t *slots, const kda_prefill_desc_t *desc,
                                    const kda_conv_t *conv, void *workspace, size_t ws_bytes,
                                    void *stream, void *const *events, int32_t num_events) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, slots, desc, conv,
                        true, workspace, ws_bytes, stream, events, num_events);
}

kda_status_t kda_chunk_prefill_static(const void *q, const void *k, const void *v,
                                      const float *g, const float *beta,
                                      const int32_t *cu_seqlens, const float *state_in,
                                      float *state_out, void *o, const int32_t *slots,
                                      const kda_prefill_desc_t *desc, void *stream) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, slots, desc, nullptr,
                        false, nullptr, 0, stream, nullptr, 0, true);
}

kda_status_t kda_chunk_prefill(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens,
                               const float *state_in, float *state_out, void *o,
                               const int32_t *slots, const kda_prefill_desc_t *desc,
                               void *workspace, size_t ws_bytes, void *stream) {
    return kda_chunk_prefill_timed(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, slots,
                                   desc, workspace, ws_bytes, stream, nullptr, 0);
}

kda_status_t kda_decode_step_lines(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, float *state_pool, const int32_t *slots,
                                   void *o, int32_t num_seqs, int32_t num_heads, int32_t d_k,
                                   int32_t d_v, int32_t num_slots, int32_t io_dtype, float scale,
                                   int64_t state_slot_stride, int64_t state_head_stride,
                                   void *stream) {
    return decode_impl(q, k, v, g, beta, state_pool, slots, o, num_seqs, num_heads, d_k, d_v,
                       num_slots, io_dtype, scale, state_slot_stride, state_head_stride,
                       KDA_CONV_NONE, nullptr, stream);
}

kda_status_t kda_decode_step_conv(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state_pool, const int32_t *slots,
                                  void *o, int32_t num_seqs, int32_t num_heads, int32_t d_k,
                                  int32_t d_v, int32_t num_slots, int32_t io_dtype, float scale,
                                  int64_t state_slot_stride, int64_t state_head_stride,
                                  int32_t conv_mode, const kda_conv_t *conv, void *stream) {
    if (conv_mode == KDA_CONV_NONE) return KDA_ERR_SHAPE;
    return decode_impl(q, k, v, g, beta, state_pool, slots, o, num_seqs, num_heads, d_k, d_v,
                       num_slots, io_dtype, scale, state_slot_stride, state_head_stride,
                       conv_mode, conv, stream);
}

kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *state_pool, const int32_t *slots, void *o,
                             int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v,
                             int32_t num_slots, int32_t io_dtype, float scale, void *stream) {
    return kda_decode_step_lines(q, k, v, g, beta, state_pool, slots, o, num_seqs, num_heads, d_k,
                                 d_v, num_slots, io_dtype, scale, 0, 0, stream);
}

kda_status_t kda_decode_tokens(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *state_pool, const int32_t *slots,
                               void *o, const int32_t *num_accepted, int32_t num_seqs,
                               int32_t num_tokens, int32_t num_heads, int32_t d_k, int32_t d_v,
                               int32_t num_slots, int32_t io_dtype, float scale, int32_t commit,
                               int64_t state_slot_stride, int64_t state_head_stride,
                               void *stream) {
    if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (!dims_supported(d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 1 || num_heads < 1 || num_slots < 1) return KDA_ERR_SHAPE;
    if (num_tokens < 1 || num_tokens > kda::kMaxDecodeTokens) return KDA_ERR_SHAPE;
    if ((long long)num_seqs * num_heads * (d_v / 64) > INT_MAX) return KDA_ERR_SHAPE;
    if ((long long)num_seqs * num_tokens * num_heads > INT_MAX) return KDA_ERR_SHAPE;
    if (!k || !v || !g || !beta || !state_pool || !slots) return KDA_ERR_NULL;
    if (!o && !commit) return KDA_ERR_NULL;      // neither outputs nor a commit
    if (o && !q) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, state_pool, slots, o, num_accepted};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    int64_t ss = 0, hs = 0;
    if (!resolve_strides(state_slot_stride, state_head_stride, num_heads, d_k, d_v, &ss, &hs))
        return KDA_ERR_SHAPE;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.pool = state_pool; a.slots = slots;
    a.o = o; a.N = num_seqs; a.H = num_heads; a.num_slots = num_slots; a.scale = scale;
    a.slot_stride = ss;
    a.head_stride = hs;
    a.T = num_tokens;
    a.accept = num_accepted;
    a.commit = commit ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();       // an earlier call's error is not this call's
    const hipError_t e = io_dtype == KDA_BF16 ? dispatch_decode_tokens<bf16>(a, d_k, d_v, s)
                                              : dispatch_decode_tokens<float>(a, d_k, d_v, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_prefill_check(const float *g, const int32_t *cu_seqlens, const int32_t *slots,
                               const kda_prefill_desc_t *desc, int32_t *flags, void *stream) {
    const kda_status_t st = check_desc(desc);
    if (st != KDA_OK) return st;
    if (!cu_seqlens || !flags) return KDA_ERR_NULL;
    if (desc->total_rows > 0 && !g) return KDA_ERR_NULL;
    const void *ptrs[] = {g, cu_seqlens, slots, flags};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    (void)hipGetLastError();       // an earlier call's error is not this call's
    const hipError_t e = kda::launch_prefill_check(g, cu_seqlens, slots, desc->total_rows,
                                                   desc->num_seqs, desc->num_heads, desc->d_k,
                                                   desc->num_slots, flags,
                                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char *kda_status_string(kda_status_t status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "a size is out of range";
        case KDA_ERR_DTYPE: return "unknown io dtype";
        case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_UNSUPPORTED:
            return "unsupported: d_k and d_v must be 64 or 128 (phase clocks: a library built with "
                   "KDA_PHASE_CLOCKS)";
        case KDA_ERR_HIP: return "a HIP kernel launch failed";
        case KDA_ERR_TOO_LARGE:
            return "the call needs more workspace than the static scratch holds "
                   "(KDA_STATIC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

static_assert(KDA_CLOCK_WAVES == kda::kClockWaves && KDA_CLOCK_ITEMS == kda::kClockItems &&
                  KDA_CLOCK_MARKS == kda::kClockMarks,
              "phase clock layout");

kda_status_t kda_phase_clocks(int32_t kernel, uint64_t *host_out, size_t count, int32_t clear) {
    if (kernel != KDA_CLOCK_INTRA && kernel != KDA_CLOCK_FUSED && kernel != KDA_CLOCK_SCAN)
        return KDA_ERR_SHAPE;
    static_assert(sizeof(uint64_t) == sizeof(unsigned long long), "clock words");
    const hipError_t e = kda::phase_clocks_copy(kernel, reinterpret_cast<unsigned long long *>(host_out),
                                                host_out ? count : 0, clear != 0);
    if (e == hipErrorNotSupported) return KDA_ERR_UNSUPPORTED;
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes, int32_t grid,
                              void *stream) {
    if (mode < KDA_STREAM_READ || mode > KDA_STREAM_UPDATE || grid < 1 || bytes % 16 != 0)
        return KDA_ERR_SHAPE;
    if (!dst || (mode != KDA_STREAM_UPDATE && !src)) return KDA_ERR_NULL;
    if (!aligned16(dst) || (src && !aligned16(src))) return KDA_ERR_ALIGN;
    if (bytes == 0) return KDA_OK;
    (void)hipGetLastError();       // an earlier call's error is not this call's
    const hipError_t e =
        kda::launch_stream_probe(mode, src, dst, bytes, grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_mfma_probe(int32_t chains, int32_t iters, uint64_t *out, void *stream) {
    if ((chains != 1 && chains != 2 && chains != 4 && chains != 8) || iters < 1 || iters > (1 << 20))
        return KDA_ERR_SHAPE;
    if (!out) return KDA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(out) % 8 != 0) return KDA_ERR_ALIGN;
    (void)hipGetLastError();       // an earlier call's error is not this call's
    const hipError_t e = kda::launch_mfma_probe(chains, iters, reinterpret_cast<unsigned long long *>(out),
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int32_t kda_version(void) { return 109; }

}  // extern "C"
