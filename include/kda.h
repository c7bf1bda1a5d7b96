/*
 * kda.h - C ABI of the MI355X (gfx950) KDA library, libkda.so.
 *
 * KDA (Kimi Delta Attention) is the linear-attention layer whose per-sequence
 * recurrent state the kern runtime keeps as a fixed slot ("kern" page,
 * section "The manifest": a state declared by bytes per sequence and handed
 * out as slots from one pool).  Per (sequence, head) the state S is a
 * d_k x d_v fp32 matrix and each token t updates it by the gated delta rule
 * with a per-key-channel decay:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * The pages name the layer without writing this update; the form above is the
 * plainest reading and the one the fp64 test oracle implements.
 *
 * Memory layouts (row-major, element strides implied, no padding):
 *   q, k      [T][H][d_k]   io dtype (bf16 or fp32)
 *   v, o      [T][H][d_v]   io dtype
 *   g         [T][H][d_k]   fp32, natural-log decay per key channel, g <= 0
 *   beta      [T][H]        fp32
 *   state     [num_slots][H][d_v][d_k] fp32: element (slot, h, j, i) holds
 *             S[i][j], the "[slot][head][v][k] f32" layout of the
 *             kern-k3-pp-prefill page, section "D inside SGLang".
 *   cu_seqlens [N+1] int32 on the device: sequence n owns rows
 *             cu_seqlens[n] .. cu_seqlens[n+1]-1 (the packed prefill of the
 *             same page, section "P: the packed prefill": up to 16 sequences
 *             back to back, split by cu_seqlens).
 *   slots     [N] int32 on the device, or NULL for slot n = n.
 *
 * Ownership and execution.  The caller owns every buffer, including the
 * workspace; the library allocates nothing and caches no tensors.  Its only
 * process-wide state is a per-device cache of the compute-unit count, which
 * sizes the persistent grids.  Every call validates its arguments on the host and
 * returns a status before anything is launched; then it enqueues its kernels
 * on `stream` (a hipStream_t; NULL is the null stream) and returns without
 * synchronising.  It never reads device memory on the host, so a call can be
 * captured into a HIP graph (the "kern" page, section "Hosts": launches
 * enqueue on the host's stream, inside its graphs).  All pointers are device
 * pointers and must be 16-byte aligned.
 *
 * Device data is not validated on the host (that would need a sync).  The
 * kernels clamp it so that no access leaves the buffers: cu_seqlens entries
 * are clamped to [0, T] and each sequence to [cu[n], T]; a slot outside
 * [0, num_slots) marks a padded sequence.  Results for non-monotone
 * cu_seqlens or duplicate slots are unspecified.  kda_prefill_check tests
 * these preconditions, and g <= 0, on the device when a caller asks for it.
 *
 * g <= 0 (a decaying state) is a precondition of the prefill's split decay
 * factors, which never exceed 1 under it.  With some g > 0 the same
 * factoring runs with factors above 1: a state that grows by at most a few
 * e-folds per 64-row chunk is computed to the usual accuracy (a GPU test
 * covers g up to +0.02), while a chunk whose cumulative growth of a channel
 * passes about 2^64 can overflow and gives unspecified results.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,       /* a size is out of range */
    KDA_ERR_DTYPE = 3,       /* unknown io dtype */
    KDA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    KDA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    KDA_ERR_UNSUPPORTED = 6, /* d_k or d_v not 64 or 128; phase clocks not built in */
    KDA_ERR_HIP = 7,         /* a kernel launch failed */
    KDA_ERR_TOO_LARGE = 8    /* the call needs more than the static scratch holds */
} kda_status_t;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/*
 * State addressing by lines.  The state block of (slot s, head h) is the dense
 * [d_v][d_k] fp32 block at
 *     pool + s * state_slot_stride + h * state_head_stride     (fp32 elements)
 * so a state pool can live inside an engine's own pages: a KDA line at the
 * start of each page, with other per-head data (a conv window) between the
 * heads ("kern-k3-pp-prefill" page, section "D inside vLLM": vLLM's hybrid
 * pages hold one KDA line at the start of each page, and the kernel's line
 * stride is the one launch parameter that changes).  A stride of 0 selects
 * the dense [num_slots][H][d_v][d_k] layout (slot stride H d_v d_k, head
 * stride d_v d_k).  Given strides must be multiples of 4 with
 * state_head_stride >= d_v d_k and
 * state_slot_stride >= (H - 1) state_head_stride + d_v d_k, so no two blocks
 * overlap; the pool must hold (num_slots - 1) slot strides plus one line.
 */

/*
 * Short conv front end.  On the prefill side of the kern-k3-pp-prefill page
 * every sequence carries a conv window next to its recurrent state (section
 * "P: the packed prefill"), its decode build fuses the conv into the step (section "D:
 * TP8 / EP8 / DCP8"), and SGLang keeps the window as [slot][tap][q | k | v]
 * bf16 (section "D inside SGLang").  The "kern" page's KDA state of
 * 19,537,920 bytes a sequence (section "The manifest") is 288 blocks of a
 * 64 KiB state plus 3 x 3 x 128 bf16, so the window holds 3 rows.  Reading
 * taken here: per head, the channels x = [q | k | v] (2 d_k + d_v of them)
 * pass through a causal per-channel conv of width 4,
 *     y_t = w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t,
 * whose three older inputs at a sequence's start come from its window; an
 * optional SiLU follows; y, rounded to the io dtype, replaces q, k and v for
 * the rest of the step.  After the call each live sequence's window holds its
 * last three raw inputs (older window rows shift in for sequences shorter
 * than three rows; a zero-length sequence leaves it as it was).  A padded
 * sequence (slot out of range) convolves from zeros and touches no window.
 */
typedef enum { KDA_CONV_NONE = 0, KDA_CONV_LINEAR = 1, KDA_CONV_SILU = 2 } kda_conv_mode_t;

typedef struct {
    const float *weight;  /* [H][4][2 d_k + d_v] fp32: tap j multiplies x_{t-3+j} */
    void *window;         /* raw inputs, io dtype, read and rewritten in place */
    /* Row i (0 = oldest) of (slot s, head h), part p (0 q, 1 k, 2 v), channel c
     * is element s*slot + h*head + i*row + p*part + c of `window`.  Zeros give
     * the dense [num_slots][H][3][2 d_k + d_v] layout (part = d_k, row =
     * 2 d_k + d_v, head = 3 row, slot = H head).  SGLang's tap-major
     * [slot][tap][q | k | v] is slot = 3 row, row = H (2 d_k + d_v),
     * part = H d_k, head = d_k (this needs d_k = d_v).  Given strides must be
     * multiples of 4 with part >= d_k; the caller keeps the addressed rows
     * from overlapping. */
    int64_t slot_stride, head_stride, row_stride, part_stride;
} kda_conv_t;

/* Sizes of one prefill call.  T = total_rows, N = num_seqs, H = num_heads. */
typedef struct {
    int32_t total_rows;  /* T >= 0 */
    int32_t num_seqs;    /* N >= 1 */
    int32_t num_heads;   /* H >= 1 */
    int32_t d_k;         /* 64 or 128 */
    int32_t d_v;         /* 64 or 128 */
    int32_t num_slots;   /* rows of the state pools (the slot index space) */
    int32_t io_dtype;    /* kda_dtype_t of q, k, v and o */
    float scale;         /* multiplies o only */
    int64_t state_slot_stride;  /* fp32 elements between slots' lines; 0 = dense */
    int64_t state_head_stride;  /* fp32 elements between heads of a line; 0 = dense */
    int32_t conv_mode;   /* kda_conv_mode_t; not NONE only with kda_chunk_prefill_conv */
    int32_t window_chunks;  /* chunk ids per window (kda_prefill_windows); 0 = the library's choice */
    int32_t fuse_chunks;    /* bf16: sequences of at most this many 64-row chunks run in the fused
                             * prefill (kda_prefill_fuse_chunks); 0 = the library's choice,
                             * < 0 = none */
} kda_prefill_desc_t;

/*
 * Number of windows of chunk ids a prefill call with `desc` runs as (0 if
 * desc is invalid, or if every sequence runs in the fused prefill because
 * kda_prefill_fuse_chunks(desc) * 64 >= total_rows): each window is an
 * intra-chunk kernel that writes the records of its chunks into the
 * workspace and a state scan that consumes them, so the workspace holds one
 * window's records (the prhub report on SGLang PR #32890, section "实现拆解",
 * splits the prefill into the same two stages).  Chunk ids number the
 * 64-row chunks of all sequences without a prefix sum: the j-th chunk of
 * sequence n (rows from start_n) has id floor(start_n / 64) + n + j, and
 * every id is below floor((total_rows - 1) / 64) + num_seqs (num_seqs when
 * total_rows is 0); a window takes window_chunks consecutive ids.  The
 * library's choice: two windows for calls with at most 64 (sequence, head)
 * pairs and at least 32 ids, one otherwise.
 */
int32_t kda_prefill_windows(const kda_prefill_desc_t *desc);

/*
 * The fused prefill (bf16 only): each (sequence, head) pair of a sequence of
 * at most F chunks runs whole in one workgroup, which computes a chunk's
 * intra-chunk terms and applies them to the state it keeps in registers at
 * once, so no per-chunk record goes through memory (the prhub report on
 * SGLang PR #32890, sections "实现拆解" and "关键文件", fuses the
 * intra-chunk stages into one persistent kernel; here the state stage joins
 * them).  Longer sequences take the windows of intra-chunk kernel and scan.
 * The fused kernel runs a pair's chunks one after another, so it pays off
 * for many short sequences and not for long ones.  Returns F for `desc`
 * (-1: no sequence is fused, or desc is invalid): desc->fuse_chunks when it
 * is positive, none when it is negative, else the library's choice from the
 * sizes alone: 8 when total_rows <= 64 num_seqs, 6 when total_rows <=
 * 128 num_seqs, 8 when total_rows <= 256 num_seqs, none otherwise.  Results agree with the unfused path to the
 * usual bf16 rounding (the same operands, summed in another order).
 */
int32_t kda_prefill_fuse_chunks(const kda_prefill_desc_t *desc);

/*
 * Bytes of device workspace kda_chunk_prefill needs for `desc` (0 if desc is
 * invalid).  The workspace holds the per-chunk operands that pass from the
 * intra-chunk kernel to the state scan, and, when a conv mode runs the conv
 * as a pass of its own (see kda_chunk_prefill_conv), the convolved q, k and
 * v.  As in the "kern" page, section "The manifest", workspace is
 * scratch that lasts one call; the caller allocates it, as its hosts
 * allocate their own pools (same page, section "Hosts"), and may reuse it
 * for every call whose size it covers once the previous call on it is done
 * in stream order.
 */
size_t kda_prefill_workspace_size(const kda_prefill_desc_t *desc);

/*
 * Chunked prefill over a packed batch of sequences (the "P: the packed
 * prefill" section of the kern-k3-pp-prefill page; the chunk geometry of 64
 * rows with 16-row sub-blocks follows the prhub report on SGLang PR #32890,
 * section "关键源码片段").  Chunks never straddle sequences; the varlen
 * bookkeeping is done on the device, with no host sync (same report, section
 * "关键文件", chunk_fwd.py).
 *
 * For each sequence n with slot s = slots ? slots[n] : n:
 *   - if 0 <= s < num_slots: the initial state is state_in[s] (zeros when
 *     state_in is NULL); rows cu[n]..cu[n+1]-1 of o are written; the final
 *     state is written to state_out[s] (skipped when state_out is NULL).
 *     state_out may equal state_in (updated in place).  A zero-length
 *     sequence copies its state through.
 *   - otherwise the sequence is a padded row: its o rows and every state slot
 *     are left untouched.
 * bf16 sequences of at most kda_prefill_fuse_chunks(desc) chunks run in the
 * fused prefill, the others in the windows of intra-chunk kernel and scan.
 * Slots not named by any live sequence are never read or written.
 *
 * The state pools are addressed by lines as described above (dense when the
 * desc's strides are 0).
 *
 * With T = 0 (every sequence empty) no row is read or written: q, k, v, g,
 * beta and o may be NULL, and each live sequence's final state is its initial
 * state.
 *
 * Errors (returned before any launch): KDA_ERR_NULL for NULL desc or
 * cu_seqlens, for NULL q, k, v, g, beta or o when T > 0, or a NULL workspace of nonzero
 * required size; KDA_ERR_SHAPE for T < 0, N < 1, H < 1, num_slots < 0,
 * slots == NULL with a state pool given and num_slots < N, or state strides
 * that break the line rules; KDA_ERR_DTYPE;
 * KDA_ERR_UNSUPPORTED; KDA_ERR_ALIGN; KDA_ERR_WORKSPACE when ws_bytes is below
 * kda_prefill_workspace_size(desc); KDA_ERR_HIP if a launch fails.
 */
kda_status_t kda_chunk_prefill(const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens,
                               const float *state_in, float *state_out,
                               void *o, const int32_t *slots,
                               const kda_prefill_desc_t *desc,
                               void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * kda_chunk_prefill with per-kernel timing.  A call runs as one or more
 * windows of chunk ids (kda_prefill_windows), each an intra-chunk kernel and
 * a state scan.  When `events` is not NULL it points to num_events hipEvent_t:
 * events[0] is recorded on `stream` before the first kernel and events[i]
 * after the i-th kernel launch, in launch order (intra of window 0, scan of
 * window 0, intra of window 1, ..., then the fused prefill when
 * kda_prefill_fuse_chunks is not negative), as long as i < num_events; so
 * 2 W + 1 events (2 W + 2 with the fused prefill) time every kernel of a
 * W-window call with hipEventElapsedTime.  The
 * events are created and owned by the caller.  Results and errors are those
 * of kda_chunk_prefill.
 */
kda_status_t kda_chunk_prefill_timed(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta,
                                     const int32_t *cu_seqlens,
                                     const float *state_in, float *state_out,
                                     void *o, const int32_t *slots,
                                     const kda_prefill_desc_t *desc,
                                     void *workspace, size_t ws_bytes,
                                     void *stream, void *const *events, int32_t num_events);

/*
 * kda_chunk_prefill_timed with the short conv front end (desc->conv_mode not
 * KDA_CONV_NONE; see "Short conv front end" above): q, k and v are the raw
 * inputs, conv->window is read and then rewritten, and the rest of the step
 * runs on the convolved values.  For bf16 with d_k = d_v and no fused
 * sequence (kda_prefill_fuse_chunks is -1) the conv is folded into the
 * intra-chunk kernel's loads, which convolve the rows they read and round
 * them to bf16 as the pass would write them; the window update follows the
 * last intra-chunk launch, after the kernels that `events` (optional, as for
 * kda_chunk_prefill_timed) bracket.  Otherwise the conv runs first as a pass
 * of its own that writes the convolved q, k and v into the workspace, then
 * the window update, then the bracketed kernels.  Both orders give the same
 * values.  Errors as for kda_chunk_prefill, plus
 * KDA_ERR_NULL for a NULL conv, weight or window, and KDA_ERR_SHAPE for a
 * conv mode out of range or window strides that break the rules above.
 * kda_chunk_prefill and kda_chunk_prefill_timed return KDA_ERR_NULL for a
 * desc with a conv mode.
 */
kda_status_t kda_chunk_prefill_conv(const void *q, const void *k, const void *v,
                                    const float *g, const float *beta,
                                    const int32_t *cu_seqlens,
                                    const float *state_in, float *state_out,
                                    void *o, const int32_t *slots,
                                    const kda_prefill_desc_t *desc, const kda_conv_t *conv,
                                    void *workspace, size_t ws_bytes,
                                    void *stream, void *const *events, int32_t num_events);

/*
 * kda_decode_step with the state pool addressed by lines (see "State
 * addressing by lines" above): the block of (slot s, head h) starts at
 * state_pool + s * state_slot_stride + h * state_head_stride; strides of 0
 * select the dense layout.  Errors as for kda_decode_step, plus KDA_ERR_SHAPE
 * for strides that break the rules above.
 */
kda_status_t kda_decode_step_lines(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta,
                                   float *state_pool, const int32_t *slots, void *o,
                                   int32_t num_seqs, int32_t num_heads,
                                   int32_t d_k, int32_t d_v, int32_t num_slots,
                                   int32_t io_dtype, float scale,
                                   int64_t state_slot_stride, int64_t state_head_stride,
                                   void *stream);

/*
 * One decode token per sequence, state updated in place (the KDA step of the
 * kern-k3-pp-prefill page, section "D: TP8 / EP8 / DCP8"; padded rows with
 * slot -1 are skipped as in its section "D inside SGLang").
 *   q, k, g [N][H][d_k]; v, o [N][H][d_v]; beta [N][H];
 *   state_pool [num_slots][H][d_v][d_k] fp32, read and written in place;
 *   slots [N] int32 (required): a slot outside [0, num_slots) leaves that
 *   sequence's o rows and all state untouched.
 * Errors as for kda_chunk_prefill (N, H >= 1; num_slots >= 1).
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             float *state_pool, const int32_t *slots, void *o,
                             int32_t num_seqs, int32_t num_heads,
                             int32_t d_k, int32_t d_v, int32_t num_slots,
                             int32_t io_dtype, float scale, void *stream);

/*
 * kda_decode_step_lines with the short conv front end fused in (conv_mode
 * KDA_CONV_LINEAR or KDA_CONV_SILU; see "Short conv front end" above): q, k
 * and v are the raw token inputs; each live sequence's window is read and
 * shifted by one row in place.  Errors as for kda_decode_step_lines, plus
 * KDA_ERR_NULL for a NULL conv, weight or window and KDA_ERR_SHAPE for a
 * conv mode out of range or bad window strides.
 */
kda_status_t kda_decode_step_conv(const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  float *state_pool, const int32_t *slots, void *o,
                                  int32_t num_seqs, int32_t num_heads,
                                  int32_t d_k, int32_t d_v, int32_t num_slots,
                                  int32_t io_dtype, float scale,
                                  int64_t state_slot_stride, int64_t state_head_stride,
                                  int32_t conv_mode, const kda_conv_t *conv, void *stream);

/*
 * Multi-token decode and speculative verify / commit: T = num_tokens tokens
 * per sequence against one state (the prhub report on SGLang PR #32890,
 * section "关键文件": the conv-MTP decode kernel, which runs a multi-token
 * verify beside the single-token step, and ReplaySSM, which keeps a small
 * per-request window of inputs and folds the accepted tokens into the state
 * exactly at commit instead of snapshotting states, bit-consistent with the
 * recurrent step).
 *   q, k, g [N T][H][d_k]; v, o [N T][H][d_v]; beta [N T][H]: row n T + t is
 *   token t of sequence n.  state_pool, slots and the state strides are as
 *   for kda_decode_step_lines (a slot outside [0, num_slots) is a padded
 *   sequence: nothing of it is read or written).
 *   o: if not NULL, o[n T + t] is token t's output after tokens 0..t, as T
 *   consecutive kda_decode_step calls would give it.  q may be NULL only when
 *   o is NULL.
 *   commit = 0: the state is only read (verify).  commit != 0: the state
 *   after the first c_n tokens is written back, c_n = num_accepted[n] clamped
 *   to [0, T], or T when num_accepted is NULL; c_n = 0 leaves the slot
 *   untouched.  num_accepted is [N] int32 on the device or NULL.
 * The committed state and every output equal, bit for bit, those of c_n
 * (respectively t + 1) consecutive kda_decode_step calls on the same tokens.
 * So a verify call (commit = 0) followed, once the accepted counts are known,
 * by a commit call (o = q = NULL, commit = 1, num_accepted) on the same k, v,
 * g, beta window leaves the state that the accepted tokens alone give.
 * Errors as for kda_decode_step_lines, plus KDA_ERR_SHAPE for num_tokens
 * outside [1, 16] and KDA_ERR_NULL when o is NULL and commit = 0 (nothing to
 * do) or when o is given without q.
 */
kda_status_t kda_decode_tokens(const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               float *state_pool, const int32_t *slots, void *o,
                               const int32_t *num_accepted,
                               int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                               int32_t d_k, int32_t d_v, int32_t num_slots,
                               int32_t io_dtype, float scale, int32_t commit,
                               int64_t state_slot_stride, int64_t state_head_stride,
                               void *stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments without the workspace; same kernels and, bit
 * for bit, the same results.  The workspace is a static device array of
 * KDA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs this
 * call on until the process ends: enough for one packed 8192-row chunk of up
 * to 18 sequences at H = 32, d_k = d_v = 128 in bf16 (315.05 MiB of records
 * for 16 sequences, 319.45 MiB for 18).  A call whose kda_prefill_workspace_size exceeds it returns
 * KDA_ERR_TOO_LARGE before anything runs.  The first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress); no call
 * allocates.  Every call on one GPU shares its array: calls that overlap on
 * one GPU (different streams, or host threads, without ordering between
 * them) race and give unspecified results.  Nothing in the array needs
 * clearing: a call reads only bytes it wrote earlier in the same call.
 * No conv mode (the desc's conv_mode must be KDA_CONV_NONE).  Errors as for
 * kda_chunk_prefill, plus KDA_ERR_TOO_LARGE.
 */
#define KDA_STATIC_SCRATCH_BYTES ((size_t)320 << 20)
kda_status_t kda_chunk_prefill_static(const void *q, const void *k, const void *v,
                                      const float *g, const float *beta,
                                      const int32_t *cu_seqlens,
                                      const float *state_in, float *state_out,
                                      void *o, const int32_t *slots,
                                      const kda_prefill_desc_t *desc, void *stream);

/*
 * Opt-in check of the device-side preconditions that kda_chunk_prefill
 * documents but does not test (testing them inside the call would need a
 * host sync; the "kern" page, section "The manifest", rejects calls outside
 * their bounds before they launch, and this gives a caller that guarantee
 * for the device data).  Enqueued on `stream`: it sets *flags (device int32,
 * written by the call, no need to clear it) to the OR of
 *   KDA_CHECK_CU_SEQLENS  cu_seqlens[0] != 0, cu_seqlens[N] != T, or a
 *                         decreasing step;
 *   KDA_CHECK_G           some g > 0 or NaN;
 *   KDA_CHECK_SLOTS       two sequences name the same slot in [0, num_slots)
 *                         (looked for when N <= 4096);
 * or 0 when all hold.  g may be NULL when T = 0, slots NULL for slot n = n.
 * Only the desc's sizes are used.  It reads nothing outside the buffers the
 * desc sizes, so it is safe on malformed data.  Errors: KDA_ERR_NULL for a
 * NULL desc, cu_seqlens or flags, or a NULL g with T > 0; desc errors as for
 * kda_chunk_prefill; KDA_ERR_ALIGN; KDA_ERR_HIP if a launch fails.
 */
enum { KDA_CHECK_CU_SEQLENS = 1, KDA_CHECK_G = 2, KDA_CHECK_SLOTS = 4 };
kda_status_t kda_prefill_check(const float *g, const int32_t *cu_seqlens, const int32_t *slots,
                               const kda_prefill_desc_t *desc, int32_t *flags, void *stream);

/*
 * Phase clocks, for attributing the prefill's time to the phases inside its
 * kernels from the kernels' own timestamps, as the "kern" page, section "The
 * harness", attributes time to every call inside the real program.  Only a
 * library built with KDA_PHASE_CLOCKS records them (python -m
 * linear_attention_prefill_amd.build --phase-clocks writes
 * libkda_clocks.so, the same kernels plus the records); any other build
 * returns KDA_ERR_UNSUPPORTED and touches nothing.
 *
 * In such a build, lane 0 of each of the 8 waves of workgroup 0 of the
 * intra-chunk kernel (kernel = KDA_CLOCK_INTRA) or of the fused prefill
 * (KDA_CLOCK_FUSED), or of the 4 waves of workgroup 0 of the state scan
 * (KDA_CLOCK_SCAN; the longest sequence's first slice group), writes the
 * core clock counter (s_memtime) at each mark of its first KDA_CLOCK_ITEMS
 * items (chunks; scan: steps) into a device array laid out
 * [wave][item][mark], KDA_CLOCK_MARKS marks an item; a mark not reached
 * stays as it was (0 after a clear).  Intra-chunk and fused marks: 0 the
 * top of the item; 1 and 2 before and after the barrier that ends the
 * factor phase; 3, 4 around the one after the A blocks; 5, 6 after the
 * first inverse level; 7, 8 after the second; 9, 10 after w and u (the fp32
 * and fused builds' barrier there); fused only: 11, 12 around the barrier
 * after the state step, 13 after the chain bookkeeping.  Scan marks: 0 the
 * top of the step; 1 after the barrier that publishes the state tiles; 2
 * after U = u - w S and the Q~ S part of o; 3 after the barrier that
 * publishes U; 4 after the state update and the o store.  Later launches
 * overwrite the array.
 *
 * kda_phase_clocks copies the first `count` words (at most 8 * 64 * 16) of
 * that kernel's array to host_out (when not NULL), then zeroes the whole
 * array when `clear` is nonzero.  Synchronous (a blocking copy): call it
 * once the launches to read are done.  Errors: KDA_ERR_SHAPE for an unknown
 * kernel, KDA_ERR_UNSUPPORTED without the records, KDA_ERR_HIP if the copy
 * fails.
 */
enum { KDA_CLOCK_INTRA = 0, KDA_CLOCK_FUSED = 1, KDA_CLOCK_SCAN = 2, KDA_CLOCK_WAVES = 8,
       KDA_CLOCK_ITEMS = 64, KDA_CLOCK_MARKS = 16 };
kda_status_t kda_phase_clocks(int32_t kernel, uint64_t *host_out, size_t count, int32_t clear);

/*
 * Streaming bandwidth probe.  The "kern" page, section "Inside", lists perf
 * among its test harness's checks; here the reference for a kernel's HBM
 * rate is what plain streaming reaches on the same chip, measured next to it
 * (bench.py reports it beside each roofline).  Enqueues on `stream` one
 * grid-stride kernel of `grid` workgroups of 256 threads over `bytes` bytes
 * (a multiple of 16) with 16-byte nontemporal accesses:
 *   KDA_STREAM_READ    reads src; dst is a sink of at least 4 grid bytes,
 *                      written only if the XOR of the data folds to one
 *                      fixed 32-bit value;
 *   KDA_STREAM_COPY    copies src to dst (not overlapping);
 *   KDA_STREAM_UPDATE  multiplies dst, read as fp32, by 1.0001 in place
 *                      (src unused, may be NULL).
 * The caller times it (events on `stream`).  Errors: KDA_ERR_SHAPE for an
 * unknown mode, grid < 1 or bytes not a multiple of 16; KDA_ERR_NULL;
 * KDA_ERR_ALIGN for pointers not 16-byte aligned; KDA_ERR_HIP if the launch
 * fails.
 */
enum { KDA_STREAM_READ = 0, KDA_STREAM_COPY = 1, KDA_STREAM_UPDATE = 2 };
kda_status_t kda_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes, int32_t grid,
                              void *stream);

/*
 * Matrix-core issue probe.  Like the streaming probe, a reference measured
 * on the same chip for the perf checks the "kern" page, section "Inside",
 * lists: here for the kernels' bf16 products.  Enqueues on `stream` one
 * workgroup of 4 waves (one per SIMD); each wave runs `iters` rounds of
 * `chains` (1, 2, 4 or 8) bf16 16x16x32 products, one on each of `chains`
 * independent accumulators, and wave w writes out[2w] = the core clocks
 * (s_memtime) and out[2w + 1] = the 100 MHz reference ticks (s_memrealtime)
 * its loop took.  `out` is caller-owned device memory of 12 uint64 (words 8
 * to 11 are a sink that is written only in a case the probe's data never
 * reach), 8-byte aligned.  Core clocks per product = out[0] / (iters
 * chains): with one accumulator each product waits for the one before, with
 * eight the matrix core's own rate shows.  Errors: KDA_ERR_SHAPE for other
 * chains or iters outside 1 .. 2^20, KDA_ERR_NULL, KDA_ERR_ALIGN,
 * KDA_ERR_HIP if the launch fails.
 */
kda_status_t kda_mfma_probe(int32_t chains, int32_t iters, uint64_t *out, void *stream);

/*
 * Static description of a status code.  Every call validates its arguments
 * on the host and returns one of these codes before anything launches, as
 * the "kern" page, section "The manifest", rejects a call outside its bounds
 * before it launches.
 */
const char *kda_status_string(kda_status_t status);

/*
 * Library ABI version (major * 100 + minor), so that a host can check which
 * C ABI the library it loaded implements before it binds the calls (the
 * "kern" page, section "Hosts": the runtime checks what a host hands it
 * against what it declares).
 */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
