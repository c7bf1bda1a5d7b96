// KDA chunked prefill for gfx950: an intra-chunk kernel and a state scan.
//
// Chunk algebra (derived from the gated delta rule; the prhub report on
// SGLang PR #32890, sections "实现拆解" and "关键文件", splits the same work
// into a fused A_kk / inverse / recompute-w-u stage and a per-chunk state
// stage, and its section "关键源码片段" fixes 64-row chunks with 16-row
// sub-blocks).  For one head and a chunk of C <= 64 rows with start state S0
// (d_k x d_v), with Gam_r the inclusive cumulative log-decay of rows <= r:
//   A_kk[r,s] = beta_r sum_c k_r[c] k_s[c] exp(Gam_r[c] - Gam_s[c])   (s < r)
//   A_qk[r,s] =        sum_c q_r[c] k_s[c] exp(Gam_r[c] - Gam_s[c])   (s <= r)
//   Tm = (I + A_kk)^-1,  w = Tm diag(beta)(K * e^Gam),  u = Tm diag(beta) V
//   U = u - w S0
//   O = scale ((Q * e^Gam) S0 + A_qk U)
//   S = diag(e^{Gam_C}) S0 + (K * e^{Gam_C - Gam})^T U
//
// Decay factoring.  With s(r) and e(r) the first and last rows of r's 16-row
// block, every row gets two factors that never exceed 1:
//   P_r = e^{Gam_r - Gam_s(r)},   Qf_r = e^{Gam_e(r) - Gam_r},
// and every (row block I, column block J <= I) pair one per-channel factor
//   F_IJ = e^{Gam_{16I} - Gam_{16J+15}}   (<= 1 for J < I).
// Then e^{Gam_a - Gam_b} = P_a Qf_b F_IJ for a in block I, b in block J, so
// A_kk and A_qk blocks are products of k P, q P and k Qf F on the matrix
// cores.  For J = I, F_II is the block's own decay span; when a channel's span
// exceeds 2^64 the diagonal block falls back to one exp per term.  Likewise
// Q e^Gam = q P e^{Gam_s}, K e^Gam = k P e^{Gam_s} and
// K e^{Gam_C - Gam} = k Qf e^{Gam_C - Gam_e}.  Two exps per element replace
// one exp per element per use.
//
// kda_intra_kernel: a persistent grid of one 8-wave workgroup per CU (two
// waves per SIMD) walks the (chunk, head) items; the next item's raw inputs
// are fetched into registers a part per phase while the current one is
// computed.  Per item: row factors (lanes hold four consecutive rows, DPP row
// scans give the block prefixes), A blocks and the four diagonal inverses in
// parallel, the off-diagonal inverse blocks in two levels on fp32 matrix
// cores (which also leave Tm diag(beta) in LDS as bf16 fragments), then w and
// u; workspace fragments are written in the scan's order.  For bf16 the row
// factors that w and u read are double-buffered, so a wave that finishes
// them starts the next item's row factors without waiting for the others.
// kda_scan_kernel: one workgroup of 4 waves per (sequence, head, group of NS
// 16-column slices of d_v); the d_v columns of S evolve independently, so
// slices need no exchange.  Wave w owns chunk rows 16w..16w+15 and a quarter
// of the key channels, swaps the rounded copies of its S and U tiles with the
// other waves through LDS, and keeps the operands of the next chunks in
// flight in registers, applying each to all NS slices.  The scan is bound by
// the record bytes each CU takes in, which a workgroup takes in once for its
// NS slices: each call uses the largest NS of 1, 2 or 4 (bf16 for NS > 1)
// that still leaves every CU a workgroup.
// kda_fused_prefill_kernel (bf16): the intra-chunk kernel's body walking
// whole (sequence, head) chains; each chunk's operands stay in LDS and a
// sixth phase applies them to the chain's state, which the waves keep in
// registers (wave w: value columns 16w .. 16w + 15).  Calls choose it for
// short sequences (kda_prefill_fuse_chunks), since a chain's chunks run one
// after another.
#include <mutex>
#include <type_traits>

#include "kda.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// Intra-chunk kernel
// ---------------------------------------------------------------------------

// Decay span (log2 units) of a 16-row block above which its diagonal block is
// computed exactly instead of with split factors.
constexpr float kDiagSpanLimit = 64.f;
constexpr int kIntraThreads = 512;     // 8 waves: two per SIMD
static_assert(kIntraThreads / 64 == kClockWaves, "one clock row per wave");
#ifdef KDA_PHASE_CLOCKS
// [kernel: 0 intra-chunk, 1 fused, 2 scan][wave][item][mark] core clock counts
__device__ unsigned long long g_phase_clock[kClockKernels * kClockWaves * kClockItems * kClockMarks];
#endif
constexpr int kCuCache = 256;          // sequence bounds kept in LDS when N < this
constexpr int kScanWarmAhead = 2;      // chunks between a scan stage's record and the one it warms
#ifndef KDA_SINGLE_CHAIN
#define KDA_SINGLE_CHAIN 0
#endif

// LDS of the intra-chunk kernel.  For bf16, V is staged as a row-major tile
// and read back as fragments; for fp32 (twice the bytes) it is read from
// global memory in fragment order.  K e^Gam and Q e^Gam are not staged: they
// are rebuilt from k P, q P and e^{Gam_s} where they are used (Q e^Gam by
// waves that would otherwise wait on the first inverse level, K e^Gam as the
// w product's operand), which keeps their products and stores out of the
// VALU-bound factor phase and 34 KB out of LDS.
template <typename E, int DK, int DV, bool FUSED> struct IntraLds {
    static constexpr bool kStage = sizeof(E) == 2;  // V staged in LDS
    // bf16: k P, V and e^{Gam_s} (all the w and u products read from the row
    // factors) in two buffers, alternating by item, so that the next item's
    // factor phase needs no barrier after this item's w and u.  fp32 has no
    // room for the second k P, and the fused prefill needs that room for the
    // chunk operands of its state step (its items end in a barrier anyway).
    static constexpr int NB = sizeof(E) == 2 && !FUSED ? 2 : 1;
    // Pitches.  A k P / q P row of d_k + 4 elements (4 mod 8) spreads the
    // factor phase's row writes and the fragment reads over the LDS banks:
    // against d_k + 8 (bf16) it stalls a third fewer cycles on bank
    // conflicts and the kernel runs 9% faster; against d_k (fp32) 7% faster.
    // Those rows are only accessed in 8-byte (bf16) or 16-byte (fp32) runs.
    // V rows keep d_v + 8, since V is staged with 16-byte row stores.
    static constexpr int KPP = DK + 4;              // pitch of k P, q P (E)
    static constexpr int KQP = DK + 4;              // pitch of k Qf (fp32)
    static constexpr int VP = DV + (sizeof(E) == 2 ? 8 : 0);   // pitch of V (E)
    static constexpr int AP = 68;                   // pitch of A_kk -> Tm (fp32)
    static constexpr int DP = 16;                   // pitch of the diagonal A_kk blocks (fp32)
    static constexpr int V_ELEMS = kStage ? kChunk * VP : 8;
};

// Raw inputs of one chunk held by one thread (prefetched for the next chunk).
template <typename E> struct Raw4;
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <> struct Raw4<float> { typedef f32x4 type; };
template <typename E> __device__ __forceinline__ f32x4 to_f32(const bf16x4 &x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <typename E> __device__ __forceinline__ f32x4 to_f32(const f32x4 &x) { return x; }

// Completes the load that produced x at this point of the program (an empty
// asm statement that consumes and redefines every 32-bit word of x).
template <typename T> __device__ __forceinline__ void settle(T &x) {
    static_assert(sizeof(T) % 4 == 0, "settle");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &x, sizeof(T));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" : "+v"(w[i]));
    __builtin_memcpy(&x, w, sizeof(T));
}

// Cross-lane moves inside a DPP row (16 lanes): row_shr:N brings lane i - N
// (0 below the row's first lane), row_newbcast:L brings lane L of the row.
template <int CTRL> __device__ __forceinline__ float dpp_row(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Inclusive prefix sum over the 16 lanes of each row.
__device__ __forceinline__ float row_scan(float x) {
    x += dpp_row<0x111>(x);
    x += dpp_row<0x112>(x);
    x += dpp_row<0x114>(x);
    x += dpp_row<0x118>(x);
    return x;
}
template <int L> __device__ __forceinline__ float row_bcast(float x) { return dpp_row<0x150 + L>(x); }
// Lane L of each quad of lanes, to the whole quad (quad_perm [L, L, L, L]).
template <int L> __device__ __forceinline__ float quad_bcast(float x) { return dpp_row<L * 0x55>(x); }

// A chunk of one head: item = cid * H + h; valid when item >= 0.
struct ChunkRef {
    int item, cid, h, row0, C;
    int n, jc;          // sequence, and the chunk's index in it
};

// Index p = I (I + 1) / 2 + J of the block pair (I, J), J <= I < 4.
__device__ __forceinline__ int pair_row(int p) { return p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3)); }

// The fused prefill's part of a call: chains (sequence, head) of at most
// fuse_max chunks run whole in one workgroup; the intra-chunk kernel and the
// scan skip them.  fuse_max < 0: no chain is fused.
struct FuseArgs {
    const int32_t *slots;
    const float *state_in;
    float *state_out;
    void *o;
    int num_slots;
    float scale;
    int64_t slot_stride, head_stride;
    int fuse_max;
};

// The short conv front end folded into the intra-chunk kernel's loads (bf16,
// d_k = d_v): each factor lane convolves its four rows of k, q and v, taking
// the three rows before them from the lane below (a DPP row shift) or, for
// a chunk's first rows, from the rows before the chunk or the sequence's
// conv window, staged per wave in LDS with the taps of its channels.
template <typename E> struct ConvFold {
    const float *weight;        // [H][4][2 d_k + d_v]
    const E *window;
    ConvWin win;
    const int32_t *slots;
    int num_slots;
};
constexpr int kCvFloats = 3 * kConvTaps * 16 + 3 * kConvWindow * 16 / 2;   // per wave: taps, then halo (bf16)

// row_shr:1 within each 16-lane row (the row's first lane gets zeros)
__device__ __forceinline__ bf16x4 dpp_shr1(const bf16x4 &x) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 w = __builtin_bit_cast(i32x2, x);
    w[0] = __builtin_amdgcn_update_dpp(0, w[0], 0x111, 0xF, 0xF, true);
    w[1] = __builtin_amdgcn_update_dpp(0, w[1], 0x111, 0xF, 0xF, true);
    return __builtin_bit_cast(bf16x4, w);
}

// The body of both persistent 8-wave kernels.  FUSED = false: the
// intra-chunk kernel, which writes each item's record to the workspace (and
// with SKIP passes over the chunks of sequences the fused prefill takes).
// FUSED = true (bf16): the fused prefill, which walks whole chains and keeps
// the record of the current chunk in LDS, where the state step that follows
// its intra-chunk phases reads it (no record round trip through memory).
template <typename E, int DK, int DV, bool FUSED, bool SKIP, int CONV = 0>
__device__ __forceinline__ void intra_chunks(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int H, int c_lo, int c_hi,
    E *__restrict__ ws, float *__restrict__ ws_dec, const FuseArgs &fa,
    const ConvFold<E> &cf = ConvFold<E>{}) {
    static_assert(DK == 64 || DK == 128, "d_k");
    static_assert(DV == 64 || DV == 128, "d_v");
    static_assert(!FUSED || sizeof(E) == 2, "the fused prefill is bf16");
    static_assert(CONV == 0 || (sizeof(E) == 2 && DK == DV && !FUSED), "folded conv: bf16, d_k = d_v");
    using LD = IntraLds<E, DK, DV, FUSED>;
    using L = WsLayout<E, DK, DV>;
    using R4 = typename Raw4<E>::type;
    constexpr int NTH = kIntraThreads;
    constexpr int KPP = LD::KPP, KQP = LD::KQP, VP = LD::VP, AP = LD::AP, DP = LD::DP;
    constexpr int KS = DK / kSlab;                     // d_k slabs
    constexpr int VT = DV / kSub;                      // d_v tiles
    constexpr int C4 = DK / 4;                         // 4-channel columns
    constexpr int FW = C4 / 4;                         // waves of the factor phase
    constexpr int KT = DK / kSub;                      // d_k tiles
    constexpr int EPU = 16 / sizeof(E);
    constexpr int VPT = LD::kStage ? kChunk * DV / EPU / NTH : 1;
    constexpr int MPW = KS / 2;                        // w row tiles per wave
    static_assert(FW <= NTH / 64 && VT <= 8, "thread mapping");

    __shared__ __align__(16) E sKPb[LD::NB * kChunk * KPP];  // k P
    __shared__ __align__(16) E sQP[kChunk * KPP];      // q P
    __shared__ __align__(16) E sVb[LD::NB * LD::V_ELEMS];   // V
    __shared__ __align__(16) float sKQ[kChunk * KQP];  // k Qf (fp32)
    __shared__ __align__(16) float sA[kChunk * AP];    // A_kk -> Tm
    __shared__ __align__(16) float sD[4 * kSub * DP];  // diagonal A_kk blocks
    __shared__ __align__(16) E sTb[6 * 512];           // Tm diag(beta) fragments, index tri_frag(m, s)
    __shared__ __align__(16) float sBsb[LD::NB * 4 * DK];   // e^{Gam} at each block's first row
    __shared__ __align__(16) float sCe[4 * DK];        // e^{Gam_C - Gam} at each block's last row
    __shared__ __align__(16) float sF[10 * DK];        // F_IJ, J <= I, index I(I+1)/2 + J
    __shared__ __align__(16) float sBeta[kChunk];
    __shared__ int sExact[4 * C4];                     // per block and 4-channel column
    __shared__ int sCu[FUSED ? 1 : kCuCache];
    // fused: the chunk's K~^T and A_qk fragments and e^{Gam_C}; its Q~ and w
    // fragments take the k Qf rows, which are dead once K~^T is formed
    __shared__ __align__(16) E sKt[FUSED ? DK * kChunk : 8];
    __shared__ __align__(16) E sAq[FUSED ? 6 * 512 : 8];
    __shared__ __align__(16) float sDec[FUSED ? DK : 4];
    static_assert(!FUSED || 2 * kChunk * DK * sizeof(E) <= sizeof(sKQ), "Q~ and w in the k Qf rows");
    E *const sQt = reinterpret_cast<E *>(sKQ);         // fused: Q~ fragments
    E *const sW = sQt + kChunk * DK;                   // fused: w fragments
    // folded conv: this wave's taps and halo rows, in the A_kk rows (dead
    // from the end of the second inverse level to the next A-block phase)
    static_assert(CONV == 0 || (kIntraThreads / 64) * kCvFloats <= kChunk * LD::AP, "conv slots");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // factor phase: lane (r, c) of wave w < FW (r = lane % 16, c = lane / 16)
    // owns channels 4 cq .. + 3, cq = 4 w + c, of rows 4 r .. 4 r + 3: a DPP
    // row of 16 lanes spans the chunk and a quad of lanes one 16-row block.
    const int r4 = lane & 15, cq = 4 * wave + lg, ch0 = 4 * cq;
    float *const sCv = sA + wave * kCvFloats;          // folded conv: [tensor][tap][16] taps
    E *const sCvh = reinterpret_cast<E *>(sCv + 3 * kConvTaps * 16);   // [tensor][row][16] halo
    const bool fthread = wave < FW;
    const int stride = gridDim.x;

    // Sequence bounds: up to 64 in one register (lane i holds cu[i], read
    // back with readlane), else up to kCuCache in LDS, else scalar loads.
    const bool cu_reg = N < 64, cu_lds = !FUSED && N < kCuCache;
    const int cu_v = (cu_reg && lane <= N) ? cu[lane] : 0;
    if (!cu_reg && cu_lds)
        for (int i = tid; i <= N; i += NTH) sCu[i] = cu[i];
    // SKIP, one window: the sequences this launch runs (more than fuse_max
    // chunks) listed in LDS with their chunk prefix, when they number at most
    // kCuCache, so that the grid steps over their chunks only; a call whose
    // sequences are all fused then has nothing to walk (the id walk would look
    // each id up to pass it over: 44 us for 128 sequences at H = 32).  More
    // sequences, or windows, take the id walk.
    __shared__ int sLong[SKIP ? kCuCache : 1];
    __shared__ int sLcum[SKIP ? kCuCache + 1 : 1];
    __shared__ int sWs[2][NTH / 64];
    int nlong = -1;                                    // -1: the id walk
    if constexpr (SKIP) {
        if (c_lo == 0 && c_hi == chunk_id_count(T, N)) {
            int count = 0, chunks = 0;                 // running totals, uniform
            for (int base = 0; base < N; base += NTH) {
                const int n = base + tid;
                int nc = 0;
                if (n < N) {
                    const int s0 = clamp_row(cu[n], T), s1 = clamp_row(cu[n + 1], T);
                    nc = s1 > s0 ? (s1 - s0 + kChunk - 1) / kChunk : 0;
                    if (nc <= fa.fuse_max) nc = 0;
                }
                const int f = nc > 0 ? 1 : 0;
                int fs = f, cs = nc;                   // inclusive scans over the wave
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int y = __shfl_up(fs, d), z = __shfl_up(cs, d);
                    if (lane >= d) {
                        fs += y;
                        cs += z;
                    }
                }
                if (lane == 63) {
                    sWs[0][wave] = fs;
                    sWs[1][wave] = cs;
                }
                __syncthreads();
                int fo = 0, co = 0, ft = 0, ct = 0;
#pragma unroll
                for (int w = 0; w < NTH / 64; ++w) {
                    if (w < wave) {
                        fo += sWs[0][w];
                        co += sWs[1][w];
                    }
                    ft += sWs[0][w];
                    ct += sWs[1][w];
                }
                const int pos = count + fo + fs - f;
                if (f && pos < kCuCache) {
                    sLong[pos] = n;
                    sLcum[pos] = chunks + co + cs - nc;
                }
                count += ft;
                chunks += ct;
                __syncthreads();                       // sWs is reused
            }
            if (count <= kCuCache) {
                nlong = count;
                if (tid == 0) sLcum[count] = chunks;
            }
        }
    }
    // Tm diag(beta) fragments (m, s), s <= m / 2: lane (i, g) holds row
    // 16 m + i, columns 32 s + kk(g, e), as the w and u products take them.
    // Their right halves for even m are the zero blocks (0, 1) and (2, 3),
    // written once here; every other half is rewritten per item where its
    // block of Tm becomes final.
    if (tid < 128) {
        const int m = 2 * (tid >> 6);                  // fragments (0, 0) and (2, 1)
        store4<E>(sTb + tri_frag(m, m >> 1) * 512 + lane * 8 + 4, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();
    // (scalar loads for the uncached case: no vector-memory wait in the loop)
    const int32_t __attribute__((address_space(4))) *cu_s =
        (const int32_t __attribute__((address_space(4))) *)cu;
    auto cu_at = [&](int i) {
        if (cu_reg) return __builtin_amdgcn_readlane(cu_v, i);
        return __builtin_amdgcn_readfirstlane(cu_lds ? sCu[i] : cu_s[i]);
    };
    // Items (chunk id cid, head h; item = cid H + h) of the window
    // [c_lo, c_hi) of chunk ids are walked from the last one down in steps of
    // the grid, so the records the state scan reads first are the ones
    // written last and are still in the caches when it starts.  Item (cid, h)
    // writes record (cid - c_lo) H + h of the window's workspace.  The step is kept as a quotient and remainder of H, so the walk
    // needs no division.  find_chunk returns the first item at or below (cid,
    // h) on this walk that belongs to a sequence (ids between sequences'
    // chunk ranges are skipped).
    const int step_q = stride / H, step_r = stride % H;
    // rows beyond which a sequence is not fused
    const int fuse_rows = fa.fuse_max * kChunk;
    auto step_down = [&](int &cid, int &h) {
        h -= step_r;
        cid -= step_q;
        if (h < 0) {
            h += H;
            --cid;
        }
    };
    // With the bounds in a register (N < 64), lane n also holds the first
    // chunk id of sequence n, and the sequence of a chunk id is one ballot
    // away: the ids are non-decreasing in n, so it is the count of lanes at
    // or below the id, less one.  (A binary search there took about 1.4k
    // clocks an item in branches, 8% of the item.)
    const int fc_v = (cu_reg && lane < N) ? clamp_row(cu_v, T) / kChunk + lane : INT_MAX;
    auto find_chunk = [&](int cid, int h) -> ChunkRef {
        for (; cid >= c_lo; step_down(cid, h)) {
            int lo = 0, start, end;
            if (cu_reg) {
                lo = __popcll(__ballot(fc_v <= cid)) - 1;
                lo = lo < 0 ? 0 : lo;
                start = clamp_row(__builtin_amdgcn_readlane(cu_v, lo), T);
                end = clamp_row(__builtin_amdgcn_readlane(cu_v, lo + 1), T);
            } else {
                int hi = N - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (clamp_row(cu_at(mid), T) / kChunk + mid <= cid) lo = mid; else hi = mid - 1;
                }
                start = clamp_row(cu_at(lo), T);
                end = clamp_row(cu_at(lo + 1), T);
            }
            const int len = end > start ? end - start : 0;
            const int jc = cid - (start / kChunk + lo);
            if (jc >= 0 && jc * kChunk < len && (!SKIP || len > fuse_rows))
                return ChunkRef{cid * H + h, cid, h, start + jc * kChunk, min(kChunk, len - jc * kChunk),
                                lo, jc};
        }
        return ChunkRef{-1, 0, 0, 0, 0, 0, 0};
    };

    // registers holding the next chunk's raw inputs
    R4 kr[4], qr[4];
    R4 vr[CONV ? 4 : 1];                               // folded conv: V in the factor lanes' order
    f32x4 gr[4];
    uint4 xv[VPT];
    float bt = 0.f;
    // k, q, g of row 4 r4 + r (one of this lane's four rows)
    auto load_row = [&](const ChunkRef &ck, int r) {
        const int row = 4 * r4 + r;
        kr[r] = qr[r] = R4{};
        if constexpr (CONV != 0) vr[r] = R4{};
        gr[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (fthread && ck.item >= 0 && row < ck.C) {
            const size_t off = ((size_t)(ck.row0 + row) * H + ck.h) * DK + ch0;
            kr[r] = *reinterpret_cast<const R4 *>(k + off);
            qr[r] = *reinterpret_cast<const R4 *>(q + off);
            gr[r] = *reinterpret_cast<const f32x4 *>(g + off);
            if constexpr (CONV != 0) vr[r] = *reinterpret_cast<const R4 *>(v + off);
        }
    };
    // Folded conv staging, per wave: taps of its 16 channels (lanes 0..47,
    // [tensor][tap][4 channels]) and the three rows before the chunk (lanes
    // 0..35, [tensor][row][4 channels]): rows of the same sequence, its conv
    // window for a first chunk, or zeros for a padded sequence.  Fetched into
    // registers a phase ahead (addresses clamped, loads unconditional), then
    // put into the wave's LDS slot.
    const float *const cv_weight = cf.weight;
    const E *const cv_window = cf.window;
    const ConvWin cv_win = cf.win;
    const int32_t *const cv_slots = cf.slots;
    const int cv_nslots = cf.num_slots;
    f32x4 cw_reg = f32x4{0.f, 0.f, 0.f, 0.f};
    R4 ch_reg = R4{};
    bool ch_zero = true;
    auto conv_fetch = [&](const ChunkRef &ck, int slot) __attribute__((always_inline)) {
        if constexpr (CONV != 0) {
            const int hh = ck.item >= 0 ? ck.h : 0;
            {
                const int l = lane < 48 ? lane : 47;
                const int p = l >> 4, j = (l >> 2) & 3, c4 = l & 3;
                cw_reg = *reinterpret_cast<const f32x4 *>(
                    cv_weight + ((size_t)hh * kConvTaps + j) * (2 * DK + DV) + p * DK + 16 * wave + 4 * c4);
            }
            {
                const int l = lane < 36 ? lane : 35;
                const int p = l / 12, i = (l >> 2) % 3, c4 = l & 3;
                const int ch = 16 * wave + 4 * c4;
                const bool inseq = ck.item >= 0 && ck.jc > 0;
                const bool live = ck.item >= 0 && ck.jc == 0 && slot >= 0 && slot < cv_nslots;
                const int row = inseq ? ck.row0 - kConvWindow + i : 0;
                // the lane's tensor picked by arithmetic on the pointer values:
                // a conditional over the captured names becomes a load through
                // a selected address, which keeps them in private memory
                const E *const src = reinterpret_cast<const E *>(
                    reinterpret_cast<uintptr_t>(q) * (p == 0) + reinterpret_cast<uintptr_t>(k) * (p == 1) +
                    reinterpret_cast<uintptr_t>(v) * (p == 2));
                const E *const addr = live ? cv_window + cv_win.at(slot, hh, i, p, ch)
                                           : src + ((size_t)row * H + hh) * DK + ch;
                ch_reg = *reinterpret_cast<const R4 *>(addr);
                ch_zero = !(inseq || live);
            }
        }
    };
    auto conv_put = [&]() __attribute__((always_inline)) {
        if constexpr (CONV != 0) {
            if (fthread) {
                if (lane < 48) *reinterpret_cast<f32x4 *>(sCv + lane * 4) = cw_reg;
                if (lane < 36) *reinterpret_cast<R4 *>(sCvh + lane * 4) = ch_zero ? R4{} : ch_reg;
            }
        }
    };
    // The folded conv of one tensor's four rows (in place, rounded to the io
    // type as the conv pass would write them; rows past the chunk's end stay
    // zero).
    auto conv_rows = [&](R4 (&x)[4], int p, int C) __attribute__((always_inline)) {
        if constexpr (CONV != 0) {
            R4 m3 = dpp_shr1(x[1]), m2 = dpp_shr1(x[2]), m1 = dpp_shr1(x[3]);
            if (r4 == 0) {
                m3 = *reinterpret_cast<const R4 *>(sCvh + (p * 3 + 0) * 16 + 4 * lg);
                m2 = *reinterpret_cast<const R4 *>(sCvh + (p * 3 + 1) * 16 + 4 * lg);
                m1 = *reinterpret_cast<const R4 *>(sCvh + (p * 3 + 2) * 16 + 4 * lg);
            }
            // one channel at a time: its four taps and seven inputs
            const float *const wp = sCv + p * kConvTaps * 16 + 4 * lg;
            float t[4][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float w0 = wp[c], w1 = wp[16 + c], w2 = wp[32 + c], w3 = wp[48 + c];
                const float xs[7] = {(float)m3[c],   (float)m2[c],   (float)m1[c],  (float)x[0][c],
                                     (float)x[1][c], (float)x[2][c], (float)x[3][c]};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t[r][c] = conv_act(conv4(w0, w1, w2, w3, xs[r], xs[r + 1], xs[r + 2], xs[r + 3]), CONV == 2);
            }
            // rounded a row at a time; a row past the chunk's end is zero
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                R4 y;
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = (E)t[r][c];
                x[r] = 4 * r4 + r < C ? y : R4{};
            }
        }
    };
    auto load_beta = [&](const ChunkRef &ck) {
        bt = (ck.item >= 0 && tid < ck.C) ? beta[(size_t)(ck.row0 + tid) * H + ck.h] : 0.f;
    };
    auto load_v = [&](const ChunkRef &ck) {
        if constexpr (LD::kStage && CONV == 0) {
#pragma unroll
            for (int p = 0; p < VPT; ++p) {
                const int u = tid + p * NTH;
                const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
                xv[p] = uint4{0, 0, 0, 0};
                if (ck.item >= 0 && r < ck.C)
                    xv[p] = *reinterpret_cast<const uint4 *>(v + ((size_t)(ck.row0 + r) * H + ck.h) * DV + c);
            }
        }
    };

    // ---- fused: the walk over chains ----
    // Chains are the (sequence, head) pairs whose sequence has at most
    // fuse_max chunks and a live slot.  With fewer than 64 sequences the
    // fused sequences are ranked longest first (ties by index) and chain c is
    // head c % H of the (c / H)-th of them; otherwise chain c is pair
    // (c / H, c % H) and the others are passed over.  Workgroup b takes
    // chains b, b + G, b + 2G, ...; a chain's state stays in registers (wave
    // w < d_v / 16 holds value columns 16 w .. 16 w + 15) for all its chunks.
    struct FChain {
        int c, n, h, slot, start, len, nch;
    };
    int fl_len = -1, fl_rank = 0, nf_seq = 0;
    if constexpr (FUSED) {
        if (cu_reg) {
            const int s0 = clamp_row(cu_v, T), s1 = clamp_row(__shfl_down(cu_v, 1), T);
            const int len = s1 > s0 ? s1 - s0 : 0;
            const bool fus = lane < N && (len + kChunk - 1) / kChunk <= fa.fuse_max;
            fl_len = fus ? len : -1;
            for (int m = 0; m < N; ++m) {
                const int lm = __shfl(fl_len, m);
                fl_rank += (lm > fl_len || (lm == fl_len && m < lane)) ? 1 : 0;
            }
            nf_seq = __popcll(__ballot(fus));
        }
    }
    const int chains = cu_reg ? nf_seq * H : N * H;
    auto resolve = [&](int c) -> FChain {
        for (; c < chains; c += stride) {
            const int h = c % H;
            int n = c / H;
            if (cu_reg) n = __ffsll((long long)__ballot(fl_len >= 0 && fl_rank == c / H)) - 1;
            const SeqSpan sp = seq_span(cu, n, T);
            const int nch = (sp.len + kChunk - 1) / kChunk;
            if (nch > fa.fuse_max) continue;
            const int slot = fa.slots ? fa.slots[n] : n;
            if (fa.slots && (slot < 0 || slot >= fa.num_slots)) continue;
            return FChain{c, n, h, slot, sp.start, sp.len, nch};
        }
        return FChain{-1, 0, 0, 0, 0, 0, 0};
    };
    auto state_at = [&](const float *base, const FChain &ch) {
        return base + ch.slot * fa.slot_stride + ch.h * fa.head_stride + (size_t)(wave * kSub + li) * DK + 4 * lg;
    };
    // A chain with no rows passes its state through (zero without state_in).
    auto pass_state = [&](const FChain &ch) {
        if (wave >= VT || !fa.state_out) return;
        float *dst = const_cast<float *>(state_at(fa.state_out, ch));
        const float *src = fa.state_in ? state_at(fa.state_in, ch) : nullptr;
#pragma unroll
        for (int t = 0; t < KT; ++t)
            *reinterpret_cast<f32x4 *>(dst + t * kSub) =
                src ? *reinterpret_cast<const f32x4 *>(src + t * kSub) : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto next_chain = [&](int c) -> FChain {   // the first chain at or after c with rows
        FChain ch = resolve(c);
        while (ch.c >= 0 && ch.nch == 0) {
            pass_state(ch);
            ch = resolve(ch.c + stride);
        }
        return ch;
    };
    auto item_of = [&](const FChain &ch, int j) -> ChunkRef {
        if (ch.c < 0) return ChunkRef{-1, 0, 0, 0, 0, 0, 0};
        const int cid = ch.start / kChunk + ch.n + j;
        return ChunkRef{cid * H + ch.h, cid, ch.h, ch.start + j * kChunk, min(kChunk, ch.len - j * kChunk),
                        ch.n, j};
    };
    // key tile t of this wave's state slice, C layout: S[16t + 4g + r][16 wave + i]
    f32x4 S[FUSED ? KT : 1];
    auto state_load = [&](const FChain &ch) {
        if (wave >= VT) return;
        const float *src = fa.state_in ? state_at(fa.state_in, ch) : nullptr;
#pragma unroll
        for (int t = 0; t < KT; ++t)
            S[t] = src ? *reinterpret_cast<const f32x4 *>(src + t * kSub) : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto state_store = [&](const FChain &ch) {
        if (wave >= VT || !fa.state_out) return;
        float *dst = const_cast<float *>(state_at(fa.state_out, ch));
#pragma unroll
        for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(dst + t * kSub) = S[t];
    };
    bf16x4 ureg[4];                                    // fused: this wave's u tile, row tile m


    // SKIP list walk: item r = k H + h, the k-th listed chunk and head h,
    // from the last one down in steps of the grid
    auto find_long = [&](int r) -> ChunkRef {
        if (r < 0) return ChunkRef{-1, 0, 0, 0, 0, 0, 0};
        const int kc = r / H, h = r - kc * H;
        int lo = 0, hi = nlong - 1;                    // the last listed sequence with sLcum <= kc
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sLcum[mid] <= kc) lo = mid; else hi = mid - 1;
        }
        const int n = __builtin_amdgcn_readfirstlane(sLong[lo]);
        const int start = clamp_row(cu_at(n), T), end = clamp_row(cu_at(n + 1), T);
        const int len = end > start ? end - start : 0;
        const int jc = kc - sLcum[lo];
        const int cid = start / kChunk + n + jc;
        return ChunkRef{cid * H + h, cid, h, start + jc * kChunk, min(kChunk, len - jc * kChunk), n, jc};
    };
    int rcur = 0;

    ChunkRef cur;
    FChain ch{-1, 0, 0, 0, 0, 0, 0};
    int jcur = 0;
    // Chain change, part q of 4: key tiles q KT/4 .. (q+1) KT/4 - 1 of the
    // finished chain pch go out and the same tiles of chain ch come in.
    // Spread over four phases, the state's 64 KB each way share the CU's
    // memory pipeline with the phases' own traffic instead of arriving as
    // one burst between two chunks.
    FChain pch{-1, 0, 0, 0, 0, 0, 0};
    bool pend = false;
    auto state_swap = [&](int q) {
        if constexpr (FUSED) {
            if (!pend || wave >= VT) return;
            float *dst = fa.state_out ? const_cast<float *>(state_at(fa.state_out, pch)) : nullptr;
            const float *src = fa.state_in && ch.c >= 0 ? state_at(fa.state_in, ch) : nullptr;
#pragma unroll
            for (int u = 0; u < KT / 4; ++u) {
                const int t = q * (KT / 4) + u;
                if (dst) *reinterpret_cast<f32x4 *>(dst + t * kSub) = S[t];
                S[t] = src ? *reinterpret_cast<const f32x4 *>(src + t * kSub) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    if constexpr (FUSED) {
        ch = next_chain((int)blockIdx.x);
        cur = item_of(ch, 0);
        if (ch.c >= 0) state_load(ch);
    } else if (SKIP && nlong >= 0) {
        rcur = __builtin_amdgcn_readfirstlane(sLcum[nlong]) * H - 1 - (int)blockIdx.x;
        cur = find_long(rcur);
    } else {
        const int item0 = c_hi * H - 1 - (int)blockIdx.x;
        cur = find_chunk(item0 / H, item0 % H);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) load_row(cur, r);
    load_beta(cur);
    load_v(cur);
    if constexpr (CONV != 0)
        conv_fetch(cur, cur.item >= 0 ? (cv_slots ? cv_slots[cur.n] : cur.n) : -1);
    // Settle the first chunk's loads here, so that the loop's own prefetches
    // are the only loads in flight at its top.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        settle(kr[r]);
        settle(qr[r]);
        settle(gr[r]);
        if constexpr (CONV != 0) settle(vr[r]);
    }
#pragma unroll
    for (int p = 0; p < VPT; ++p) settle(xv[p]);
    settle(bt);
    if constexpr (CONV != 0) {
        settle(cw_reg);
        settle(ch_reg);
        conv_put();
    }

    // Phase clocks (a KDA_PHASE_CLOCKS build only): lane 0 of each wave of
    // workgroup 0 records the core clock counter at mark i of item clk_it.
    int clk_it = 0;
    auto clock_mark = [&](int i) {
#ifdef KDA_PHASE_CLOCKS
        if (blockIdx.x == 0 && lane == 0 && clk_it < kClockItems)
            g_phase_clock[(((FUSED ? 1 : 0) * kClockWaves + wave) * kClockItems + clk_it) * kClockMarks + i] =
                __builtin_amdgcn_s_memtime();
#else
        (void)i;
#endif
    };
    int buf = 0;
    while (cur.item >= 0) {
        clock_mark(0);
        E *const sKP = sKPb + buf * (kChunk * KPP);
        E *const sV = sVb + buf * LD::V_ELEMS;
        float *const sBs = sBsb + buf * (4 * DK);
        const int C = cur.C;
        const size_t rec = (size_t)(cur.item - c_lo * H);   // = (cid - c_lo) H + h
        E *const Rw = FUSED ? sW : ws + rec * L::kRecElems;
        E *const Rq = FUSED ? sQt : Rw + L::kWElems;
        E *const Rk = FUSED ? sKt : Rq + L::kQElems;
        E *const Ra = FUSED ? sAq : Rk + L::kKElems;
        E *const Ru = Ra + L::kAElems;
        float *const Rd = FUSED ? sDec : ws_dec + rec * DK;
        FChain nch_ch = ch;
        int nj = jcur + 1;
        const ChunkRef nxt = [&]() -> ChunkRef {
            if constexpr (FUSED) {
                if (nj >= ch.nch) {
                    nch_ch = next_chain(ch.c + stride);
                    nj = 0;
                }
                return item_of(nch_ch, nj);
            } else {
                if (SKIP && nlong >= 0) {
                    rcur -= stride;
                    return find_long(rcur);
                }
                int ncid = cur.cid, nh = cur.h;
                step_down(ncid, nh);
                return find_chunk(ncid, nh);
            }
        }();
        // folded conv: the next chunk's slot (its window for a first chunk)
        const int nslot = CONV != 0 && nxt.item >= 0 ? (cv_slots ? cv_slots[nxt.n] : nxt.n) : -1;

        // ---- per-row factors (log2 units); everything derived from k, q, V
        // leaves the registers ----
        if (tid < kChunk) sBeta[tid] = bt;
        if (fthread) {
            if constexpr (CONV != 0) {
                conv_rows(vr, 2, C);
#pragma unroll
                for (int r = 0; r < 4; ++r) *reinterpret_cast<R4 *>(sV + (4 * r4 + r) * VP + ch0) = vr[r];
                conv_rows(qr, 0, C);
                conv_rows(kr, 1, C);
            }
            // gl: inclusive prefix of g over this lane's 4 rows; ex: the sum over
            // the lanes before it (exclusive row scan); Gs, Ge: Gam at the
            // block's first and last rows; total: Gam at the chunk's last row.
            f32x4 gl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) gl[r] = gr[r] * kLog2e;
#pragma unroll
            for (int r = 1; r < 4; ++r) gl[r] += gl[r - 1];
            f32x4 ex, Gs, Ge, total;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float inc = row_scan(gl[3][x]);
                ex[x] = inc - gl[3][x];
                Gs[x] = quad_bcast<0>(ex[x] + gl[0][x]);
                Ge[x] = quad_bcast<3>(inc);
                total[x] = row_bcast<15>(inc);
            }
            const int I = r4 >> 2;
            f32x4 ebs, ce;                             // e^{Gam_s}, e^{Gam_C - Gam_e} of the block
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ebs[x] = fast_exp2(Gs[x]);
                ce[x] = fast_exp2(total[x] - Ge[x]);
            }
            if ((r4 & 3) == 0) {
                *reinterpret_cast<f32x4 *>(sBs + I * DK + ch0) = ebs;
                *reinterpret_cast<f32x4 *>(sCe + I * DK + ch0) = ce;
                bool exd = false;
#pragma unroll
                for (int x = 0; x < 4; ++x) exd |= (Gs[x] - Ge[x]) > kDiagSpanLimit;
                sExact[I * C4 + cq] = exd ? 1 : 0;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * r4 + r;
                const f32x4 gam = ex + gl[r];
                const f32x4 kf = to_f32<E>(kr[r]), qf = to_f32<E>(qr[r]);
                f32x4 kp, qp, kq;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float P = fast_exp2(gam[x] - Gs[x]);
                    const float Qf = fast_exp2(Ge[x] - gam[x]);
                    kp[x] = kf[x] * P;
                    qp[x] = qf[x] * P;
                    kq[x] = kf[x] * Qf;
                }
                store4<E>(sKP + row * KPP + ch0, kp);
                store4<E>(sQP + row * KPP + ch0, qp);
                *reinterpret_cast<f32x4 *>(sKQ + row * KQP + ch0) = kq;
            }
            // F_IJ = e^{Gam_s(I) - Gam_e(J)}, pair I (I + 1) / 2 + J = r, on lanes r < 10
            {
                const int p = r4 < 10 ? r4 : 0;
                const int pI = pair_row(p), pJ = p - pI * (pI + 1) / 2;
                f32x4 F;
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    F[x] = fast_exp2(__shfl(Gs[x], (lane & 48) + 4 * pI) - __shfl(Ge[x], (lane & 48) + 4 * pJ));
                if (r4 < 10) *reinterpret_cast<f32x4 *>(sF + r4 * DK + ch0) = F;
            }
            if (r4 == 15) {
                f32x4 d;
#pragma unroll
                for (int x = 0; x < 4; ++x) d[x] = fast_exp2(total[x]);
                *reinterpret_cast<f32x4 *>(Rd + ch0) = d;
            }
        }
        if constexpr (CONV == 0 && LD::kStage) {
#pragma unroll
            for (int p = 0; p < VPT; ++p) {
                const int u = tid + p * NTH;
                const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
                *reinterpret_cast<uint4 *>(sV + r * VP + c) = xv[p];
            }
        }
        // The raw registers are free: fetch the next chunk's, a part at a time
        // (V, beta and the first row here, one row in each later phase), so
        // that no wave stalls behind a burst of loads.
        load_v(nxt);
        load_beta(nxt);
        load_row(nxt, 0);
        state_swap(0);
        clock_mark(1);
        __syncthreads();
        clock_mark(2);

        // ---- A_kk and A_qk blocks, transposed products: lane (i, g) receives
        // A[16I + i][16J + 4g + r] ----
        auto ablock = [&](int I, int J, f32x4 &accK, f32x4 &accQ) {
            accK = f32x4{0.f, 0.f, 0.f, 0.f};
            accQ = accK;
            const int ra = I * kSub + li, rb = J * kSub + li;
            const float *Fp = sF + (I * (I + 1) / 2 + J) * DK;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int c0 = s * kSlab + 4 * lg, c1 = c0 + 16;
                const Frag<E> aK = frag_from_runs<E>(sKP + ra * KPP + c0, sKP + ra * KPP + c1);
                const Frag<E> aQ = frag_from_runs<E>(sQP + ra * KPP + c0, sQP + ra * KPP + c1);
                const f32x4 b0 = *reinterpret_cast<const f32x4 *>(sKQ + rb * KQP + c0) *
                                 *reinterpret_cast<const f32x4 *>(Fp + c0);
                const f32x4 b1 = *reinterpret_cast<const f32x4 *>(sKQ + rb * KQP + c1) *
                                 *reinterpret_cast<const f32x4 *>(Fp + c1);
                const Frag<E> bK = frag_from_tiles<E>(b0, b1);
                mma(accK, bK, aK);
                mma(accQ, bK, aQ);
            }
        };
        // Exact diagonal block I, for decay spans beyond the split-factor
        // range: lane (i, g) sums A[16I + i][16I + 4g + r] over every channel
        // with one exp per term.  Row 16I + i of the chunk sits in lane i of
        // each 16-lane group, whose shuffle scan yields the prefix sums of g.
        // Slow but light on registers; unscaled, unmasked.
        auto diag_exact = [&](int I, f32x4 &accK, f32x4 &accQ) {
            accK = f32x4{0.f, 0.f, 0.f, 0.f};
            accQ = accK;
            const int row = I * kSub + li;
            const bool in = row < C;
            const size_t base = ((size_t)(cur.row0 + (in ? row : 0)) * H + cur.h) * DK;
#pragma unroll 1
            for (int c0 = 0; c0 < DK; c0 += 4) {
                f32x4 gv = {0.f, 0.f, 0.f, 0.f}, kv = gv, qv = gv;
                if (in) {
                    gv = *reinterpret_cast<const f32x4 *>(g + base + c0);
                    kv = to_f32<E>(*reinterpret_cast<const R4 *>(k + base + c0));
                    qv = to_f32<E>(*reinterpret_cast<const R4 *>(q + base + c0));
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    float G = gv[x] * kLog2e;
#pragma unroll
                    for (int d = 1; d < kSub; d <<= 1) {
                        const float t = __shfl_up(G, d, kSub);
                        if (li >= d) G += t;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 4 * lg + r;
                        const float Gj = __shfl(G, 16 * lg + j);
                        const float kj = __shfl(kv[x], 16 * lg + j);
                        const float e = j <= li ? fast_exp2(G - Gj) : 0.f;
                        accK[r] = fmaf(kv[x] * kj, e, accK[r]);
                        accQ[r] = fmaf(qv[x] * kj, e, accQ[r]);
                    }
                }
            }
        };
        // A_qk block (I, J) is half J % 2 of the scan's fragment (I, J / 2):
        // lane (i, g) holds its elements 4 (J % 2) .. + 3.
        auto put_aqk = [&](int I, int J, const f32x4 &vq) {
            store4<E>(Ra + tri_frag(I, J >> 1) * 512 + lane * 8 + 4 * (J & 1), vq);
        };

        // Waves 0..3: diagonal block I = wave and its inverse by forward
        // substitution (every 16-lane group computes columns 0..15; group 0
        // stores them).  Waves 4..7: the six blocks below the diagonal,
        // (1,0) (3,2) | (2,0) (3,1) | (2,1) | (3,0), and the zero blocks
        // (0,1) and (2,3), which are read as parts of 32-column slabs.
        if (wave < 4) {
            const int I = wave;
            f32x4 dK, dQ;
            if (__any(lane < C4 && sExact[I * C4 + (lane & (C4 - 1))] != 0)) diag_exact(I, dK, dQ);
            else ablock(I, I, dK, dQ);
            const float b = sBeta[I * kSub + li];
            f32x4 vk, vq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 4 * lg + r;
                vk[r] = col < li ? dK[r] * b : 0.f;
                vq[r] = col <= li ? dQ[r] : 0.f;
            }
            put_aqk(I, I, vq);
            if (!(I & 1)) put_aqk(I, I + 1, f32x4{0.f, 0.f, 0.f, 0.f});
            float *D = sD + I * kSub * DP;
            *reinterpret_cast<f32x4 *>(D + li * DP + 4 * lg) = vk;
            // Column jj = li of (I + D)^-1 by forward substitution: row ii
            // sums its terms in the order mm = 0, 1, ..., each as soon as
            // entry mm is final, and takes the sum off the unit vector's
            // entry.  The block was written by this wave only; LDS accesses
            // of a wave complete in order.
            float tcol[kSub];
            if constexpr (sizeof(E) == 2) {
                // The unit vector comes from an opaque bit per item.  Selects
                // on ii < jj and ii == jj would be hoisted out of the item
                // loop as 32 lane masks, spilled to vector-register lanes and
                // read back on the chain: 1.06x slower for the kernel.
                unsigned unit = 1u << li;
                asm volatile("" : "+v"(unit));
#pragma unroll
                for (int ii = 0; ii < kSub; ++ii) {
                    float acc = 0.f;
#pragma unroll
                    for (int mm = 0; mm < ii; ++mm) acc = fmaf(D[ii * DP + mm], tcol[mm], acc);
                    tcol[ii] = (float)__builtin_amdgcn_ubfe(unit, ii, 1) - acc;
                }
            } else {
                // fp32: its raw inputs take twice the registers, which leaves
                // no room for the 16 unit entries; the masks are used instead.
                const int jj = li;
#pragma unroll
                for (int ii = 0; ii < kSub; ++ii) {
                    float acc = 0.f;
#pragma unroll
                    for (int mm = 0; mm < ii; ++mm) acc = fmaf(D[ii * DP + mm], tcol[mm], acc);
                    tcol[ii] = ii < jj ? 0.f : (ii == jj ? 1.f : -acc);
                }
            }
            if (lg == 0) {
#pragma unroll
                for (int ii = 0; ii < kSub; ++ii) sA[(I * kSub + ii) * AP + I * kSub + li] = tcol[ii];
            }
        } else {
            const int w4 = wave - 4;
            const int nb = w4 < 2 ? 2 : 1;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                if (bi >= nb) break;
                const int I = bi == 0 ? (w4 == 0 ? 1 : (w4 == 3 ? 3 : 2)) : 3;
                const int J = bi == 0 ? (w4 == 2 ? 1 : 0) : (w4 == 0 ? 2 : 1);
                f32x4 oK, oQ;
                ablock(I, J, oK, oQ);
                put_aqk(I, J, oQ);
                *reinterpret_cast<f32x4 *>(sA + (I * kSub + li) * AP + J * kSub + 4 * lg) =
                    oK * sBeta[I * kSub + li];
            }
            if (w4 >= 2) {
                const int I = w4 == 2 ? 0 : 2;
                *reinterpret_cast<f32x4 *>(sA + (I * kSub + li) * AP + (I + 1) * kSub + 4 * lg) =
                    f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        load_row(nxt, 1);
        state_swap(1);
        clock_mark(3);
        __syncthreads();   // sA holds A_kk below the diagonal and the diagonal inverses
        clock_mark(4);

        // Q e^Gam = (q P) e^{Gam_s} in the scan's fragment order: fragment
        // (m, s) holds row 16m + i, channels 32s + kk(g, e).
        auto form_q = [&](int f) {
            const int row = (f / KS) * kSub + li, c0 = (f % KS) * kSlab + 4 * lg;
            Frag<E> fr = frag_from_runs<E>(sQP + row * KPP + c0, sQP + row * KPP + c0 + 16);
            const float *eb = sBs + (f / KS) * DK + c0;
#pragma unroll
            for (int e = 0; e < 8; ++e) fr.set(e, fr.get(e) * eb[(e & 3) + 16 * (e >> 2)]);
            store_frag<E>(Rq + f * 512, lane, fr);
        };
        // K e^{Gam_C - Gam}, transposed, in the scan's order: fragment (t, s)
        // holds key channels 16t + i over chunk rows 32s + kk(g, e).
        auto form_k = [&](int f) {
            const int ch = (f >> 1) * kSub + li;
            const float ce0 = sCe[(2 * (f & 1)) * DK + ch], ce1 = sCe[(2 * (f & 1) + 1) * DK + ch];
            Frag<E> fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = (f & 1) * kSlab + kk_of(lg, e);
                fr.set(e, sKQ[row * KQP + ch] * (e < 4 ? ce0 : ce1));
            }
            store_frag<E>(Rk + f * 512, lane, fr);
        };
        // ---- off-diagonal blocks of Tm on fp32 matrix cores ----
        // level 1 (waves 0, 1), in place: Tm_10 = -Tm_11 (A_10 Tm_00), Tm_32 = -Tm_33 (A_32 Tm_22).
        // Meanwhile waves 2..7 write Q e^Gam, or, fused, K e^{Gam_C - Gam}
        // (its k Qf rows then take Q e^Gam and w).
        if (wave >= 2) {
            if constexpr (FUSED) {
                for (int f = wave - 2; f < 2 * KT; f += 6) form_k(f);
            } else {
                for (int f = wave - 2; f < 4 * KS; f += 6) form_q(f);
            }
        }
        if (wave < 2) {
            const int I = wave ? 3 : 1, J = I - 1;
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                P = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(I * kSub + li) * AP + J * kSub + lg + 4 * ks],
                                                         sA[(J * kSub + lg + 4 * ks) * AP + J * kSub + li], P, 0, 0, 0);
            // P in C layout is the A operand of P^T with contraction index
            // 4g + r, so (Tm_II P)^T = P^T Tm_II^T leaves lane (i, g) holding
            // row i, columns 4g .. 4g + 3 of Tm_IJ: one 16-byte row store, and
            // the left half of Tm diag(beta) fragment (I, J / 2)
            f32x4 Tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Tt = __builtin_amdgcn_mfma_f32_16x16x4f32(P[r], sA[(I * kSub + li) * AP + I * kSub + 4 * lg + r], Tt, 0, 0, 0);
            Tt = -Tt;
            *reinterpret_cast<f32x4 *>(sA + (I * kSub + li) * AP + J * kSub + 4 * lg) = Tt;
            store4<E>(sTb + tri_frag(I, J >> 1) * 512 + lane * 8 + 4 * (J & 1),
                      Tt * *reinterpret_cast<const f32x4 *>(sBeta + J * kSub + 4 * lg));
        }
        if (wave >= 4) {
            // the diagonal half of Tm diag(beta) fragment (I, I / 2), I = wave - 4
            const int I = wave - 4;
            store4<E>(sTb + tri_frag(I, I >> 1) * 512 + lane * 8 + 4 * (I & 1),
                      *reinterpret_cast<const f32x4 *>(sA + (I * kSub + li) * AP + I * kSub + 4 * lg) *
                          *reinterpret_cast<const f32x4 *>(sBeta + I * kSub + 4 * lg));
        }
        load_row(nxt, 2);
        state_swap(2);
        clock_mark(5);
        __syncthreads();
        clock_mark(6);
        // level 2 (waves 0..3, output tile (ti, tj)), straight into the Tm
        // diag(beta) fragments (2 + ti, 0): Tm[32:64, 0:32] = -Tm_hi (A[32:64, 0:32] Tm_lo).
        // Meanwhile waves 4..7 write K e^{Gam_C - Gam}, or, fused, Q e^Gam.
        if (wave >= 4) {
            if constexpr (FUSED) {
                for (int f = wave - 4; f < 4 * KS; f += 4) form_q(f);
            } else {
                for (int f = wave - 4; f < 2 * KT; f += 4) form_k(f);
            }
        }
        if (wave < 4) {
            const int ti = wave >> 1, tj = wave & 1;
            f32x4 Qt[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                Qt[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
                    Qt[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        sA[(32 + kt * kSub + li) * AP + lg + 4 * ks],
                        sA[(lg + 4 * ks) * AP + tj * kSub + li], Qt[kt], 0, 0, 0);
            }
            // transposed as in level 1: lane (i, g) receives row i, columns
            // 4g .. 4g + 3 of the tile
            f32x4 Tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Tt = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        Qt[kt][r], sA[(32 + ti * kSub + li) * AP + 32 + kt * kSub + 4 * lg + r], Tt, 0, 0, 0);
            }
            store4<E>(sTb + tri_frag(2 + ti, 0) * 512 + lane * 8 + 4 * tj,
                      -Tt * *reinterpret_cast<const f32x4 *>(sBeta + tj * kSub + 4 * lg));
        }
        load_row(nxt, 3);
        conv_fetch(nxt, nslot);
        state_swap(3);
        pend = false;
        clock_mark(7);
        __syncthreads();
        clock_mark(8);

        // ---- w and u on the matrix cores, with diag(beta) folded into Tm ----
        // fragment (m, s) of Tm diag(beta): row 16 m + i, columns 32 s + kk(g, e)
        auto tm_frag = [&](int m, int s) { return load_frag<E>(sTb + tri_frag(m, s) * 512, lane); };
        // w: wave owns d_k slab `wslab` of row tiles wm0 .. wm0 + MPW - 1;
        // u: wave owns value tile `wave` (if any)
        const int wslab = wave % KS, wm0 = (wave / KS) * MPW;
        const int smax = (wm0 + MPW - 1) >> 1;
        if (wave < VT) {
            // u tile (value columns 16 wave ..): Tm diag(beta) V, lane (i, g)
            // holds u[16m + 4g + r][16 wave + i]; V fragments: value column
            // 16 wave + i, rows 32 s + kk(g, e)
            Frag<E> vf[2];
            if constexpr (LD::kStage) {
#pragma unroll
                for (int s = 0; s < 2; ++s) vf[s] = frag_cols<E>(sV, VP, s * kSlab, wave * kSub, lane);
            } else {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = s * kSlab + kk_of(lg, e);
                        vf[s].set(e, row < C ? (float)v[((size_t)(cur.row0 + row) * H + cur.h) * DV + wave * kSub + li]
                                             : 0.f);
                    }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma(acc, tm_frag(m, 0), vf[0]);
                if (m >= 2) mma(acc, tm_frag(m, 1), vf[1]);
                if constexpr (FUSED) {
                    ureg[m] = bf16x4{(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
                } else {
                    store4<E>(Ru + wave * (64 * 16) + m * 256 + lane * 4, acc);
                }
            }
        }
        {
            // w slab `wslab`, computed transposed as X^T Tm^T: lane (i, g)
            // receives w[16m + i][32 wslab + kk(g, e)], the scan's A-operand
            // order.  K e^Gam fragments: channel 16 (2 wslab + nn) + i, rows
            // 32 s + kk(g, e).
            Frag<E> xf[2][2];
#pragma unroll
            for (int nn = 0; nn < 2; ++nn)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s > smax) continue;
                    const int n0 = (2 * wslab + nn) * kSub;
                    xf[nn][s] = frag_cols<E>(sKP, KPP, s * kSlab, n0, lane);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xf[nn][s].set(e, xf[nn][s].get(e) * sBs[(2 * s + (e >> 2)) * DK + n0 + li]);
                }
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi) {
                const int m = wm0 + mi;
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s > (m >> 1)) break;
                    const Frag<E> t = tm_frag(m, s);
                    mma(acc0, xf[0][s], t);
                    mma(acc1, xf[1][s], t);
                }
                store_frag<E>(Rw + (m * KS + wslab) * 512, lane, frag_from_tiles<E>(acc0, acc1));
            }
        }
        // Single-buffered, LDS is rewritten by the next chunk.  Double-
        // buffered, the next chunk's factor phase writes only buffers that
        // w and u no longer read, and its first barrier orders everything
        // after it behind this chunk's w and u.
        conv_put();                                    // the next chunk's taps and halo
        clock_mark(9);
        if constexpr (LD::NB == 1) __syncthreads();
        clock_mark(10);
        if constexpr (FUSED) {
            // ---- the chunk's state step, wave w < d_v / 16 on its slice:
            // U = u - w S, O = Q~ S + A_qk U, S = diag(e^{Gam_C}) S + K~^T U,
            // all operands from LDS but u (this wave's registers) ----
            if (wave < VT) {
                Frag<E> SB[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s) SB[s] = frag_from_tiles<E>(S[2 * s], S[2 * s + 1]);
                // row tile m of U: lane holds U[16m + 4g + r][16 wave + i]
                f32x4 U[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) U[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int m = 0; m < 4; ++m) mma(U[m], load_frag<E>(sW + (m * KS + s) * 512, lane), SB[s]);
#pragma unroll
                for (int m = 0; m < 4; ++m) U[m] = raw_to_f32(ureg[m]) - U[m];
                Frag<E> UB[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) UB[s] = frag_from_tiles<E>(U[2 * s], U[2 * s + 1]);
                // O, transposed: lane holds row 16m + i, columns 16 wave + 4g + r
                f32x4 O[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) mma(O[m], SB[s], load_frag<E>(sQt + (m * KS + s) * 512, lane));
#pragma unroll
                    for (int s = 0; s <= (m >> 1); ++s)
                        mma(O[m], UB[s], load_frag<E>(sAq + tri_frag(m, s) * 512, lane));
                }
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    S[t] *= *reinterpret_cast<const f32x4 *>(sDec + t * kSub + 4 * lg);
                    mma(S[t], load_frag<E>(sKt + (2 * t) * 512, lane), UB[0]);
                    mma(S[t], load_frag<E>(sKt + (2 * t + 1) * 512, lane), UB[1]);
                }
                E *const orow = static_cast<E *>(fa.o) + ((size_t)(cur.row0 + li) * H + cur.h) * DV +
                                wave * kSub + 4 * lg;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (m * kSub + li < C) store4<E>(orow + (size_t)m * kSub * H * DV, O[m] * fa.scale);
            }
            clock_mark(11);
            __syncthreads();   // the next chunk's factor phase rewrites every operand
            clock_mark(12);
            if (nj == 0) {     // the chain is done: its state goes out and the next
                pch = ch;      // chain's comes in a quarter at a time over the next
                ch = nch_ch;   // chunk's first four phases (state_swap)
                pend = true;
            }
            jcur = nj;
            clock_mark(13);
        }
        buf ^= LD::NB - 1;
        cur = nxt;
        ++clk_it;
    }
    if constexpr (FUSED) {
        if (pend) state_store(pch);   // the last chain's state (no chunk followed it)
    }
}

// SKIP: pass over the chunks of sequences of at most fuse_max chunks (the
// fused prefill's); a separate instantiation, since the test in the chunk
// walk costs the plain kernel about a microsecond.
// CONV: 1 or 2 with the short conv folded into the loads (no activation or
// SiLU); q, k and v are then the raw inputs.
template <typename E, int DK, int DV, bool SKIP, int CONV>
__global__ __launch_bounds__(kIntraThreads, 1) void kda_intra_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int H, int c_lo, int c_hi,
    E *__restrict__ ws, float *__restrict__ ws_dec, int fuse_max, ConvFold<E> cf) {
    FuseArgs fa{};
    fa.fuse_max = fuse_max;
    intra_chunks<E, DK, DV, false, SKIP, CONV>(q, k, v, g, beta, cu, T, N, H, c_lo, c_hi, ws, ws_dec,
                                               fa, cf);
}

template <int DK, int DV>
__global__ __launch_bounds__(kIntraThreads, 1) void kda_fused_prefill_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int H, FuseArgs fa) {
    intra_chunks<bf16, DK, DV, true, false>(q, k, v, g, beta, cu, T, N, H, 0, 0, nullptr, nullptr, fa);
}

// ---------------------------------------------------------------------------
// State scan
// ---------------------------------------------------------------------------

// Operands of one chunk for one wave (row tile m = wave, TPW key tiles).
template <typename E, int DK, int NS> struct ScanStage {
    static constexpr int KS = DK / kSlab;
    static constexpr int TPW = DK / 64;
    Frag<E> wf[KS], qf[KS], af[2], kf[TPW][2];
    typename Raw4<E>::type u[NS];              // per slice; raw: converted where it is used
    float d;                                   // e^{Gam_C} of key row 16 TPW wave + (lane % (16 TPW))
    int pf;                                    // L2 warm-up word (first stage of the rotation only)
};

// Work order of the scan kernels.  Sequences are taken longest first (for up
// to 64 sequences; every wave ranks them the same way), then head by head;
// (sequence, head) pairs are dealt round robin to the 8 XCDs (workgroups go
// to XCD b % 8), so each XCD gets an equal share of every sequence, while the
// JT column groups of one pair stay on one XCD and share its L2.
struct ScanWork {
    int n, h, j;        // sequence (by rank), head, column group
    bool valid;
};
__device__ __forceinline__ ScanWork scan_work(int b, int B, int N, int H, int JT, const int32_t *cu,
                                              int T, int lane) {
    const int NP = N * H;
    int q, j;
    if (NP % 8 == 0) {
        const int k = b >> 3;
        j = k % JT;
        q = (k / JT) * 8 + (b & 7);
    } else {
        j = b % JT;
        q = b / JT;
    }
    ScanWork w{0, 0, j, q < NP && b < B};
    if (!w.valid) return w;
    w.h = q % H;
    int n = q / H;
    if (N <= 64) {
        const int lane_len = lane < N ? seq_span(cu, lane, T).len : -1;
        int rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = __shfl(lane_len, m);
            rank += (lm > lane_len || (lm == lane_len && m < lane)) ? 1 : 0;
        }
        const unsigned long long hit = __ballot(lane < N && rank == n);
        n = hit ? __ffsll((long long)hit) - 1 : n;
    }
    w.n = n;
    return w;
}

template <typename E, int DK, int DV, int NS>
__global__ __launch_bounds__(256, 1) void kda_scan_kernel(
    const E *__restrict__ ws, const float *__restrict__ ws_dec,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots,
    const float *state_in, float *state_out, E *__restrict__ o,
    int T, int N, int H, int num_slots, float scale, int64_t slot_stride, int64_t head_stride,
    int c_lo, int c_hi, float *__restrict__ carry, int fuse_max) {
    constexpr int VT = DV / kSub, KS = DK / kSlab;
    constexpr int TPW = DK / 64;                       // key tiles per wave
    using L = WsLayout<E, DK, DV>;
    using Stage = ScanStage<E, DK, NS>;
    // Register stages of chunk operands in flight, at one workgroup per CU:
    // a second workgroup on a CU does not take records in any faster (with
    // more slices than CUs it doubles the CU's time), while deeper stages
    // keep more loads in flight.  One slice (bf16): five.  Two or four
    // slices, whose extra S, u and output tiles take registers: three (16
    // packed sequences: 253.4 -> 251.0 us a step against two stages at two
    // workgroups per CU).  fp32, one slice: three, with the L2 warm-up, which
    // rides on the one-slice three-stage rotation only.  Five stages pull
    // records as fast as three with the warm-up, without the warm-up's extra
    // touches of record lines, which slow the next call's intra-chunk kernel
    // by about 3 us on one 8192-row sequence.
    constexpr int STAGES = NS > 1 ? 3 : (sizeof(E) == 2 ? 5 : 3);
    static_assert(STAGES >= 2 && STAGES <= 5, "register stages");
    constexpr bool kWarm = NS == 1 && STAGES == 3;
    // rounded copies of the state slabs and of U, [slice][slab][lane][8]
    __shared__ __align__(16) E sSb[NS * KS * 64 * 8];
    __shared__ __align__(16) E sUb[NS * 2 * 64 * 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const ScanWork wk = scan_work(blockIdx.x, gridDim.x, N, H, VT / NS, cu, T, lane);
    if (!wk.valid) return;
    const int h = wk.h, n = wk.n, jt = wk.j;           // jt: group of NS slices
    const int slot = slots ? slots[n] : n;
    if (slots && (slot < 0 || slot >= num_slots)) return;   // padded sequence
    const SeqSpan sp = seq_span(cu, n, T);
    const int j0 = jt * NS * kSub;                     // first column; slice ns at j0 + 16 ns
    // This launch's chunks of the sequence: those whose ids lie in the window
    // [c_lo, c_hi).  The state comes from state_in at the sequence's first
    // chunk and from the carry buffer after an earlier window; it goes to
    // state_out after the last chunk and to the carry buffer otherwise.  A
    // sequence with no rows is passed through by the window that holds its
    // (empty) first chunk id.
    const int nch_all = (sp.len + kChunk - 1) / kChunk;
    if (nch_all <= fuse_max) return;                   // a fused chain
    const int j_lo = max(0, c_lo - sp.first_chunk);
    const int j_hi = min(nch_all, c_hi - sp.first_chunk);
    if (nch_all == 0 ? (sp.first_chunk < c_lo || sp.first_chunk >= c_hi) : j_lo >= j_hi) return;
    const bool first_part = j_lo == 0, last_part = j_hi == nch_all;
    float *const carry_blk = carry + ((size_t)n * H + h) * ((size_t)DV * DK);

    // my key tiles t = wave * TPW + i of slice ns, C layout: lane holds
    // S[16t + 4g + r][j0 + 16 ns + i]
    f32x4 S[NS][TPW];
    const float *s_src = first_part ? (state_in ? state_in + slot * slot_stride + h * head_stride
                                                : nullptr)
                                    : carry_blk;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        if (s_src) {
            const float *src = s_src + (size_t)(j0 + ns * kSub + li) * DK;
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                S[ns][i] = *reinterpret_cast<const f32x4 *>(src + (wave * TPW + i) * kSub + 4 * lg);
        } else {
#pragma unroll
            for (int i = 0; i < TPW; ++i) S[ns][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // The state load is settled once the first stages' loads are issued
    // behind it (so both latencies overlap) and before the chunk loop:
    // otherwise the wait inserted for it at the top of the loop would also
    // drain every prefetched chunk.
    auto settle_state = [&]() {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = S[ns][i][r];
                    asm volatile("" : "+v"(x));
                    S[ns][i][r] = x;
                }
            }
    };

    // Record of chunk cc, by part; each part of a stage is refilled with the
    // chunk STAGES ahead as soon as its last use in the current step has been
    // issued, so loads trickle out between the matrix-core products instead
    // of queueing behind them in one burst.
    // chunks j_lo .. j_hi - 1 of the sequence, renumbered from 0
    const int nch = j_hi - j_lo;
    auto rec_of = [&](int cc) { return (size_t)(sp.first_chunk + j_lo + cc - c_lo) * H + h; };
    // L2 warm-up.  All slices of a head ask for the same record lines at
    // about the same time, so without it most operand loads wait on an L2
    // miss still in flight.  Whenever the first stage of the rotation is
    // refilled with chunk c, the waves of the head's slices touch the
    // 128-byte lines of the records of chunks c + kScanWarmAhead .. + 2: the
    // VT / NS * 4 waves take the three records in turn, 64 lines a wave and one
    // word a lane, so the operand loads mostly hit in L2.  The word is
    // consumed when the stage is, three steps later, so nothing waits for it.
    constexpr int kRecLines = (int)((L::kRecElems * sizeof(E) + 127) / 128);
    const int pf_wave = jt * 4 + wave;                 // uniform
    const int pf_rec = pf_wave % 3, pf_line = min((pf_wave / 3) * 64 + lane, kRecLines - 1);
    auto load_w = [&](Stage &X, int cc, bool warm) {
        if (warm) {
            const int cw = min(cc + kScanWarmAhead + pf_rec, nch - 1);
            X.pf = reinterpret_cast<const int *>(ws + rec_of(cw) * L::kRecElems)[pf_line * 32];
        }
        const E *Rw = ws + rec_of(cc) * L::kRecElems;
#pragma unroll
        for (int s = 0; s < KS; ++s) X.wf[s] = load_frag<E>(Rw + (wave * KS + s) * 512, lane);
        const E *Ru = Rw + L::kWElems + L::kQElems + L::kKElems + L::kAElems;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
            X.u[ns] = *reinterpret_cast<const typename Raw4<E>::type *>(
                Ru + (jt * NS + ns) * (64 * 16) + wave * 256 + lane * 4);
    };
    auto load_q = [&](Stage &X, int cc) {
        const E *Rq = ws + rec_of(cc) * L::kRecElems + L::kWElems;
#pragma unroll
        for (int s = 0; s < KS; ++s) X.qf[s] = load_frag<E>(Rq + (wave * KS + s) * 512, lane);
    };
    auto load_k = [&](Stage &X, int cc) {
        const size_t rec = rec_of(cc);
        const E *Rk = ws + rec * L::kRecElems + L::kWElems + L::kQElems;
        const E *Ra = Rk + L::kKElems;
        X.af[0] = load_frag<E>(Ra + tri_frag(wave, 0) * 512, lane);
        // waves 0 and 1 have no second fragment: they reload their first,
        // which the L1 serves, instead of pulling an unused kilobyte
        X.af[1] = load_frag<E>(Ra + tri_frag(wave, wave >= 2 ? 1 : 0) * 512, lane);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave * TPW + i;
            X.kf[i][0] = load_frag<E>(Rk + (t * 2) * 512, lane);
            X.kf[i][1] = load_frag<E>(Rk + (t * 2 + 1) * 512, lane);
        }
        // this wave's 16 TPW decay factors, one per lane (lanes repeat them)
        X.d = ws_dec[rec * DK + wave * (TPW * kSub) + (lane & (TPW * kSub - 1))];
    };
    auto load_stage = [&](Stage &X, int cc, bool warm) {
        load_w(X, cc, warm);
        load_k(X, cc);
        load_q(X, cc);
    };

    // Refills are unconditional (clamped to the last chunk) inside the main
    // loop: a conditional load would leave a stage register holding either
    // the old or the new value, and the copy that merges them waits for
    // every load in flight.
    // Phase clocks (a KDA_PHASE_CLOCKS build only): lane 0 of each wave of
    // workgroup 0 (the longest chain's first slice group) records the core
    // clock counter at mark i of step cc.
    auto clock_mark = [&](int cc, int i) {
#ifdef KDA_PHASE_CLOCKS
        if (blockIdx.x == 0 && lane == 0 && cc < kClockItems)
            g_phase_clock[((2 * kClockWaves + wave) * kClockItems + cc) * kClockMarks + i] =
                __builtin_amdgcn_s_memtime();
#else
        (void)cc; (void)i;
#endif
    };
    // A step's tail: the A_qk U part of its output, the output store and
    // the refill of its stage's last part.  With several slices the tail of
    // step cc runs in step cc + 1, after that step's first barrier, where it
    // no longer delays the next publication of S: nothing on the state's
    // dependent chain (S -> U -> S) waits for it (16 packed sequences: scan
    // 102.2 -> 100.2 us).  o0, o1 and ub carry a step's values to its tail.
    constexpr bool kDeferTail = NS > 1;
    static_assert(!(kDeferTail && kWarm), "the warm-up rotation runs one slice");
    f32x4 o0[NS], o1[NS];
    Frag<E> ub[NS][2];
    // my tile of O = Q~ S + A_qk U, transposed: lane holds row 16 wave + i,
    // columns j0 + 16 ns + 4g + r
    auto tail_mma = [&](Stage &X) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            mma(o0[ns], ub[ns][0], X.af[0]);
            if (wave >= 2) {
                if constexpr (KDA_SINGLE_CHAIN && NS > 1) mma(o0[ns], ub[ns][1], X.af[1]);
                else mma(o1[ns], ub[ns][1], X.af[1]);
            }
        }
    };
    auto tail_out = [&](Stage &X, int cc, bool refill) {
        const int nx = cc + STAGES < nch ? cc + STAGES : nch - 1;
        if (refill) load_k(X, nx);
        const int row = wave * kSub + li;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
            if (row < sp.len - (j_lo + cc) * kChunk)
                store4<E>(o + ((size_t)(sp.start + (j_lo + cc) * kChunk + row) * H + h) * DV + j0 + ns * kSub + 4 * lg,
                          (o0[ns] + o1[ns]) * scale);
    };
    // Step cc on stage X; Xp is the previous step's stage, whose tail is
    // pending when tail_p (deferred tails only), refilled when refill_p.
    auto step = [&](Stage &X, int cc, bool refill, bool warm, Stage &Xp, bool tail_p, bool refill_p) {
        const int nx = cc + STAGES < nch ? cc + STAGES : nch - 1;
        clock_mark(cc, 0);
        // publish my state tiles (rounded to E) and read every slab
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int t = wave * TPW + i;
                store4<E>(sSb + ns * (KS * 512) + ((t >> 1) * 64 + lane) * 8 + (t & 1) * 4, S[ns][i]);
            }
        __syncthreads();
        clock_mark(cc, 1);
        if (warm) asm volatile("" ::"v"(X.pf));   // the warm-up word, loaded three steps ago
        // this step's decay factors, one per key row of my tiles
        float dfac[TPW][4];
        auto shuffle_decay = [&]() {
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) dfac[i][r] = __shfl(X.d, i * kSub + 4 * lg + r);
        };
        if constexpr (kDeferTail) {
            shuffle_decay();
            if (tail_p) {
                tail_mma(Xp);
                tail_out(Xp, cc - 1, refill_p);
            }
        }
        // per slice: my tile of U = u - w S (two independent accumulation
        // chains), and the Q~ S part of the output, which does not need U
        f32x4 un[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            Frag<E> Sb[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) Sb[s] = load_frag<E>(sSb + ns * (KS * 512) + s * 512, lane);
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
            o0[ns] = f32x4{0.f, 0.f, 0.f, 0.f};
            o1[ns] = o0[ns];
            if constexpr (KDA_SINGLE_CHAIN && NS > 1) {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    mma(a0, X.wf[s], Sb[s]);
                    mma(o0[ns], Sb[s], X.qf[s]);
                }
                un[ns] = to_f32<E>(X.u[ns]) - a0;
            } else {
#pragma unroll
                for (int s = 0; s < KS; s += 2) {
                    mma(a0, X.wf[s], Sb[s]);
                    mma(a1, X.wf[s + 1], Sb[s + 1]);
                }
                un[ns] = to_f32<E>(X.u[ns]) - (a0 + a1);
#pragma unroll
                for (int s = 0; s < KS; s += 2) {
                    mma(o0[ns], Sb[s], X.qf[s]);
                    mma(o1[ns], Sb[s + 1], X.qf[s + 1]);
                }
            }
        }
        // the decay of my state tiles (their undecayed copy is in LDS)
        auto apply_decay = [&](bool pin) {
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
#pragma unroll
                for (int i = 0; i < TPW; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = S[ns][i][r] * dfac[i][r];
                        if (pin) asm volatile("" : "+v"(x));
                        S[ns][i][r] = x;
                    }
        };
        // With several slices the multiplies stay here, among the products
        // above: left to the compiler they and the shuffles they wait on
        // sink to the top of the state update, on the dependent chain.
        if constexpr (kDeferTail) apply_decay(true);
        clock_mark(cc, 2);
        if (refill) load_w(X, nx, warm);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
            store4<E>(sUb + ns * 1024 + ((wave >> 1) * 64 + lane) * 8 + (wave & 1) * 4, un[ns]);
        if (refill) load_q(X, nx);
        if constexpr (!kDeferTail) {
            shuffle_decay();
            apply_decay(false);
        }
        __syncthreads();
        clock_mark(cc, 3);
        // every slice's U at once: one LDS round trip before the products
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            ub[ns][0] = load_frag<E>(sUb + ns * 1024, lane);
            ub[ns][1] = load_frag<E>(sUb + ns * 1024 + 512, lane);
        }
        if constexpr (!kDeferTail) tail_mma(X);
        // my key tiles of S = diag(e^{Gam_C}) S + K~^T U
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                mma(S[ns][i], X.kf[i][0], ub[ns][0]);
                mma(S[ns][i], X.kf[i][1], ub[ns][1]);
            }
        if constexpr (!kDeferTail) tail_out(X, cc, refill);
        clock_mark(cc, 4);
    };

    if (nch > 0) {
        if constexpr (!kWarm) {
            // step k runs on stage k % STAGES
            Stage X[STAGES];
#pragma unroll
            for (int i = 0; i < STAGES; ++i) load_stage(X[i], i < nch ? i : nch - 1, false);
            settle_state();
            int cc = 0;
            for (; cc + STAGES - 1 < nch; cc += STAGES) {
#pragma unroll
                for (int i = 0; i < STAGES; ++i)
                    step(X[i], cc + i, true, false, X[(i + STAGES - 1) % STAGES], cc + i > 0, true);
            }
#pragma unroll
            for (int i = 0; i < STAGES - 1; ++i)
                if (cc + i < nch)
                    step(X[i], cc + i, false, false, X[(i + STAGES - 1) % STAGES], cc + i > 0, i == 0);
            if constexpr (kDeferTail) {
                // the last step's tail (its stage needs no refill)
#pragma unroll
                for (int i = 0; i < STAGES; ++i)
                    if ((nch - 1) % STAGES == i) {
                        tail_mma(X[i]);
                        tail_out(X[i], nch - 1, false);
                    }
            }
        } else {
            Stage A, Bs, Cs;
            load_stage(A, 0, kWarm);
            load_stage(Bs, nch > 1 ? 1 : 0, false);
            load_stage(Cs, nch > 2 ? 2 : nch - 1, false);
            settle_state();
            int cc = 0;
            for (; cc + 2 < nch; cc += 3) {
                step(A, cc, true, kWarm, Cs, false, false);
                step(Bs, cc + 1, true, false, A, false, false);
                step(Cs, cc + 2, true, false, Bs, false, false);
            }
            if (cc < nch) step(A, cc, false, kWarm, Cs, false, false);
            if (cc + 1 < nch) step(Bs, cc + 1, false, false, A, false, false);
        }
    }

    float *const s_dst = last_part ? (state_out ? state_out + slot * slot_stride + h * head_stride
                                                : nullptr)
                                   : carry_blk;
    if (s_dst) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            float *dst = s_dst + (size_t)(j0 + ns * kSub + li) * DK;
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                *reinterpret_cast<f32x4 *>(dst + (wave * TPW + i) * kSub + 4 * lg) = S[ns][i];
        }
    }
}

template <typename E, int DK, int DV>
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    const PrefillPlan pl = prefill_plan(a.T, a.N, a.H, DK, DV, sizeof(E) == 2, a.window_chunks);
    const FuseArgs fa{a.slots, a.state_in, a.state_out, a.o, a.num_slots, a.scale,
                      a.slot_stride, a.head_stride,
                      prefill_fuse_max(a.T, a.N, a.H, sizeof(E) == 2, a.fuse_chunks)};
    char *const base = reinterpret_cast<char *>(a.workspace);
    E *const ws = reinterpret_cast<E *>(base);
    float *const ws_dec = reinterpret_cast<float *>(base + pl.dec_offset);
    float *const carry = reinterpret_cast<float *>(base + pl.carry_offset);
    // An error left by an unrelated earlier call is not this call's: clear
    // it, so that the checks below see only this call's launches.
    (void)hipGetLastError();
    int ev = 0;
    auto mark = [&]() {
        if (ev < a.num_events && a.events[ev]) (void)hipEventRecord(a.events[ev], stream);
        ++ev;
    };
    // The scan is bound by the record bytes each CU takes in, and a workgroup
    // of NS 16-column slices takes them in once for all NS.  So each call
    // gets the largest NS (1, 2 or 4; bf16 for NS > 1) that still leaves at
    // least one workgroup per CU.
    const long long slices = (long long)a.N * a.H * (DV / kSub);
    auto scan = [&](auto ns, int c_lo, int c_hi) -> hipError_t {
        constexpr int NS = decltype(ns)::value;
        kda_scan_kernel<E, DK, DV, NS><<<dim3((int)(slices / NS)), dim3(256), 0, stream>>>(
            ws, ws_dec, a.cu_seqlens, a.slots, a.state_in, a.state_out, static_cast<E *>(a.o),
            a.T, a.N, a.H, a.num_slots, a.scale, a.slot_stride, a.head_stride, c_lo, c_hi, carry,
            fa.fuse_max);
        return hipGetLastError();
    };
    auto scan_window = [&](int c_lo, int c_hi) -> hipError_t {
        if constexpr (sizeof(E) == 2) {
            if (slices >= 4LL * a.num_cus) return scan(std::integral_constant<int, 4>{}, c_lo, c_hi);
            if (slices >= 2LL * a.num_cus) return scan(std::integral_constant<int, 2>{}, c_lo, c_hi);
        }
        return scan(std::integral_constant<int, 1>{}, c_lo, c_hi);
    };
    // Windows of chunk ids, each an intra launch that writes its records and
    // a scan launch that reads them while they are recent (the workspace
    // holds one window's records and is reused by the next).
    mark();
    // No sequence has more than T rows: when the fused prefill takes
    // sequences of T rows, the intra-chunk kernel and scan have nothing to do.
    const bool all_fused = fa.fuse_max >= 0 && (long long)fa.fuse_max * kChunk >= a.T;
    for (int w = 0; w < pl.windows && !all_fused; ++w) {
        const int c_lo = w * pl.window_chunks;
        const int c_hi = c_lo + pl.window_chunks < pl.chunk_ids ? c_lo + pl.window_chunks : pl.chunk_ids;
        const long long items = (long long)(c_hi - c_lo) * a.H;
        const int grid = (int)(items < (long long)a.num_cus ? items : (long long)a.num_cus);
        auto intra = fa.fuse_max >= 0 ? kda_intra_kernel<E, DK, DV, true, 0>
                                      : kda_intra_kernel<E, DK, DV, false, 0>;
        ConvFold<E> cf{};
        if constexpr (sizeof(E) == 2 && DK == DV) {
            if (a.conv) {
                // the conv folded into the loads; the call never fuses then
                intra = a.conv->silu ? kda_intra_kernel<E, DK, DV, false, 2>
                                     : kda_intra_kernel<E, DK, DV, false, 1>;
                cf = ConvFold<E>{a.conv->weight, static_cast<const E *>(a.conv->window), a.conv->win,
                                 a.conv->slots, a.conv->num_slots};
            }
        }
        intra<<<dim3(grid), dim3(kIntraThreads), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            a.g, a.beta, a.cu_seqlens, a.T, a.N, a.H, c_lo, c_hi, ws, ws_dec, fa.fuse_max, cf);
        // A failed intra launch leaves stale records: the scan must not run
        // on them and overwrite o and the caller's states.
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        mark();
        e = scan_window(c_lo, c_hi);
        if (e != hipSuccess) return e;
        mark();
    }
    if (a.conv) {
        // each sequence's conv window, now that no intra-chunk launch reads it
        const hipError_t e = launch_conv_window<E, DK, DV>(*a.conv, stream);
        if (e != hipSuccess) return e;
    }
    if constexpr (sizeof(E) == 2) {
        if (fa.fuse_max >= 0) {
            const long long chains = (long long)a.N * a.H;
            const int grid = (int)(chains < (long long)a.num_cus ? chains : (long long)a.num_cus);
            kda_fused_prefill_kernel<DK, DV><<<dim3(grid), dim3(kIntraThreads), 0, stream>>>(
                static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
                a.g, a.beta, a.cu_seqlens, a.T, a.N, a.H, fa);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            mark();
        }
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free prefill
// ---------------------------------------------------------------------------

// Every GPU the library runs kda_chunk_prefill_static on holds its own copy
// of this array until the process ends.  In host code its name is only a
// stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[KDA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t static_scratch(hipStream_t stream, void **ptr) {
    int dev = 0;
    if (!stream || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // the symbol's address on `dev`, looked up with `dev` current
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

PrefillPlan prefill_plan(int T, int N, int H, int dk, int dv, bool bf16, int window_chunks) {
    PrefillPlan p;
    const size_t es = bf16 ? 2 : 4;
    const size_t rec = ((size_t)kChunk * (3 * dk + dv) + 6 * 512) * es;
    p.chunk_ids = chunk_id_count(T, N);
    // Default: two windows for calls with few (sequence, head) pairs and
    // enough chunks, one otherwise.  Such calls scan long chains with one
    // slice per workgroup, which take records in at a per-CU rate that is
    // higher when they come from the last-level cache; half the records of
    // an 8192-row call (150 MB at H = 32) stay there until the scan reads
    // them (one 8192-row sequence at H = 32: scan 129 -> 109 us, intra
    // 131 -> 145 us, step 256 -> 244 us).  Calls with many pairs run many
    // short chains whose workgroups would each start twice (16 packed
    // sequences: step 258 -> 277 us with two windows).  An 8192-row sequence
    // has 128 chunk ids, so each of its windows holds 64 chunks x 32 heads =
    // 8 whole rounds of a 256-workgroup grid; an id count of T / 64 + N gave
    // the first window 65 chunks and a ninth round for 32 of its workgroups
    // (step 242 -> 232 us, intra 143 -> 137 us).
    size_t wc = (size_t)p.chunk_ids;
    if (window_chunks > 0) wc = (size_t)window_chunks;
    else if ((long long)N * H <= 64 && p.chunk_ids >= 32) wc = ((size_t)p.chunk_ids + 1) / 2;
    if (wc < 1) wc = 1;
    p.windows = (int)(((size_t)p.chunk_ids + wc - 1) / wc);
    if (p.windows < 1) p.windows = 1;
    p.window_chunks = (p.chunk_ids + p.windows - 1) / p.windows;
    const size_t recs = (size_t)p.window_chunks * H;
    p.dec_offset = recs * rec;
    p.carry_offset = (p.dec_offset + recs * (size_t)dk * 4 + 255) / 256 * 256;
    const size_t carry = p.windows > 1 ? (size_t)N * H * dv * dk * 4 : 0;
    p.bytes = p.carry_offset + carry;
    return p;
}

// The fused kernel runs a chain's chunks one after another at about 10 us a
// chunk, which beats the intra-chunk kernel plus scan only for short chains: 16 packed sequences (average 8 chunks,
// longest 37) 250 us a step with none fused, 258 us fusing those of up to
// 2 chunks; 128 sequences averaging one chunk 457 -> 360 us (8 chunks);
// 64 sequences of 2 chunks 343 -> 264 us (4); 256 sequences of 32 rows
// 698 -> 518 us (H = 32, d = 128).
// The default, from the sizes alone (the lengths are device data): sequences
// of up to 8 chunks when they average at most one chunk, up to 6 when at
// most two, up to 8 again when at most four, none when longer.  Measured on
// Dirichlet length mixes of 32 to 192 sequences in 8192 rows at H = 32 and
// on equal lengths: each band's F is within a few percent of the best F for
// every mix tried, 2-25% faster than fusing nothing; 16 to 28 sequences (the
// packed chunk among them) run fastest with nothing fused.
int prefill_fuse_max(int T, int N, int H, bool bf16, int fuse_chunks) {
    (void)H;
    if (!bf16 || fuse_chunks < 0) return -1;
    if (fuse_chunks > 0) return fuse_chunks;
    if ((long long)T <= (long long)kChunk * N) return 8;
    if ((long long)T <= 2LL * kChunk * N) return 6;
    if ((long long)T <= 4LL * kChunk * N) return 8;
    return -1;
}

size_t prefill_workspace_bytes(int T, int N, int H, int dk, int dv, bool bf16, int window_chunks) {
    return prefill_plan(T, N, H, dk, dv, bf16, window_chunks).bytes;
}

size_t conv_workspace_bytes(int T, int H, int dk, int dv, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return 256 + 2 * up((size_t)T * H * dk * es) + up((size_t)T * H * dv * es);
}

#define KDA_INST(E, DK, DV) \
    template hipError_t launch_prefill<E, DK, DV>(const PrefillArgs &, hipStream_t);
KDA_INST(bf16, 64, 64)
KDA_INST(bf16, 64, 128)
KDA_INST(bf16, 128, 64)
KDA_INST(bf16, 128, 128)
KDA_INST(float, 64, 64)
KDA_INST(float, 64, 128)
KDA_INST(float, 128, 64)
KDA_INST(float, 128, 128)
#undef KDA_INST

// ---------------------------------------------------------------------------
// Phase clocks (instrumented builds)
// ---------------------------------------------------------------------------

hipError_t phase_clocks_copy(int kernel, unsigned long long *host, size_t count, bool clear) {
#ifdef KDA_PHASE_CLOCKS
    constexpr size_t per = (size_t)kClockWaves * kClockItems * kClockMarks;
    if (kernel < 0 || kernel >= kClockKernels) return hipErrorInvalidValue;
    const size_t off = (size_t)kernel * per * sizeof(unsigned long long);
    if (host && count) {
        const hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_clock),
                                                 (count < per ? count : per) * sizeof(unsigned long long), off,
                                                 hipMemcpyDeviceToHost);
        if (e != hipSuccess) return e;
    }
    if (clear) {
        static const unsigned long long zeros[per] = {};
        return hipMemcpyToSymbol(HIP_SYMBOL(g_phase_clock), zeros, sizeof(zeros), off, hipMemcpyHostToDevice);
    }
    return hipSuccess;
#else
    (void)kernel; (void)host; (void)count; (void)clear;
    return hipErrorNotSupported;
#endif
}

}  // namespace kda
