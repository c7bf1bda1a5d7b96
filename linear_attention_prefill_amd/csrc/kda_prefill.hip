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
// kda_intra_kernel: one workgroup (4 waves) per (chunk, head), fully
// parallel, two workgroups per CU for bf16.  kda_scan_kernel: one workgroup
// of 4 waves per (sequence, head, 16-column slice of d_v); the d_v columns of
// S evolve independently, so slices need no exchange.  Wave w owns chunk rows
// 16w..16w+15 and a quarter of the key channels, swaps the rounded copies of
// its S and U tiles with the other waves through LDS, and keeps the operands
// of the next two chunks in flight in registers.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// Intra-chunk kernel
// ---------------------------------------------------------------------------

// Decay span (log2 units) of a 16-row block above which its diagonal block is
// computed exactly instead of with split factors.
constexpr float kDiagSpanLimit = 64.f;

template <typename E, int DK, int DV> struct IntraLds {
    static constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
    static constexpr int KPP = DK + PAD;             // pitch of k P, q P (E)
    static constexpr int KQP = DK + 4;               // pitch of k Qf (fp32)
    static constexpr int VP = DV + PAD;              // pitch of V (E)
    static constexpr int AP = 68;                    // pitch of A_kk / Tm (fp32)
    static constexpr int AQP = sizeof(E) == 2 ? 72 : 68;   // pitch of A_qk (E)
    static constexpr int max_(int a, int b) { return a > b ? a : b; }
    // byte sizes of the three regions and their later tenants
    static constexpr int R1 = max_(kChunk * KPP * (int)sizeof(E), kChunk * AQP * (int)sizeof(E));
    static constexpr int R2 = max_(kChunk * KPP * (int)sizeof(E), kChunk * AP * 4);
    static constexpr int R3 = max_(kChunk * KQP * 4, kChunk * VP * (int)sizeof(E));
};

// Raw inputs of one chunk held by one thread (prefetched for the next chunk).
template <typename E> struct Raw4;
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <> struct Raw4<float> { typedef f32x4 type; };
template <typename E> __device__ __forceinline__ f32x4 to_f32(const bf16x4 &x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <typename E> __device__ __forceinline__ f32x4 to_f32(const f32x4 &x) { return x; }

// A chunk of one head: item = cid * H + h; valid when item >= 0.
struct ChunkRef {
    int item, cid, h, row0, C;
};

// First chunk at or after `item` in steps of `stride` that belongs to a
// sequence (ids between sequences' chunk ranges are skipped).
__device__ __forceinline__ ChunkRef find_chunk(int item, int stride, int n_items,
                                               const int32_t *cu, int T, int N, int H) {
    for (; item < n_items; item += stride) {
        const int cid = item / H;
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (clamp_row(cu[mid], T) / kChunk + mid <= cid) lo = mid; else hi = mid - 1;
        }
        const SeqSpan sp = seq_span(cu, lo, T);
        const int jc = cid - sp.first_chunk;
        if (jc >= 0 && jc * kChunk < sp.len)
            return ChunkRef{item, cid, item - cid * H, sp.start + jc * kChunk, min(kChunk, sp.len - jc * kChunk)};
    }
    return ChunkRef{-1, 0, 0, 0, 0};
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256, 1) void kda_intra_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int H,
    E *__restrict__ ws, float *__restrict__ ws_dec) {
    static_assert(DK == 64 || DK == 128, "d_k");
    static_assert(DV == 64 || DV == 128, "d_v");
    using LD = IntraLds<E, DK, DV>;
    using L = WsLayout<E, DK, DV>;
    using R4 = typename Raw4<E>::type;
    constexpr int NTH = 256;
    constexpr int KPP = LD::KPP, KQP = LD::KQP, VP = LD::VP, AP = LD::AP, AQP = LD::AQP;
    constexpr int KS = DK / kSlab;                     // d_k slabs
    constexpr int KT = DK / kSub;                      // d_k tiles
    constexpr int VT = DV / kSub;                      // d_v tiles
    constexpr int C4 = DK / 4;                         // 4-channel columns
    constexpr int RG = NTH / C4;                       // row groups (prefix sum)
    constexpr int RPG = kChunk / RG;                   // rows per group
    constexpr int BPG = kSub / RPG;                    // groups per 16-row block
    constexpr int EPU = 16 / sizeof(E);
    constexpr int VPT = kChunk * DV / EPU / NTH;

    __shared__ __align__(16) char sR1[LD::R1];         // k P;  later A_qk
    __shared__ __align__(16) char sR2[LD::R2];         // q P (and prefix totals); later A_kk -> Tm
    __shared__ __align__(16) char sR3[LD::R3];         // k Qf (fp32); later V
    __shared__ __align__(16) float sF[10 * DK];        // F_IJ, J <= I, index I(I+1)/2 + J
    __shared__ __align__(16) float sBs[4 * DK];        // e^{Gam_16I}
    __shared__ __align__(16) float sCe[4 * DK];        // e^{Gam_C - Gam_16I+15}
    __shared__ float sBeta[kChunk];
    __shared__ int sExact[4];
    E *const sKP = reinterpret_cast<E *>(sR1);
    E *const sQP = reinterpret_cast<E *>(sR2);
    float *const sKQ = reinterpret_cast<float *>(sR3);
    float *const sTot = reinterpret_cast<float *>(sR2);   // [RG][DK] totals, then [4][DK] firsts
    E *const sAqk = reinterpret_cast<E *>(sR1);
    float *const sA = reinterpret_cast<float *>(sR2);
    E *const sV = reinterpret_cast<E *>(sR3);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // thread (c4, rg): channels 4 c4 .. 4 c4 + 3 of rows RPG rg .. RPG rg + RPG - 1
    const int c4 = tid % C4, rg = tid / C4, ch0 = 4 * c4;
    const int n_items = (T / kChunk + N) * H;
    const int stride = gridDim.x;

    // registers holding the next chunk's raw inputs
    R4 kr[RPG], qr[RPG];
    f32x4 gr[RPG];
    uint4 xv[VPT];
    float bt = 0.f;
    auto load_kqg = [&](const ChunkRef &ck) {
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int row = rg * RPG + r;
            kr[r] = qr[r] = R4{};
            gr[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ck.item >= 0 && row < ck.C) {
                const size_t off = ((size_t)(ck.row0 + row) * H + ck.h) * DK + ch0;
                kr[r] = *reinterpret_cast<const R4 *>(k + off);
                qr[r] = *reinterpret_cast<const R4 *>(q + off);
                gr[r] = *reinterpret_cast<const f32x4 *>(g + off);
            }
        }
        bt = (ck.item >= 0 && tid < ck.C) ? beta[(size_t)(ck.row0 + tid) * H + ck.h] : 0.f;
    };
    auto load_v = [&](const ChunkRef &ck) {
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int u = tid + p * NTH;
            const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
            xv[p] = uint4{0, 0, 0, 0};
            if (ck.item >= 0 && r < ck.C)
                xv[p] = *reinterpret_cast<const uint4 *>(v + ((size_t)(ck.row0 + r) * H + ck.h) * DV + c);
        }
    };

    ChunkRef cur = find_chunk(blockIdx.x, stride, n_items, cu, T, N, H);
    load_kqg(cur);
    load_v(cur);
    while (cur.item >= 0) {
        const int C = cur.C;
        const size_t rec = (size_t)cur.item;           // = cid * H + h
        E *const Rw = ws + rec * L::kRecElems;
        E *const Rq = Rw + L::kWElems;
        E *const Rk = Rq + L::kQElems;
        E *const Ra = Rk + L::kKElems;
        E *const Ru = Ra + L::kAElems;
        const ChunkRef nxt = find_chunk(cur.item + stride, stride, n_items, cu, T, N, H);

        // ---- prefix sums of g (log2 units): group totals and block-first values ----
        f32x4 gl[RPG];
#pragma unroll
        for (int r = 0; r < RPG; ++r) gl[r] = gr[r] * kLog2e;
#pragma unroll
        for (int r = 1; r < RPG; ++r) gl[r] += gl[r - 1];
        *reinterpret_cast<f32x4 *>(sTot + rg * DK + ch0) = gl[RPG - 1];
        if (rg % BPG == 0) *reinterpret_cast<f32x4 *>(sTot + RG * DK + (rg / BPG) * DK + ch0) = gl[0];
        if (tid < kChunk) sBeta[tid] = bt;
        if (tid < 4) sExact[tid] = 0;
        __syncthreads();

        // ---- per-row factors (registers), per-block factors (threads c < DK) ----
        const int blk = rg / BPG;
        f32x4 pre = {0.f, 0.f, 0.f, 0.f}, btot = pre, before = pre;
        for (int p = 0; p < blk * BPG; ++p) before += *reinterpret_cast<const f32x4 *>(sTot + p * DK + ch0);
#pragma unroll
        for (int p = 0; p < BPG; ++p) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(sTot + (blk * BPG + p) * DK + ch0);
            btot += t;
            if (p < rg % BPG) pre += t;
        }
        const f32x4 gs = *reinterpret_cast<const f32x4 *>(sTot + RG * DK + blk * DK + ch0);
        f32x4 ebs;                                     // e^{Gam} at the block's first row
#pragma unroll
        for (int x = 0; x < 4; ++x) ebs[x] = fast_exp2(before[x] + gs[x]);
        // k P and k Qf go to LDS at once (their regions hold nothing live);
        // Q e^Gam goes straight to the workspace in the scan's fragment order;
        // q P waits for the barrier, since its region holds the prefix totals.
        R4 qpk[RPG];
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            const int row = rg * RPG + r;
            const f32x4 bp = pre + gl[r];              // block-local inclusive prefix
            const f32x4 kf = to_f32<E>(kr[r]), qf = to_f32<E>(qr[r]);
            f32x4 kp, qp, kq, qh;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float P = fast_exp2(bp[x] - gs[x]);
                const float Qf = fast_exp2(btot[x] - bp[x]);
                kp[x] = kf[x] * P;
                qp[x] = qf[x] * P;
                kq[x] = kf[x] * Qf;
                qh[x] = qp[x] * ebs[x];
            }
            store4<E>(sKP + row * KPP + ch0, kp);
            *reinterpret_cast<f32x4 *>(sKQ + row * KQP + ch0) = kq;
            // fragment (m, s) = (row / 16, ch0 / 32); lane (row % 16) + 16 g with
            // g = (ch0 % 16) / 4; half (ch0 % 32) / 16 selects elements 4..7
            const int m = row >> 4, s = ch0 >> 5;
            const int fl = (row & 15) + 16 * ((ch0 & 15) >> 2);
            store4<E>(Rq + (m * KS + s) * 512 + fl * 8 + 4 * ((ch0 & 31) >> 4), qh);
            store4<E>(reinterpret_cast<E *>(&qpk[r]), qp);
        }
        float fF[10], fBs[4], fCe[4], fdec = 0.f;
        bool exact[4] = {false, false, false, false};
        if (tid < DK) {
            const int c = tid;
            float Gs[4], Ge[4], run = 0.f;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                float bt2 = 0.f;
#pragma unroll
                for (int p = 0; p < BPG; ++p) bt2 += sTot[(I * BPG + p) * DK + c];
                Gs[I] = run + sTot[RG * DK + I * DK + c];
                Ge[I] = run + bt2;
                run = Ge[I];
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int J = 0; J <= I; ++J) fF[I * (I + 1) / 2 + J] = fast_exp2(Gs[I] - Ge[J]);
                fBs[I] = fast_exp2(Gs[I]);
                fCe[I] = fast_exp2(Ge[3] - Ge[I]);
                exact[I] = (Gs[I] - Ge[I]) > kDiagSpanLimit;
            }
            fdec = fast_exp2(Ge[3]);
        }
        __syncthreads();   // prefix totals are no longer read; their region takes q P

#pragma unroll
        for (int r = 0; r < RPG; ++r)
            *reinterpret_cast<R4 *>(sQP + (rg * RPG + r) * KPP + ch0) = qpk[r];
        if (tid < DK) {
#pragma unroll
            for (int i = 0; i < 10; ++i) sF[i * DK + tid] = fF[i];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                sBs[I * DK + tid] = fBs[I];
                sCe[I * DK + tid] = fCe[I];
                if (exact[I]) sExact[I] = 1;
            }
            ws_dec[rec * DK + tid] = fdec;
        }
        // the raw k, q, g registers are free: fetch the next chunk's
        load_kqg(nxt);
        __syncthreads();

        // ---- K~^T fragments: (t, s) holds key channels 16t.. over chunk rows 32s.. ----
        for (int f = wave; f < KT * 2; f += 4) {
            const int t = f >> 1, s = f & 1;
            const int ch = t * kSub + li;
            Frag<E> fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = s * kSlab + kk_of(lg, e);
                fr.set(e, sKQ[row * KQP + ch] * sCe[(row >> 4) * DK + ch]);
            }
            store_frag<E>(Rk + (t * 2 + s) * 512, lane, fr);
        }
        // ---- X = diag(beta) K e^Gam for w, kept in registers (wave w: d_k slab w) ----
        Frag<E> xf[2][2];
        if (wave < KS) {
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) {
                const int ch = (2 * wave + nn) * kSub + li;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = s * kSlab + kk_of(lg, e);
                        xf[nn][s].set(e, sBeta[row] * (float)sKP[row * KPP + ch] * sBs[(row >> 4) * DK + ch]);
                    }
                }
            }
        }

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
        // Exact diagonal block (decay span beyond the split-factor range): lane
        // (row li, channel quarter lg) sums one exp per (column, channel) over
        // its quarter, reading the chunk from global memory, then the quarters
        // are reduced.
        auto diag_exact = [&](int I, f32x4 &accK, f32x4 &accQ) {
            constexpr int CQ = DK / 4;
            float aK[kSub], aQ[kSub];
#pragma unroll
            for (int jj = 0; jj < kSub; ++jj) { aK[jj] = 0.f; aQ[jj] = 0.f; }
            const int ri = I * kSub + li;
            for (int c = lg * CQ; c < (lg + 1) * CQ; ++c) {
                float gcum[kSub], kc[kSub];
                float run = 0.f;
#pragma unroll
                for (int jj = 0; jj < kSub; ++jj) {
                    const int row = I * kSub + jj;
                    float gg = 0.f, kk = 0.f;
                    if (row < C) {
                        const size_t off = ((size_t)(cur.row0 + row) * H + cur.h) * DK + c;
                        gg = g[off];
                        kk = (float)k[off];
                    }
                    run += gg * kLog2e;
                    gcum[jj] = run;
                    kc[jj] = kk;
                }
                float gi = 0.f, ki = 0.f, qi = 0.f;
#pragma unroll
                for (int jj = 0; jj < kSub; ++jj) {
                    if (jj == li) { gi = gcum[jj]; ki = kc[jj]; }
                }
                if (ri < C) qi = (float)q[((size_t)(cur.row0 + ri) * H + cur.h) * DK + c];
#pragma unroll
                for (int jj = 0; jj < kSub; ++jj) {
                    const float e = jj <= li ? fast_exp2(gi - gcum[jj]) : 0.f;
                    const float t = kc[jj] * e;
                    aK[jj] = fmaf(ki, t, aK[jj]);
                    aQ[jj] = fmaf(qi, t, aQ[jj]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < kSub; ++jj) {
                aK[jj] += __shfl_xor(aK[jj], 16);
                aK[jj] += __shfl_xor(aK[jj], 32);
                aQ[jj] += __shfl_xor(aQ[jj], 16);
                aQ[jj] += __shfl_xor(aQ[jj], 32);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int jj = 0; jj < kSub; ++jj) {
                    if (jj == 4 * lg + r) { sk = aK[jj]; sq = aQ[jj]; }
                }
                accK[r] = sk;
                accQ[r] = sq;
            }
        };
        // wave w: diagonal block w, and off-diagonal pairs w and w + 4 of
        // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        auto pair_i = [](int p) { return p == 0 ? 1 : (p < 3 ? 2 : 3); };
        auto pair_j = [](int p) { return p == 0 ? 0 : (p < 3 ? p - 1 : p - 3); };
        const int p0 = wave, p1 = wave + 4;
        f32x4 dK, dQ, oK[2], oQ[2];
        if (sExact[wave]) diag_exact(wave, dK, dQ);
        else ablock(wave, wave, dK, dQ);
        ablock(pair_i(p0), pair_j(p0), oK[0], oQ[0]);
        if (p1 < 6) ablock(pair_i(p1), pair_j(p1), oK[1], oQ[1]);
        __syncthreads();   // k P, q P, k Qf are no longer read

        // ---- A_kk (beta-scaled) -> sA, A_qk -> sAqk, V -> where k Qf was ----
        for (int idx = tid; idx < 6 * 256; idx += NTH) {     // blocks above the diagonal
            const int b = idx >> 8, e = idx & 255;
            const int I = b < 3 ? 0 : (b < 5 ? 1 : 2);
            const int J = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
            const int r = I * kSub + (e >> 4), c = J * kSub + (e & 15);
            sA[r * AP + c] = 0.f;
            sAqk[r * AQP + c] = (E)0.f;
        }
        {
            auto put = [&](int I, int J, const f32x4 &aK, const f32x4 &aQ, bool diag) {
                const int row = I * kSub + li;
                const float b = sBeta[row];
                f32x4 vk, vq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = 4 * lg + r;
                    vk[r] = (!diag || col < li) ? aK[r] * b : 0.f;
                    vq[r] = (!diag || col <= li) ? aQ[r] : 0.f;
                }
                *reinterpret_cast<f32x4 *>(sA + row * AP + J * kSub + 4 * lg) = vk;
                store4<E>(sAqk + row * AQP + J * kSub + 4 * lg, vq);
            };
            put(wave, wave, dK, dQ, true);
            put(pair_i(p0), pair_j(p0), oK[0], oQ[0], false);
            if (p1 < 6) put(pair_i(p1), pair_j(p1), oK[1], oQ[1], false);
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int u = tid + p * NTH;
            const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
            *reinterpret_cast<uint4 *>(sV + r * VP + c) = xv[p];
        }
        load_v(nxt);
        __syncthreads();

        // ---- A_qk fragments; diagonal 16x16 inverses of I + A_kk in place ----
        {
            const int m = wave;
            const int row = m * kSub + li;
            for (int s = 0; s <= (m >> 1); ++s) {
                const int c0 = s * kSlab + 4 * lg;
                store_frag<E>(Ra + tri_frag(m, s) * 512, lane,
                              frag_from_runs<E>(sAqk + row * AQP + c0, sAqk + row * AQP + c0 + 16));
            }
        }
        if (wave == 0) {
            // Tm_II by forward substitution, lane = (block, column); every read of
            // A_II precedes the writes, all within this wave.
            const int I = lane >> 4, jj = lane & 15;
            float t[kSub];
#pragma unroll
            for (int ii = 0; ii < kSub; ++ii) {
                float s = 0.f;
#pragma unroll
                for (int mm = 0; mm < ii; ++mm) s = fmaf(sA[(I * kSub + ii) * AP + I * kSub + mm], t[mm], s);
                t[ii] = ii < jj ? 0.f : (ii == jj ? 1.f : -s);
            }
#pragma unroll
            for (int ii = 0; ii < kSub; ++ii) sA[(I * kSub + ii) * AP + I * kSub + jj] = t[ii];
        }
        __syncthreads();

        // ---- off-diagonal blocks of Tm on fp32 matrix cores, in place ----
        // level 1 (waves 0, 1): Tm_10 = -Tm_11 (A_10 Tm_00), Tm_32 = -Tm_33 (A_32 Tm_22)
        if (wave < 2) {
            const int I = wave ? 3 : 1, J = I - 1;
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                P = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(I * kSub + li) * AP + J * kSub + lg + 4 * ks],
                                                         sA[(J * kSub + lg + 4 * ks) * AP + J * kSub + li], P, 0, 0, 0);
            // P in C layout is the B operand with contraction index 4g + r
            f32x4 Tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Tt = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(I * kSub + li) * AP + I * kSub + 4 * lg + r], P[r], Tt, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[(I * kSub + 4 * lg + r) * AP + J * kSub + li] = -Tt[r];
        }
        __syncthreads();
        // level 2 (wave = output tile (ti, tj)): Tm[32:64, 0:32] = -Tm_hi (A[32:64, 0:32] Tm_lo)
        {
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
            f32x4 Tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Tt = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        sA[(32 + ti * kSub + li) * AP + 32 + kt * kSub + 4 * lg + r], Qt[kt][r], Tt, 0, 0, 0);
            }
            __syncthreads();   // every wave has read A[32:64, 0:32]
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[(32 + ti * kSub + 4 * lg + r) * AP + tj * kSub + li] = -Tt[r];
        }
        __syncthreads();

        // ---- w and u on the matrix cores ----
        Frag<E> tf[6];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int s = 0; s <= (m >> 1); ++s) {
                const int row = m * kSub + li, c0 = s * kSlab + 4 * lg;
                tf[tri_frag(m, s)] = frag_from_tiles<E>(*reinterpret_cast<const f32x4 *>(sA + row * AP + c0),
                                                        *reinterpret_cast<const f32x4 *>(sA + row * AP + c0 + 16));
            }
        }
        if (wave < KS) {
            // w slab `wave` (key channels 32 wave ..), computed transposed as
            // X^T Tm^T: lane (i, g) receives w[16m + i][16n + 4g + r], the scan's
            // A-operand order.
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
                for (int s = 0; s <= (m >> 1); ++s) {
                    mma(acc0, xf[0][s], tf[tri_frag(m, s)]);
                    mma(acc1, xf[1][s], tf[tri_frag(m, s)]);
                }
                store_frag<E>(Rw + (m * KS + wave) * 512, lane, frag_from_tiles<E>(acc0, acc1));
            }
        }
        for (int jt = wave; jt < VT; jt += 4) {
            // u tile (value columns 16 jt ..): Tm diag(beta) V, lane (i, g) holds
            // u[16m + 4g + r][16 jt + i].
            const int ch = jt * kSub + li;
            Frag<E> vf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = s * kSlab + kk_of(lg, e);
                    vf[s].set(e, sBeta[row] * (float)sV[row * VP + ch]);
                }
            }
            E *dst = Ru + jt * (64 * 16) + lane * 16;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= (m >> 1); ++s) mma(acc, tf[tri_frag(m, s)], vf[s]);
                store4<E>(dst + 4 * m, acc);
            }
        }
        __syncthreads();   // LDS is rewritten by the next chunk
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// State scan
// ---------------------------------------------------------------------------

// Operands of one chunk for one wave (row tile m = wave, TPW key tiles).
template <typename E, int DK> struct ScanStage {
    static constexpr int KS = DK / kSlab;
    static constexpr int TPW = DK / 64;
    Frag<E> wf[KS], qf[KS], af[2], kf[TPW][2];
    typename Raw4<E>::type u;                  // raw: converted where it is used
    f32x4 d[TPW];
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_scan_kernel(
    const E *__restrict__ ws, const float *__restrict__ ws_dec,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots,
    const float *state_in, float *state_out, E *__restrict__ o,
    int T, int N, int H, int num_slots, float scale) {
    constexpr int VT = DV / kSub, KS = DK / kSlab;
    constexpr int TPW = DK / 64;                       // key tiles per wave
    using L = WsLayout<E, DK, DV>;
    using Stage = ScanStage<E, DK>;
    // rounded copies of the state slabs and of U, [slab][lane][8]
    __shared__ __align__(16) E sSb[KS * 64 * 8];
    __shared__ __align__(16) E sUb[2 * 64 * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // Work order.  Sequences are taken longest first (for up to 64 sequences;
    // every wave ranks them the same way), then head by head; (sequence,
    // head) pairs are dealt round robin to the 8 XCDs (workgroups go to XCD
    // b % 8), so each XCD gets an equal share of every sequence, while the
    // d_v slices of one pair stay on one XCD and share its L2.
    const int B = gridDim.x, b = blockIdx.x;
    const int NP = N * H;
    int q, jt;
    if (NP % 8 == 0) {
        const int k = b >> 3;
        jt = k % VT;
        q = (k / VT) * 8 + (b & 7);
    } else {
        jt = b % VT;
        q = b / VT;
    }
    if (q >= NP || b >= B) return;
    const int h = q % H;
    int n = q / H;                                      // rank of the sequence
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
    const int slot = slots ? slots[n] : n;
    if (slots && (slot < 0 || slot >= num_slots)) return;   // padded sequence
    const SeqSpan sp = seq_span(cu, n, T);
    const int j0 = jt * kSub;

    // my key tiles t = wave * TPW + i, C layout: lane holds S[16t + 4g + r][j0 + i]
    f32x4 S[TPW];
    if (state_in) {
        const float *src = state_in + (((size_t)slot * H + h) * DV + j0 + li) * DK;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
            S[i] = *reinterpret_cast<const f32x4 *>(src + (wave * TPW + i) * kSub + 4 * lg);
    } else {
#pragma unroll
        for (int i = 0; i < TPW; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Settle the state load here: otherwise the wait inserted for it at the
    // top of the chunk loop would also drain every prefetched chunk.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = S[i][r];
            asm volatile("" : "+v"(x));
            S[i][r] = x;
        }
    }

    // Record of chunk cc, by part; each part of a stage is refilled with the
    // chunk three ahead as soon as its last use in the current step has been
    // issued, so loads trickle out between the matrix-core products instead
    // of queueing behind them in one burst.
    auto rec_of = [&](int cc) { return (size_t)(sp.first_chunk + cc) * H + h; };
    auto load_w = [&](Stage &X, int cc) {
        const E *Rw = ws + rec_of(cc) * L::kRecElems;
#pragma unroll
        for (int s = 0; s < KS; ++s) X.wf[s] = load_frag<E>(Rw + (wave * KS + s) * 512, lane);
        const E *Ru = Rw + L::kWElems + L::kQElems + L::kKElems + L::kAElems;
        X.u = *reinterpret_cast<const typename Raw4<E>::type *>(Ru + jt * (64 * 16) + lane * 16 + 4 * wave);
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
        X.af[1] = load_frag<E>(Ra + tri_frag(wave, 1) * 512, lane);   // unused by waves 0, 1
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave * TPW + i;
            X.kf[i][0] = load_frag<E>(Rk + (t * 2) * 512, lane);
            X.kf[i][1] = load_frag<E>(Rk + (t * 2 + 1) * 512, lane);
            X.d[i] = *reinterpret_cast<const f32x4 *>(ws_dec + rec * DK + t * kSub + 4 * lg);
        }
    };
    auto load_stage = [&](Stage &X, int cc) {
        load_w(X, cc);
        load_k(X, cc);
        load_q(X, cc);
    };

    const int nch = (sp.len + kChunk - 1) / kChunk;
    // Refills are unconditional (clamped to the last chunk) inside the main
    // loop: a conditional load would leave a stage register holding either
    // the old or the new value, and the copy that merges them waits for
    // every load in flight.
    auto step = [&](Stage &X, int cc, bool refill) {
        const int nx = cc + 3 < nch ? cc + 3 : nch - 1;
        // publish my state tiles (rounded to E) and read every slab
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave * TPW + i;
            store4<E>(sSb + ((t >> 1) * 64 + lane) * 8 + (t & 1) * 4, S[i]);
        }
        __syncthreads();
        Frag<E> Sb[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) Sb[s] = load_frag<E>(sSb + s * 512, lane);
        // my tile of U = u - w S (two independent accumulation chains)
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            mma(a0, X.wf[s], Sb[s]);
            mma(a1, X.wf[s + 1], Sb[s + 1]);
        }
        const f32x4 un = to_f32<E>(X.u) - (a0 + a1);
        if (refill) load_w(X, nx);
        store4<E>(sUb + ((wave >> 1) * 64 + lane) * 8 + (wave & 1) * 4, un);
        // Q~ S part of the output does not need U: issue it before the barrier
        f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            mma(o0, Sb[s], X.qf[s]);
            mma(o1, Sb[s + 1], X.qf[s + 1]);
        }
        if (refill) load_q(X, nx);
#pragma unroll
        for (int i = 0; i < TPW; ++i) S[i] *= X.d[i];
        __syncthreads();
        Frag<E> ub[2];
        ub[0] = load_frag<E>(sUb, lane);
        ub[1] = load_frag<E>(sUb + 512, lane);
        // my tile of O = Q~ S + A_qk U, transposed: lane holds row 16 wave + i,
        // columns j0 + 4g + r
        mma(o0, ub[0], X.af[0]);
        if (wave >= 2) mma(o1, ub[1], X.af[1]);
        // my key tiles of S = diag(e^{Gam_C}) S + K~^T U
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            mma(S[i], X.kf[i][0], ub[0]);
            mma(S[i], X.kf[i][1], ub[1]);
        }
        if (refill) load_k(X, nx);
        const int row = wave * kSub + li;
        if (row < sp.len - cc * kChunk)
            store4<E>(o + ((size_t)(sp.start + cc * kChunk + row) * H + h) * DV + j0 + 4 * lg,
                      (o0 + o1) * scale);
    };

    if (nch > 0) {
        Stage A, Bs, Cs;
        load_stage(A, 0);
        load_stage(Bs, nch > 1 ? 1 : 0);
        load_stage(Cs, nch > 2 ? 2 : nch - 1);
        int cc = 0;
        for (; cc + 2 < nch; cc += 3) {
            step(A, cc, true);
            step(Bs, cc + 1, true);
            step(Cs, cc + 2, true);
        }
        if (cc < nch) step(A, cc, false);
        if (cc + 1 < nch) step(Bs, cc + 1, false);
    }

    if (state_out) {
        float *dst = state_out + (((size_t)slot * H + h) * DV + j0 + li) * DK;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
            *reinterpret_cast<f32x4 *>(dst + (wave * TPW + i) * kSub + 4 * lg) = S[i];
    }
}

template <typename E, int DK, int DV>
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    using L = WsLayout<E, DK, DV>;
    const int max_chunks = a.T / kChunk + a.N;
    E *ws = reinterpret_cast<E *>(a.workspace);
    float *ws_dec = reinterpret_cast<float *>(reinterpret_cast<char *>(a.workspace) +
                                              (size_t)max_chunks * a.H * L::kRecElems * sizeof(E));
    if (a.events[0]) (void)hipEventRecord(a.events[0], stream);
    if (max_chunks > 0) {
        const long long items = (long long)max_chunks * a.H;
        const int per_cu = 1;
        const int grid = (int)(items < (long long)a.num_cus * per_cu ? items : (long long)a.num_cus * per_cu);
        kda_intra_kernel<E, DK, DV><<<dim3(grid), dim3(256), 0, stream>>>(
            static_cast<const E *>(a.q), static_cast<const E *>(a.k), static_cast<const E *>(a.v),
            a.g, a.beta, a.cu_seqlens, a.T, a.N, a.H, ws, ws_dec);
    }
    if (a.events[1]) (void)hipEventRecord(a.events[1], stream);
    const int nblocks = a.N * a.H * (DV / kSub);
    kda_scan_kernel<E, DK, DV><<<dim3(nblocks), dim3(256), 0, stream>>>(
        ws, ws_dec, a.cu_seqlens, a.slots, a.state_in, a.state_out, static_cast<E *>(a.o),
        a.T, a.N, a.H, a.num_slots, a.scale);
    const hipError_t e = hipGetLastError();
    if (a.events[2]) (void)hipEventRecord(a.events[2], stream);
    return e;
}

size_t prefill_workspace_bytes(int T, int N, int H, int dk, int dv, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const size_t rec = (size_t)kChunk * (3 * dk + dv) + 6 * 512;
    const size_t max_chunks = (size_t)(T / kChunk) + (size_t)N;
    return max_chunks * (size_t)H * (rec * es + (size_t)dk * 4);
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

}  // namespace kda
