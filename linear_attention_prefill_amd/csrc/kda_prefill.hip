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
// kda_intra_kernel: one workgroup (4 waves) per (chunk, head), fully
// parallel, two workgroups per CU.  All global loads are issued at once; Gam
// is a blocked prefix sum; every 16x16 block of A_kk and A_qk runs on the
// matrix cores with the decay split at a reference row so that no factor
// overflows (off-diagonal blocks: the row before the block, both factors
// <= 1; diagonal blocks: the block's middle row, with an exact one-exp-per-
// term fallback when a channel decays by more than 2^64 inside the block).
// I + A_kk is inverted in place by blocked forward substitution in LDS; w
// and u run on the matrix cores.  Outputs go to the workspace in the scan's
// register order.
//
// kda_scan_kernel: one workgroup of 4 waves per (sequence, head, 16-column
// slice of d_v).  The d_v columns of S evolve independently, so slices need no
// exchange.  Wave w owns chunk rows 16w..16w+15 and key channels
// (d_k/4) w ..; per chunk it computes its tile of U = u - w S, of
// O = Q~ S + A_qk U and of S = diag(e^{Gam_C}) S + K~^T U, swapping the bf16
// copies of its S and U tiles with the other waves through LDS.  The next
// chunk's operands are loaded into registers while the current one is
// computed.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// Intra-chunk kernel
// ---------------------------------------------------------------------------

// Span (log2 units) of the decay inside a 16-row block above which the
// diagonal block is computed exactly instead of with split factors.
constexpr float kDiagSpanLimit = 64.f;

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256, sizeof(E) == 2 ? 2 : 1) void kda_intra_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int H,
    E *__restrict__ ws, float *__restrict__ ws_dec) {
    static_assert(DK == 64 || DK == 128, "d_k");
    static_assert(DV == 64 || DV == 128, "d_v");
    constexpr int NTH = 256;
    constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
    constexpr int KP = DK + PAD;                       // row pitch of sK (elements)
    constexpr int DQV = DK > DV ? DK : DV;
    constexpr int QP = DQV + PAD;                      // row pitch of sQV
    constexpr int GP = DK + 4;                         // row pitch of Gam (floats)
    constexpr int AP = 65;                             // row pitch of the 64x64 matrices
    constexpr int KS = DK / kSlab;                     // d_k slabs
    constexpr int KT = DK / kSub;                      // d_k tiles
    constexpr int VT = DV / kSub;                      // d_v tiles
    constexpr int G_FL = kChunk * GP;
    constexpr int A_FL = kChunk * AP;
    constexpr int REGION = G_FL > 2 * A_FL ? G_FL : 2 * A_FL;
    constexpr int C4 = DK / 4;                         // float4 columns of g
    constexpr int RG = NTH / C4;                       // row groups of the prefix sum
    constexpr int RPG = kChunk / RG;                   // rows per group
    using L = WsLayout<E, DK, DV>;

    __shared__ __align__(16) E sK[kChunk * KP];
    __shared__ __align__(16) E sQV[kChunk * QP];       // Q, later V
    __shared__ __align__(16) float sR[REGION];         // Gam*log2(e); later A_kk->Tm, A_qk
    __shared__ __align__(16) float sTot[RG * DK];      // prefix-sum group totals
    __shared__ float sBeta[kChunk];
    float *const sG = sR;
    float *const sA = sR;                              // A_kk (beta-scaled), then Tm in place
    float *const sQA = sR + A_FL;                      // A_qk, then inverse scratch

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int cid = blockIdx.x, h = blockIdx.y;

    // ---- locate the chunk: largest n with floor(start_n/64) + n <= cid ----
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (clamp_row(cu[mid], T) / kChunk + mid <= cid) lo = mid; else hi = mid - 1;
    }
    const SeqSpan sp = seq_span(cu, lo, T);
    const int jc = cid - sp.first_chunk;
    if (jc < 0 || jc * kChunk >= sp.len) return;       // id not used by any sequence
    const int row0 = sp.start + jc * kChunk;
    const int C = min(kChunk, sp.len - jc * kChunk);
    const size_t rec = (size_t)cid * H + h;
    E *const Rw = ws + rec * L::kRecElems;
    E *const Rq = Rw + L::kWElems;
    E *const Rk = Rq + L::kQElems;
    E *const Ra = Rk + L::kKElems;
    E *const Ru = Ra + L::kAElems;

    // ---- issue every global load of the chunk at once ----
    constexpr int EPU = 16 / sizeof(E);
    constexpr int KPT = kChunk * DK / EPU / NTH;
    constexpr int VPT = kChunk * DV / EPU / NTH;
    uint4 xk[KPT], xq[KPT], xv[VPT];
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DK / EPU), c = (u % (DK / EPU)) * EPU;
        xk[p] = uint4{0, 0, 0, 0};
        xq[p] = uint4{0, 0, 0, 0};
        if (r < C) {
            const size_t off = ((size_t)(row0 + r) * H + h) * DK + c;
            xk[p] = *reinterpret_cast<const uint4 *>(k + off);
            xq[p] = *reinterpret_cast<const uint4 *>(q + off);
        }
    }
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
        xv[p] = uint4{0, 0, 0, 0};
        if (r < C) xv[p] = *reinterpret_cast<const uint4 *>(v + ((size_t)(row0 + r) * H + h) * DV + c);
    }
    const int c4 = tid % C4, rg = tid / C4;
    f32x4 gv[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int row = rg * RPG + r;
        gv[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < C) gv[r] = *reinterpret_cast<const f32x4 *>(g + ((size_t)(row0 + row) * H + h) * DK + 4 * c4);
    }
    const float bt = (tid < C) ? beta[(size_t)(row0 + tid) * H + h] : 0.f;

    // ---- K, Q to LDS; Gam = inclusive prefix sum of g over rows ----
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DK / EPU), c = (u % (DK / EPU)) * EPU;
        *reinterpret_cast<uint4 *>(sK + r * KP + c) = xk[p];
        *reinterpret_cast<uint4 *>(sQV + r * QP + c) = xq[p];
    }
    if (tid < kChunk) sBeta[tid] = bt;
#pragma unroll
    for (int r = 1; r < RPG; ++r) gv[r] += gv[r - 1];
    *reinterpret_cast<f32x4 *>(sTot + rg * DK + 4 * c4) = gv[RPG - 1];
    __syncthreads();
    {
        f32x4 off = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < rg; ++p) off += *reinterpret_cast<const f32x4 *>(sTot + p * DK + 4 * c4);
#pragma unroll
        for (int r = 0; r < RPG; ++r)
            *reinterpret_cast<f32x4 *>(sG + (rg * RPG + r) * GP + 4 * c4) = (gv[r] + off) * kLog2e;
    }
    __syncthreads();

    // ---- Q * e^Gam fragments (A operand of the scan's output product) ----
    {
        const int row = wave * kSub + li;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            Frag<E> f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = s * kSlab + 16 * hf + 4 * lg;
                const f32x4 q4 = load4<E>(sQV + row * QP + ch);
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sG + row * GP + ch);
#pragma unroll
                for (int r = 0; r < 4; ++r) f.set(4 * hf + r, q4[r] * fast_exp2(g4[r]));
            }
            store_frag<E>(Rq + (wave * KS + s) * 512, lane, f);
        }
    }
    // ---- K~ = K * e^{Gam_C - Gam}, transposed: fragment (t, s) holds key
    // channels 16t..16t+15 over chunk rows 32s..32s+31.  Rows past C are zero
    // in K and Gam is flat there, so row 63 holds Gam_C. ----
    for (int f = wave; f < KT * 2; f += 4) {
        const int t = f >> 1, s = f & 1;
        const int ch = t * kSub + li;
        const float glast = sG[(kChunk - 1) * GP + ch];
        Frag<E> fr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int row = s * kSlab + kk_of(lg, e);
            fr.set(e, (float)sK[row * KP + ch] * fast_exp2(glast - sG[row * GP + ch]));
        }
        store_frag<E>(Rk + (t * 2 + s) * 512, lane, fr);
    }
    for (int c = tid; c < DK; c += NTH) ws_dec[rec * DK + c] = fast_exp2(sG[(kChunk - 1) * GP + c]);

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
                    xf[nn][s].set(e, sBeta[row] * (float)sK[row * KP + ch] * fast_exp2(sG[row * GP + ch]));
                }
            }
        }
    }

    // ---- A_kk and A_qk blocks on the matrix cores (C layout in registers) ----
    // A block (I, J) with reference row ref: rows a of block I scaled by
    // e^{Gam_a - Gam_ref} (q and k alike), rows b of block J by e^{Gam_ref - Gam_b}.
    auto ablock = [&](int I, int J, int ref, f32x4 &accK, f32x4 &accQ) {
        accK = f32x4{0.f, 0.f, 0.f, 0.f};
        accQ = accK;
        const int ra = I * kSub + li, rb = J * kSub + li;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            Frag<E> aK, aQ, bK;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ch = s * kSlab + 16 * hf + 4 * lg;
                const f32x4 ga = *reinterpret_cast<const f32x4 *>(sG + ra * GP + ch);
                const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + ref * GP + ch);
                const f32x4 gb = *reinterpret_cast<const f32x4 *>(sG + rb * GP + ch);
                const f32x4 ka = load4<E>(sK + ra * KP + ch);
                const f32x4 qa = load4<E>(sQV + ra * QP + ch);
                const f32x4 kb = load4<E>(sK + rb * KP + ch);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ea = fast_exp2(ga[r] - gr[r]);
                    const float eb = fast_exp2(gr[r] - gb[r]);
                    aK.set(4 * hf + r, ka[r] * ea);
                    aQ.set(4 * hf + r, qa[r] * ea);
                    bK.set(4 * hf + r, kb[r] * eb);
                }
            }
            mma(accK, aK, bK);
            mma(accQ, aQ, bK);
        }
    };
    // Exact diagonal block: one exp per (row, column, channel); lane
    // (column li, channel quarter lg), reduced over the quarters.
    auto diag_exact = [&](int I, f32x4 &accK, f32x4 &accQ) {
        constexpr int CQ = DK / 4;
        float aK[kSub], aQ[kSub];
#pragma unroll
        for (int ii = 0; ii < kSub; ++ii) { aK[ii] = 0.f; aQ[ii] = 0.f; }
        const int rj = I * kSub + li;
        for (int c = lg * CQ; c < (lg + 1) * CQ; c += 4) {
            const f32x4 kj = load4<E>(sK + rj * KP + c);
            const f32x4 gj = *reinterpret_cast<const f32x4 *>(sG + rj * GP + c);
#pragma unroll
            for (int ii = 0; ii < kSub; ++ii) {
                const int ri = I * kSub + ii;
                const f32x4 ki = load4<E>(sK + ri * KP + c);
                const f32x4 qi = load4<E>(sQV + ri * QP + c);
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(sG + ri * GP + c);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = ii >= li ? fast_exp2(gi[r] - gj[r]) : 0.f;
                    const float t = kj[r] * e;
                    aK[ii] = fmaf(ki[r], t, aK[ii]);
                    aQ[ii] = fmaf(qi[r], t, aQ[ii]);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < kSub; ++ii) {
            aK[ii] += __shfl_xor(aK[ii], 16);
            aK[ii] += __shfl_xor(aK[ii], 32);
            aQ[ii] += __shfl_xor(aQ[ii], 16);
            aQ[ii] += __shfl_xor(aQ[ii], 32);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int ii = 0; ii < kSub; ++ii) {
                if (ii == 4 * lg + r) { sk = aK[ii]; sq = aQ[ii]; }
            }
            accK[r] = sk;
            accQ[r] = sq;
        }
    };

    // wave w: diagonal block w, and off-diagonal pairs w and w + 4 of
    // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    f32x4 dK, dQ, oK[2], oQ[2];
    {
        const int I = wave;
        float span = 0.f;
        for (int c = lane; c < DK; c += 64)
            span = fmaxf(span, sG[(I * kSub) * GP + c] - sG[(I * kSub + kSub - 1) * GP + c]);
        if (__any(span > kDiagSpanLimit)) diag_exact(I, dK, dQ);
        else ablock(I, I, I * kSub + 7, dK, dQ);
    }
    const int p0 = wave, p1 = wave + 4;
    auto pair_i = [](int p) { return p == 0 ? 1 : (p < 3 ? 2 : 3); };
    auto pair_j = [](int p) { return p == 0 ? 0 : (p < 3 ? p - 1 : p - 3); };
    ablock(pair_i(p0), pair_j(p0), pair_i(p0) * kSub - 1, oK[0], oQ[0]);
    if (p1 < 6) ablock(pair_i(p1), pair_j(p1), pair_i(p1) * kSub - 1, oK[1], oQ[1]);
    __syncthreads();   // Gam and Q are no longer read

    // ---- A_kk (beta-scaled) and A_qk into the region; V over Q ----
    for (int idx = tid; idx < 6 * 256; idx += NTH) {     // blocks above the diagonal
        const int b = idx >> 8, e = idx & 255;
        const int I = b < 3 ? 0 : (b < 5 ? 1 : 2);
        const int J = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
        const int r = I * kSub + (e >> 4), c = J * kSub + (e & 15);
        sA[r * AP + c] = 0.f;
        sQA[r * AP + c] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int rr = 4 * lg + r;
        int row = wave * kSub + rr, col = wave * kSub + li;
        sA[row * AP + col] = rr > li ? dK[r] * sBeta[row] : 0.f;
        sQA[row * AP + col] = rr >= li ? dQ[r] : 0.f;
        row = pair_i(p0) * kSub + rr;
        col = pair_j(p0) * kSub + li;
        sA[row * AP + col] = oK[0][r] * sBeta[row];
        sQA[row * AP + col] = oQ[0][r];
        if (p1 < 6) {
            row = pair_i(p1) * kSub + rr;
            col = pair_j(p1) * kSub + li;
            sA[row * AP + col] = oK[1][r] * sBeta[row];
            sQA[row * AP + col] = oQ[1][r];
        }
    }
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
        *reinterpret_cast<uint4 *>(sQV + r * QP + c) = xv[p];
    }
    __syncthreads();

    // ---- A_qk fragments; diagonal 16x16 inverses in place ----
    {
        const int m = wave;
        const int row = m * kSub + li;
        for (int s = 0; s <= (m >> 1); ++s) {
            Frag<E> f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int col = s * kSlab + 16 * hf + 4 * lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) f.set(4 * hf + r, sQA[row * AP + col + r]);
            }
            store_frag<E>(Ra + tri_frag(m, s) * 512, lane, f);
        }
    }
    if (wave == 0) {
        // Tm_II = (I + A_II)^-1 by forward substitution, lane = (block, column);
        // every read of A_II precedes the writes, all within this wave.
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

    // ---- off-diagonal blocks of Tm, in place; scratch in the A_qk area ----
    float *const sS = sQA;
    // level 1: Tm_10 = -Tm_11 A_10 Tm_00, Tm_32 = -Tm_33 A_32 Tm_22
    for (int idx = tid; idx < 512; idx += NTH) {
        const int which = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int I = which ? 3 : 1, J = I - 1;
        float s = 0.f;
#pragma unroll
        for (int m2 = 0; m2 < kSub; ++m2)
            s = fmaf(sA[(I * kSub + r) * AP + J * kSub + m2], sA[(J * kSub + m2) * AP + J * kSub + c], s);
        sS[idx] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < 512; idx += NTH) {
        const int which = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int I = which ? 3 : 1, J = I - 1;
        float s = 0.f;
#pragma unroll
        for (int m2 = 0; m2 < kSub; ++m2)
            s = fmaf(sA[(I * kSub + r) * AP + I * kSub + m2], sS[(which << 8) + m2 * 16 + c], s);
        sA[(I * kSub + r) * AP + J * kSub + c] = -s;
    }
    __syncthreads();
    // level 2: Tm[32:64, 0:32] = -Tm_hi (A[32:64, 0:32] Tm_lo)
    for (int idx = tid; idx < 1024; idx += NTH) {
        const int r = idx >> 5, c = idx & 31;
        float s = 0.f;
#pragma unroll 8
        for (int m2 = 0; m2 < 32; ++m2) s = fmaf(sA[(32 + r) * AP + m2], sA[m2 * AP + c], s);
        sS[r * 33 + c] = s;
    }
    __syncthreads();
    {
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * NTH;
            const int r = idx >> 5, c = idx & 31;
            float s = 0.f;
#pragma unroll 8
            for (int m2 = 0; m2 < 32; ++m2) s = fmaf(sA[(32 + r) * AP + 32 + m2], sS[m2 * 33 + c], s);
            res[j] = -s;
        }
        // A[32:64, 0:32] is read above by no thread; Tm_hi lives in [32:64, 32:64].
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * NTH;
            sA[(32 + (idx >> 5)) * AP + (idx & 31)] = res[j];
        }
    }
    __syncthreads();

    // ---- w and u on the matrix cores ----
    Frag<E> tf[6];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int s = 0; s <= (m >> 1); ++s) {
            const int row = m * kSub + li;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int col = s * kSlab + 16 * hf + 4 * lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) tf[tri_frag(m, s)].set(4 * hf + r, sA[row * AP + col + r]);
            }
        }
    }
    if (wave < KS) {
        // w slab `wave` (key channels 32 wave ..), computed transposed as
        // X^T Tm^T: lane (i, g) receives w[16m + i][16n + 4g + r], the scan's
        // A-operand order.
        f32x4 acc[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) {
                acc[m][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= (m >> 1); ++s) mma(acc[m][nn], xf[nn][s], tf[tri_frag(m, s)]);
            }
            store_frag<E>(Rw + (m * KS + wave) * 512, lane, frag_from_tiles<E>(acc[m][0], acc[m][1]));
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
                vf[s].set(e, sBeta[row] * (float)sQV[row * QP + ch]);
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
}

// ---------------------------------------------------------------------------
// State scan
// ---------------------------------------------------------------------------

// Operands of one chunk for one wave (row tile m = wave, TPW key tiles).
template <typename E, int DK> struct ScanStage {
    static constexpr int KS = DK / kSlab;
    static constexpr int TPW = DK / 64;
    Frag<E> wf[KS], qf[KS], af[2], kf[TPW][2];
    f32x4 u, d[TPW];
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
    // bf16/fp32 copies of the state slabs and of U, [slab][lane][8]
    __shared__ __align__(16) E sSb[KS * 64 * 8];
    __shared__ __align__(16) E sUb[2 * 64 * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // Keep the d_v slices of one (sequence, head) on one XCD: workgroups are
    // dealt to the 8 XCDs round robin, so block b runs on XCD b % 8.
    const int B = gridDim.x, b = blockIdx.x;
    const int lin = (B % 8 == 0) ? (b % 8) * (B / 8) + b / 8 : b;
    const int jt = lin % VT;
    const int h = (lin / VT) % H;
    const int n = lin / (VT * H);
    if (n >= N) return;
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

    auto load_stage = [&](Stage &X, int cc) {
        const size_t rec = (size_t)(sp.first_chunk + cc) * H + h;
        const E *Rw = ws + rec * L::kRecElems;
        const E *Rq = Rw + L::kWElems;
        const E *Rk = Rq + L::kQElems;
        const E *Ra = Rk + L::kKElems;
        const E *Ru = Ra + L::kAElems;
#pragma unroll
        for (int s = 0; s < KS; ++s) X.wf[s] = load_frag<E>(Rw + (wave * KS + s) * 512, lane);
#pragma unroll
        for (int s = 0; s < KS; ++s) X.qf[s] = load_frag<E>(Rq + (wave * KS + s) * 512, lane);
        X.af[0] = load_frag<E>(Ra + tri_frag(wave, 0) * 512, lane);
        if (wave >= 2) X.af[1] = load_frag<E>(Ra + tri_frag(wave, 1) * 512, lane);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave * TPW + i;
            X.kf[i][0] = load_frag<E>(Rk + (t * 2) * 512, lane);
            X.kf[i][1] = load_frag<E>(Rk + (t * 2 + 1) * 512, lane);
            X.d[i] = *reinterpret_cast<const f32x4 *>(ws_dec + rec * DK + t * kSub + 4 * lg);
        }
        X.u = load4<E>(Ru + jt * (64 * 16) + lane * 16 + 4 * wave);
    };

    auto step = [&](const Stage &X, int cc) {
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
        // my tile of U = u - w S
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(acc, X.wf[s], Sb[s]);
        const f32x4 un = X.u - acc;
        store4<E>(sUb + ((wave >> 1) * 64 + lane) * 8 + (wave & 1) * 4, un);
        __syncthreads();
        Frag<E> ub[2];
        ub[0] = load_frag<E>(sUb, lane);
        ub[1] = load_frag<E>(sUb + 512, lane);
        // my tile of O = Q~ S + A_qk U, transposed products: lane holds row
        // 16 wave + i, columns j0 + 4g + r
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(acc, Sb[s], X.qf[s]);
        mma(acc, ub[0], X.af[0]);
        if (wave >= 2) mma(acc, ub[1], X.af[1]);
        const int row = wave * kSub + li;
        if (row < sp.len - cc * kChunk)
            store4<E>(o + ((size_t)(sp.start + cc * kChunk + row) * H + h) * DV + j0 + 4 * lg, acc * scale);
        // my key tiles of S = diag(e^{Gam_C}) S + K~^T U
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            S[i] *= X.d[i];
            mma(S[i], X.kf[i][0], ub[0]);
            mma(S[i], X.kf[i][1], ub[1]);
        }
    };

    const int nch = (sp.len + kChunk - 1) / kChunk;
    Stage A, Bs;
    if (nch > 0) load_stage(A, 0);
    if (nch > 1) load_stage(Bs, 1);
    for (int cc = 0; cc < nch; cc += 2) {
        step(A, cc);
        if (cc + 2 < nch) load_stage(A, cc + 2);
        if (cc + 1 < nch) {
            step(Bs, cc + 1);
            if (cc + 3 < nch) load_stage(Bs, cc + 3);
        }
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
        kda_intra_kernel<E, DK, DV><<<dim3(max_chunks, a.H), dim3(256), 0, stream>>>(
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
