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
// parallel.  It builds Gam, A_kk and A_qk (off-diagonal 16x16 blocks on the
// matrix cores with both gating factors <= 1, diagonal blocks exactly in fp32
// with one exp per element), inverts I + A_kk by blocked forward
// substitution in LDS, forms w and u on the matrix cores, and writes w,
// Q*e^Gam, (K*e^{Gam_C-Gam})^T, A_qk, u and e^{Gam_C} to the workspace in the
// scan's register order.
//
// kda_scan_kernel: one wave per (sequence, head, 16-column slice of d_v).
// The d_v columns of S evolve independently, so the slices need no exchange.
// The wave keeps its d_k x 16 slice of S in fp32 registers and walks the
// sequence's chunks in order: U = u - w S, O = Q~ S + A_qk U,
// S = diag(e^{Gam_C}) S + K~^T U.  All four products run on the matrix cores
// with the operands straight from the workspace.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void kda_intra_kernel(
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
    constexpr int GP = DK + 4;                         // row pitch of sG (floats)
    constexpr int AP = 65;                             // row pitch of the 64x64 matrices
    constexpr int KS = DK / kSlab;                     // d_k slabs
    constexpr int KT = DK / kSub;                      // d_k tiles
    constexpr int VT = DV / kSub;                      // d_v tiles
    using L = WsLayout<E, DK, DV>;

    __shared__ __align__(16) E sK[kChunk * KP];
    __shared__ __align__(16) E sQV[kChunk * QP];       // Q, later V
    __shared__ __align__(16) float sG[kChunk * GP];    // Gam * log2(e)
    __shared__ __align__(16) float sA[kChunk * AP];    // A_kk, strictly lower, beta-scaled
    __shared__ __align__(16) float sAT[kChunk * AP];   // A_qk, later Tm
    __shared__ __align__(16) float sScr[32 * 33];      // cumsum partials / inverse scratch
    __shared__ float sBeta[kChunk];

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
    E *R = ws + rec * L::kRecElems;
    E *Rw = R;
    E *Rq = Rw + L::kWElems;
    E *Rk = Rq + L::kQElems;
    E *Ra = Rk + L::kKElems;
    E *Ru = Ra + L::kAElems;

    // ---- load K, Q to LDS; V to registers (it lands where Q was) ----
    constexpr int EPU = 16 / sizeof(E);                // elements per 16-byte unit
    constexpr int UK = kChunk * DK / EPU;
    constexpr int UV = kChunk * DV / EPU;
    constexpr int VPT = UV / NTH;
    for (int u = tid; u < UK; u += NTH) {
        const int r = u / (DK / EPU), c = (u % (DK / EPU)) * EPU;
        uint4 xk = {0, 0, 0, 0}, xq = {0, 0, 0, 0};
        if (r < C) {
            const size_t off = ((size_t)(row0 + r) * H + h) * DK + c;
            xk = *reinterpret_cast<const uint4 *>(k + off);
            xq = *reinterpret_cast<const uint4 *>(q + off);
        }
        *reinterpret_cast<uint4 *>(sK + r * KP + c) = xk;
        *reinterpret_cast<uint4 *>(sQV + r * QP + c) = xq;
    }
    uint4 vreg[VPT];
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
        vreg[p] = uint4{0, 0, 0, 0};
        if (r < C) vreg[p] = *reinterpret_cast<const uint4 *>(v + ((size_t)(row0 + r) * H + h) * DV + c);
    }
    if (tid < kChunk) sBeta[tid] = tid < C ? beta[(size_t)(row0 + tid) * H + h] : 0.f;

    // ---- Gam: inclusive cumsum of g over rows, per channel ----
    {
        constexpr int PARTS = NTH / DK;
        constexpr int RP = kChunk / PARTS;
        const int c = tid % DK, part = tid / DK;
        float gv[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const int row = part * RP + r;
            gv[r] = row < C ? g[((size_t)(row0 + row) * H + h) * DK + c] : 0.f;
        }
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < RP; ++r) { acc += gv[r]; gv[r] = acc; }
        sScr[part * DK + c] = acc;
        __syncthreads();
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += sScr[p * DK + c];
#pragma unroll
        for (int r = 0; r < RP; ++r) sG[(part * RP + r) * GP + c] = (gv[r] + off) * kLog2e;
    }
    __syncthreads();

    // ---- Q * e^Gam fragments (A operand of the scan's output product) ----
    {
        const int m = wave;
        const int row = m * kSub + li;
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
            store_frag<E>(Rq + (m * KS + s) * 512, lane, f);
        }
    }

    // ---- A_kk, A_qk: zero the upper blocks ----
    for (int idx = tid; idx < 6 * 256; idx += NTH) {
        const int b = idx >> 8, e = idx & 255;
        const int I = b < 3 ? 0 : (b < 5 ? 1 : 2);
        const int J = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
        const int r = I * kSub + (e >> 4), c = J * kSub + (e & 15);
        sA[r * AP + c] = 0.f;
        sAT[r * AP + c] = 0.f;
    }
    // ---- off-diagonal blocks (I > J) on the matrix cores ----
    // Reference row ref = 16 I - 1: rows of block I take e^{Gam_r - Gam_ref},
    // rows of block J take e^{Gam_ref - Gam_s}; both exponents are <= 0.
    for (int p = wave; p < 6; p += 4) {
        const int I = p == 0 ? 1 : (p < 3 ? 2 : 3);
        const int J = p == 0 ? 0 : (p < 3 ? p - 1 : p - 3);
        const int ref = I * kSub - 1;
        const int ra = I * kSub + li, rb = J * kSub + li;
        f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = I * kSub + 4 * lg + r, col = J * kSub + li;
            sA[row * AP + col] = accK[r] * sBeta[row];
            sAT[row * AP + col] = accQ[r];
        }
    }
    // ---- diagonal blocks, exact: one exp per (row, col, channel) ----
    {
        const int I = wave;
        const int jj = li, cq = lg;
        constexpr int CQ = DK / 4;
        float accK[kSub], accQ[kSub];
#pragma unroll
        for (int ii = 0; ii < kSub; ++ii) { accK[ii] = 0.f; accQ[ii] = 0.f; }
        const int rj = I * kSub + jj;
        for (int c = cq * CQ; c < (cq + 1) * CQ; c += 4) {
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
                    const float e = ii >= jj ? fast_exp2(gi[r] - gj[r]) : 0.f;
                    const float t = kj[r] * e;
                    accK[ii] = fmaf(ki[r], t, accK[ii]);
                    accQ[ii] = fmaf(qi[r], t, accQ[ii]);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < kSub; ++ii) {
            accK[ii] += __shfl_xor(accK[ii], 16);
            accK[ii] += __shfl_xor(accK[ii], 32);
            accQ[ii] += __shfl_xor(accQ[ii], 16);
            accQ[ii] += __shfl_xor(accQ[ii], 32);
        }
#pragma unroll
        for (int ii = 0; ii < kSub; ++ii) {
            if ((ii >> 2) == cq) {
                const int row = I * kSub + ii, col = I * kSub + jj;
                sA[row * AP + col] = ii > jj ? accK[ii] * sBeta[row] : 0.f;
                sAT[row * AP + col] = ii >= jj ? accQ[ii] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- A_qk fragments (A operand of the scan's A_qk U product) ----
    {
        const int m = wave;
        const int row = m * kSub + li;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            Frag<E> f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int col = s * kSlab + 16 * hf + 4 * lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) f.set(4 * hf + r, sAT[row * AP + col + r]);
            }
            store_frag<E>(Ra + (m * 2 + s) * 512, lane, f);
        }
    }
    __syncthreads();

    // ---- V into the Q region; diagonal inverses; K~^T fragments ----
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
        const int u = tid + p * NTH;
        const int r = u / (DV / EPU), c = (u % (DV / EPU)) * EPU;
        *reinterpret_cast<uint4 *>(sQV + r * QP + c) = vreg[p];
    }
    if (wave == 0) {
        // Tm_II = (I + A_II)^-1 by forward substitution, lane = (block, column).
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
        for (int ii = 0; ii < kSub; ++ii) sAT[(I * kSub + ii) * AP + I * kSub + jj] = t[ii];
        // The blocks above the diagonal of sAT were zeroed for A_qk and stay
        // zero for Tm; the blocks below it are overwritten next.
    } else {
        // K~ = K * e^{Gam_C - Gam}, stored transposed: fragment (t, s) holds
        // rows 16t..16t+15 of K~^T (key channels) over chunk rows 32s..32s+31.
        // Rows past C are zero in K, and Gam is flat there, so row 63 holds Gam_C.
        for (int f = wave - 1; f < KT * 2; f += 3) {
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
        const int c = tid - 64;
        if (c < DK) ws_dec[rec * DK + c] = fast_exp2(sG[(kChunk - 1) * GP + c]);
    }
    __syncthreads();

    // ---- off-diagonal blocks of Tm ----
    // level 1: Tm_10 = -Tm_11 A_10 Tm_00, Tm_32 = -Tm_33 A_32 Tm_22
    for (int idx = tid; idx < 512; idx += NTH) {
        const int which = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int I = which ? 3 : 1, J = I - 1;
        float s = 0.f;
#pragma unroll
        for (int m2 = 0; m2 < kSub; ++m2)
            s = fmaf(sA[(I * kSub + r) * AP + J * kSub + m2], sAT[(J * kSub + m2) * AP + J * kSub + c], s);
        sScr[idx] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < 512; idx += NTH) {
        const int which = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int I = which ? 3 : 1, J = I - 1;
        float s = 0.f;
#pragma unroll
        for (int m2 = 0; m2 < kSub; ++m2)
            s = fmaf(sAT[(I * kSub + r) * AP + I * kSub + m2], sScr[(which << 8) + m2 * 16 + c], s);
        sAT[(I * kSub + r) * AP + J * kSub + c] = -s;
    }
    __syncthreads();
    // level 2: Tm[32:64, 0:32] = -Tm_hi (A[32:64, 0:32] Tm_lo)
    for (int idx = tid; idx < 1024; idx += NTH) {
        const int r = idx >> 5, c = idx & 31;
        float s = 0.f;
#pragma unroll 8
        for (int m2 = 0; m2 < 32; ++m2) s = fmaf(sA[(32 + r) * AP + m2], sAT[m2 * AP + c], s);
        sScr[r * 33 + c] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < 1024; idx += NTH) {
        const int r = idx >> 5, c = idx & 31;
        float s = 0.f;
#pragma unroll 8
        for (int m2 = 0; m2 < 32; ++m2) s = fmaf(sAT[(32 + r) * AP + 32 + m2], sScr[m2 * 33 + c], s);
        sAT[(32 + r) * AP + c] = -s;
    }
    __syncthreads();

    // ---- w and u on the matrix cores ----
    // Tm fragments (A operand, row tile m, chunk-row slab s <= m/2).
    Frag<E> tf[6];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int s = 0; s <= (m >> 1); ++s) {
            const int fi = m == 0 ? 0 : (m == 1 ? 1 : (m == 2 ? 2 + s : 4 + s));
            const int row = m * kSub + li;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int col = s * kSlab + 16 * hf + 4 * lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) tf[fi].set(4 * hf + r, sAT[row * AP + col + r]);
            }
        }
    }
    for (int it = wave; it < KS + VT; it += 4) {
        if (it < KS) {
            // w slab it (key channels 32 it .. 32 it + 31), computed transposed:
            // (X^T Tm^T) with X = diag(beta) K e^Gam gives lane (i, g) the
            // values w[16m + i][16n + 4g + r], the scan's A-operand order.
            f32x4 acc[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m) { acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f}; acc[m][1] = acc[m][0]; }
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) {
                const int ch = (2 * it + nn) * kSub + li;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    Frag<E> xf;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = s * kSlab + kk_of(lg, e);
                        xf.set(e, sBeta[row] * (float)sK[row * KP + ch] * fast_exp2(sG[row * GP + ch]));
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        if (s <= (m >> 1)) {
                            const int fi = m == 0 ? 0 : (m == 1 ? 1 : (m == 2 ? 2 + s : 4 + s));
                            mma(acc[m][nn], xf, tf[fi]);
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                Frag<E> out = frag_from_tiles<E>(acc[m][0], acc[m][1]);
                store_frag<E>(Rw + (m * KS + it) * 512, lane, out);
            }
        } else {
            // u tile (value columns 16 jt .. 16 jt + 15): Tm diag(beta) V,
            // lane (i, g) holds u[16m + 4g + r][16 jt + i].
            const int jt = it - KS;
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
                for (int s = 0; s <= (m >> 1); ++s) {
                    const int fi = m == 0 ? 0 : (m == 1 ? 1 : (m == 2 ? 2 + s : 4 + s));
                    mma(acc, tf[fi], vf[s]);
                }
                store4<E>(dst + 4 * m, acc);
            }
        }
    }
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(64) void kda_scan_kernel(
    const E *__restrict__ ws, const float *__restrict__ ws_dec,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ slots,
    const float *state_in, float *state_out, E *__restrict__ o,
    int T, int N, int H, int num_slots, float scale) {
    constexpr int VT = DV / kSub, KS = DK / kSlab, KT = DK / kSub;
    using L = WsLayout<E, DK, DV>;
    const int lane = threadIdx.x, li = lane & 15, lg = lane >> 4;
    // Spread the d_v slices of one (sequence, head) over one XCD: workgroups
    // are dealt to the 8 XCDs round robin, so block b runs on XCD b % 8.
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

    f32x4 S[KT];
    if (state_in) {
        const float *src = state_in + (((size_t)slot * H + h) * DV + j0 + li) * DK;
#pragma unroll
        for (int t = 0; t < KT; ++t) S[t] = *reinterpret_cast<const f32x4 *>(src + t * kSub + 4 * lg);
    } else {
#pragma unroll
        for (int t = 0; t < KT; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nch = (sp.len + kChunk - 1) / kChunk;
    for (int cc = 0; cc < nch; ++cc) {
        const size_t rec = (size_t)(sp.first_chunk + cc) * H + h;
        const E *Rw = ws + rec * L::kRecElems;
        const E *Rq = Rw + L::kWElems;
        const E *Rk = Rq + L::kQElems;
        const E *Ra = Rk + L::kKElems;
        const E *Ru = Ra + L::kAElems + jt * (64 * 16) + lane * 16;
        const float *Dc = ws_dec + rec * DK;
        const int C = min(kChunk, sp.len - cc * kChunk);

        Frag<E> Sb[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) Sb[s] = frag_from_tiles<E>(S[2 * s], S[2 * s + 1]);

        // U = u - w S   (C layout: lane holds rows 16m + 4g + r, column j0 + i)
        f32x4 un[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) mma(acc, load_frag<E>(Rw + (m * KS + s) * 512, lane), Sb[s]);
            un[m] = load4<E>(Ru + 4 * m) - acc;
        }
        Frag<E> ub[2];
        ub[0] = frag_from_tiles<E>(un[0], un[1]);
        ub[1] = frag_from_tiles<E>(un[2], un[3]);

        // O = Q~ S + A_qk U, transposed products: lane holds row 16m + i,
        // columns j0 + 4g + r, so each lane writes four adjacent outputs.
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) mma(acc, Sb[s], load_frag<E>(Rq + (m * KS + s) * 512, lane));
#pragma unroll
            for (int s = 0; s <= (m >> 1); ++s) mma(acc, ub[s], load_frag<E>(Ra + (m * 2 + s) * 512, lane));
            const int row = m * kSub + li;
            if (row < C)
                store4<E>(o + ((size_t)(sp.start + cc * kChunk + row) * H + h) * DV + j0 + 4 * lg, acc * scale);
        }

        // S = diag(e^{Gam_C}) S + K~^T U
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Dc + t * kSub + 4 * lg);
            S[t] *= d4;
#pragma unroll
            for (int s = 0; s < 2; ++s) mma(S[t], load_frag<E>(Rk + (t * 2 + s) * 512, lane), ub[s]);
        }
    }

    if (state_out) {
        float *dst = state_out + (((size_t)slot * H + h) * DV + j0 + li) * DK;
#pragma unroll
        for (int t = 0; t < KT; ++t) *reinterpret_cast<f32x4 *>(dst + t * kSub + 4 * lg) = S[t];
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
    kda_scan_kernel<E, DK, DV><<<dim3(nblocks), dim3(64), 0, stream>>>(
        ws, ws_dec, a.cu_seqlens, a.slots, a.state_in, a.state_out, static_cast<E *>(a.o),
        a.T, a.N, a.H, a.num_slots, a.scale);
    const hipError_t e = hipGetLastError();
    if (a.events[2]) (void)hipEventRecord(a.events[2], stream);
    return e;
}

size_t prefill_workspace_bytes(int T, int N, int H, int dk, int dv, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const size_t rec = (size_t)kChunk * (2 * dk + dk + kChunk + dv);
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
