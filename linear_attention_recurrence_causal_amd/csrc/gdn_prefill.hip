// gdn_prefill.hip -- fused single-pass chunked prefill of the Gated DeltaNet
// core (gfx950): the path taken when the caller passes no workspace.
//
// The chunked form and the MFMA operand layout are described in
// gdn_chunk_common.h.  One workgroup owns (sequence b, value head h, a slice
// of N = 16*NW state columns); wave w owns 16 columns and keeps its 128 x 16
// fp32 slice of S in MFMA accumulator registers for the whole call.  Per
// chunk:
//   front  raw qkv (+3-token halo, or the carried conv state) -> depthwise
//          conv (fp32) -> SiLU -> bf16 -> LDS (Q, K, V^T)
//   rows   K^T, gates g, beta (fp32) and the inclusive scan of g, L2 norms
//   masks  K K^T and Q K^T lower 16x16 tiles on MFMA (bf16 in, fp32 out),
//          decay masks -> A and P (bf16)
//   diag   inverses of the 16x16 diagonal blocks of I + A by substitution
//   state  per wave, on MFMA: K S0, Q S0 (S0 as bf16), R, Delta by blocked
//          forward substitution, and S <- exp(gamma_C) S + K^T Delta' with
//          Delta' split into bf16 hi + lo (two MFMAs): the product that builds
//          the state carries ~16 significant bits, everything else bf16
//          operands with fp32 accumulate
//   out    O = Gamma n_q Q S0 + P Delta, O rows -> HBM (16-byte stores);
//          checkpoint slots when the chunk end is a multiple of the interval.
// The chunk loop is software-pipelined: the S-independent work of chunk c + 1
// (front, rows, masks, diag; double-buffered Q, K, V^T) runs beside the state
// and output work of chunk c.
#include "gdn_chunk_common.h"

namespace gdn {

namespace {

using namespace chunked;

constexpr int kVtLd = kC + 12;      // bf16 row stride of V^T

template <int NW, bool PRECISE = false>
struct alignas(16) Smem {
    static constexpr int N = 16 * NW;
    static constexpr int VLd = N + 8;
    static constexpr int NCH = 2 * kD + N;
    // Double-buffered per chunk: while the state phase of chunk c reads
    // buffer c % 2, the front end of chunk c + 1 fills the other one.
    __bf16 Ks[2][kC * kKsLd];
    __bf16 Qs[2][kC * kKsLd];     // Qs[c % 2] also stages chunk c's output once Q S0 is done
    __bf16 Vt[2][N * kVtLd];      // V transposed: [column][token]
    __bf16 Kt[kD * kKtLd];
    __bf16 Ps[kC * kKtLd];        // P = M .* (n_q n_k^T) .* Q K^T, lower incl. diagonal
    __bf16 AN[kC * kKtLd];        // -A below the diagonal blocks, T_mm - I on them
    float AdT[4 * 16 * kXLd];     // the four diagonal 16x16 blocks of A, transposed (fp32)
    float Ws[4 * NCH];            // conv taps, [tap][channel]
    alignas(16) float beta[kC];
    alignas(16) float gam[kC];
    alignas(16) float nq[kC];
    alignas(16) float nk[kC];
    float tokS[4][kC];            // per row: beta | beta Gamma n_k | Gamma n_q | exp(gamma_C - gamma) n_k
    // precise mode: the bf16 lo parts of P and AN (same layout)
    __bf16 Ps_lo[PRECISE ? kC * kKtLd : 8];
    __bf16 AN_lo[PRECISE ? kC * kKtLd : 8];
    static_assert(kC * VLd <= kC * kKsLd, "output staging fits a Q buffer");
    static_assert(NW != 8 || (10 * 64 * 16 <= kC * kKsLd * 2 && 10 * 64 * 16 <= N * kVtLd * 2),
                  "raw Gram tiles fit the dead K and V^T buffers");
};

// Global channel of the WG's channel index ch (q: 0..127, k: 128..255, v: 256..)
__device__ __forceinline__ int64_t global_channel(int ch, int kh, int h, int zcol0, int Hk) {
    if (ch < kD) return (int64_t)kh * kD + ch;
    if (ch < 2 * kD) return (int64_t)Hk * kD + (int64_t)kh * kD + (ch - kD);
    return 2 * (int64_t)Hk * kD + (int64_t)h * kD + zcol0 + (ch - 2 * kD);
}

// Per-workgroup constants.
struct Ctx {
    int b, kh, h, zcol0;
    int64_t L, sp;
    float neg_A, dt_h;
};

constexpr int kTilesPerWave = 4;   // 20 Gram tiles over waves 3..7

// Front end of one work item (4 channels x 8 chunk rows) into buffer `buf`:
// q, k channels -> Q, K rows, v channels -> V^T rows.
template <bool INTERIOR, int NW, class SM>
__device__ __forceinline__ void front_item(const PrefillParams& p, SM& sm, const Ctx& cx, int buf,
                                           int64_t local0, int item) {
    constexpr int NCH = SM::NCH;
    constexpr int CG4 = NCH / 4;
    const int cg = item % CG4, seg = item / CG4;
    const int ch0 = cg * 4;
    const int64_t gc = global_channel(ch0, cx.kh, cx.h, cx.zcol0, p.num_k_heads);
    const int tau0 = seg * 8;
    float w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(&sm.Ws[j * NCH + ch0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[j][i] = wv[i];
    }
    bf16x4 ub[8];
    conv_item<INTERIOR>(p, cx.b, gc, local0, tau0, w, ub);
    if (ch0 >= 2 * kD) {
        // v channels: 8 tokens of each of the 4 channels, stored as V^T rows
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 col{ub[0][i], ub[1][i], ub[2][i], ub[3][i], ub[4][i], ub[5][i], ub[6][i], ub[7][i]};
            *reinterpret_cast<bf16x8*>(&sm.Vt[buf][(ch0 - 2 * kD + i) * kVtLd + tau0]) = col;
        }
    } else {
        __bf16* dst0 = ch0 < kD ? &sm.Qs[buf][pos(ch0)] : &sm.Ks[buf][pos(ch0 - kD)];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) *reinterpret_cast<bf16x4*>(dst0 + (tau0 + tt) * kKsLd) = ub[tt];
    }
}

// ---- A1: front end of a chunk into Q, K, V^T buffer `buf`
template <int NW, class SM>
__device__ __forceinline__ void phase_front(const PrefillParams& p, SM& sm, const Ctx& cx, int buf,
                                            int64_t local0, int tid) {
    constexpr int NT = 64 * NW;
    constexpr int CG4 = SM::NCH / 4;
    // interior chunks (all 64 rows and the 3-row halo inside the call) take a
    // path with no clamping and no masking
    if (local0 >= 3 && local0 + kC <= cx.L) {
        for (int item = tid; item < CG4 * 8; item += NT) front_item<true, NW>(p, sm, cx, buf, local0, item);
    } else {
        for (int item = tid; item < CG4 * 8; item += NT) front_item<false, NW>(p, sm, cx, buf, local0, item);
    }
}

// ---- A2: K^T, gates + inclusive scan of g, L2 norms; with 8 waves also the
// raw Gram tiles, into the dead K / V^T buffer `gbuf` (fp32, accumulator layout)
template <int NW, class SM>
__device__ __forceinline__ void phase_rows(const PrefillParams& p, SM& sm, const Ctx& cx, int buf,
                                           int gbuf, int64_t local0, int tid) {
    constexpr int NT = 64 * NW;
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, lq = lane / 16;
    const __bf16* Ks = sm.Ks[buf];
    const __bf16* Qs = sm.Qs[buf];
    for (int e = tid; e < kD * (kC / 8); e += NT) {
        // K^T[d][tau0 .. tau0+7] from eight K rows; lanes walk d, so the
        // 2-byte LDS reads of one instruction hit consecutive addresses
        const int d = e % kD, tau0 = (e / kD) * 8;
        const int pd = pos(d);
        bf16x4 c0, c1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c0[i] = Ks[(tau0 + i) * kKsLd + pd];
            c1[i] = Ks[(tau0 + 4 + i) * kKsLd + pd];
        }
        *reinterpret_cast<bf16x4*>(&sm.Kt[d * kKtLd + pos(tau0)]) = c0;
        *reinterpret_cast<bf16x4*>(&sm.Kt[d * kKtLd + pos(tau0 + 4)]) = c1;
    }
    for (int job = tid; job < 3 * kC; job += NT) {
        if (job < kC) {
            gates_scan(p, cx.b, cx.h, cx.neg_A, cx.dt_h, local0, lane, sm.gam, sm.beta);
        } else {
            const bool isq = job < 2 * kC;
            const int tau = job % kC;
            const float n = row_inv_norm((isq ? Qs : Ks) + tau * kKsLd, isq ? p.q_scale : 1.0f, p.l2_eps);
            (isq ? sm.nq : sm.nk)[tau] = n;
        }
    }
    if constexpr (NW == 8) {
        // raw K K^T / Q K^T tiles need only Q and K: waves 3..7 (idle after
        // the K^T copy) compute them here; the masks follow in A3
        if (wave >= 3) {
            f32x4* G = reinterpret_cast<f32x4*>(sm.Ks[gbuf]);
            f32x4* GQ = reinterpret_cast<f32x4*>(sm.Vt[gbuf]);
#pragma unroll 1
            for (int k = 0; k < kTilesPerWave; ++k) {
                const int ti = (wave - 3) + 5 * k;
                const f32x4 t = gram_tile(Ks, Qs, ti, li, lq);
                if (ti < 10) G[ti * 64 + lane] = t;
                else GQ[(ti - 10) * 64 + lane] = t;
            }
        }
    }
}

// ---- A3: decay masks on the Gram tiles; per-row scales
template <int NW, bool PRECISE, class SM>
__device__ __forceinline__ void phase_masks(SM& sm, int buf, int gbuf, int tid) {
    constexpr int NT = 64 * NW;
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, lq = lane / 16;
    if constexpr (NW == 8) {
        // job = (tile pair, lane): both the K K^T and the Q K^T tile of one
        // lower tile pair, 640 jobs over 512 threads, branch-free within a wave
        const f32x4* G = reinterpret_cast<const f32x4*>(sm.Ks[gbuf]);
        const f32x4* GQ = reinterpret_cast<const f32x4*>(sm.Vt[gbuf]);
        for (int j = tid; j < 10 * 64; j += NT) mask_pair<PRECISE>(sm, j >> 6, G[j], GQ[j], j & 63);
        if (wave == NW - 1) row_scales(sm, lane);
    } else {
        if (wave == 0) row_scales(sm, lane);
        for (int pi = wave - 1; pi >= 0 && pi < 10; pi += NW - 1)
            mask_pair<PRECISE>(sm, pi, gram_tile(sm.Ks[buf], sm.Qs[buf], pi, li, lq),
                      gram_tile(sm.Ks[buf], sm.Qs[buf], 10 + pi, li, lq), lane);
    }
}

// ---- B1: state-dependent products of a chunk, per wave (16 state columns):
// K S0, Q S0, R, the blocked substitution for Delta, and the state update.
// Every block of LDS operands is loaded in one batch (fenced with a
// scheduling barrier) before the products that use it.  Returns Q S0 and
// Delta (bf16, as the B operands of P Delta) for B2.
template <class SM>
__device__ __forceinline__ void phase_state(SM& sm, int buf, f32x4 S[8], f32x4 QS[4], bf16x8 BD[2], bf16x8*,
                                            int wave, int li, int lq) {
    const int cw = 16 * wave + li;   // column inside the slice
    const __bf16* Ks = sm.Ks[buf];
    const __bf16* Qs = sm.Qs[buf];
    bf16x8 Bs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Bs[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
    f32x4 KS[4];
#pragma unroll
    for (int mh = 0; mh < 4; mh += 2) {
        bf16x8 ak[2][4], aq[2][4];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = (16 * (mh + mm) + li) * kKsLd + 32 * ks + 8 * lq;
                ak[mm][ks] = lds_load8(&Ks[off]);
                aq[mm][ks] = lds_load8(&Qs[off]);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            f32x4 k = {0.f, 0.f, 0.f, 0.f}, q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                k = mfma16(ak[mm][ks], Bs[ks], k);
                q = mfma16(aq[mm][ks], Bs[ks], q);
            }
            KS[mh + mm] = k;
            QS[mh + mm] = q;
        }
    }
    // row scales and V for this lane's 16 rows (16m + 4 lq + e), and the A
    // operands of the substitution (token block k of an AN row sits at
    // 32(k/2) + 8 lq + 4(k%2))
    f32x4 sb[4], sr[4];
    bf16x4 vv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = 16 * m + 4 * lq;
        sb[m] = *reinterpret_cast<const f32x4*>(&sm.tokS[0][r0]);
        sr[m] = *reinterpret_cast<const f32x4*>(&sm.tokS[1][r0]);
        vv[m] = lds_load4(&sm.Vt[buf][cw * kVtLd + r0]);
    }
    const __bf16* an = &sm.AN[li * kKtLd + 8 * lq];
    const bf16x4 d0 = lds_load4(an), d1 = lds_load4(an + 16 * kKtLd + 4);
    const bf16x4 d2 = lds_load4(an + 32 * kKtLd + 32), d3 = lds_load4(an + 48 * kKtLd + 36);
    const bf16x4 a10 = lds_load4(an + 16 * kKtLd);
    const bf16x8 a2x = lds_load8(an + 32 * kKtLd), a3x = lds_load8(an + 48 * kKtLd);
    const bf16x4 a32 = lds_load4(an + 48 * kKtLd + 32);
    __builtin_amdgcn_sched_barrier(0);
    // R = beta V - beta Gamma n_k (K S0)
    f32x4 R[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) R[m][e] = sb[m][e] * float(vv[m][e]) - sr[m][e] * KS[m][e];
    f32x4 Dl[4];
    bf16x4 Db[4];
    const bf16x4 dg[4] = {d0, d1, d2, d3};
    delta_substitution(R, dg, a10, a2x, a3x, a32, Dl, Db);
    BD[0] = cat4(Db[0], Db[1]);
    BD[1] = cat4(Db[2], Db[3]);
    // S <- exp(gamma_C) S + K^T Delta',  Delta' = exp(gamma_C - gamma) n_k Delta  (hi + lo)
    f32x4 su[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) su[m] = *reinterpret_cast<const f32x4*>(&sm.tokS[3][16 * m + 4 * lq]);
    bf16x8 akt[8][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) akt[t][ks] = lds_load8(&sm.Kt[(16 * t + li) * kKtLd + 32 * ks + 8 * lq]);
    const float eC = expf(sm.gam[kC - 1]);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 BH[2], BL[2];
    split_hi_lo(su, Dl, BH, BL);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t == 4) {
            // second half of the K^T operands
#pragma unroll
            for (int tt = 4; tt < 8; ++tt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    akt[tt][ks] = lds_load8(&sm.Kt[(16 * tt + li) * kKtLd + 32 * ks + 8 * lq]);
        }
        f32x4 acc = S[t] * eC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            acc = mfma16(akt[t][ks], BH[ks], acc);
            acc = mfma16(akt[t][ks], BL[ks], acc);
        }
        S[t] = acc;
    }
}

// ---- B1 of the precise mode: the same products with the substitution
// (delta_substitution_hl) and Delta on bf16 hi + lo operands (three MFMAs
// per product, the lo x lo term dropped); Q S0 and K S0 take S0 rounded once
// to bf16, as in the default precision.  Returns Delta's hi and lo parts for
// B2.
template <class SM>
__device__ __forceinline__ void phase_state_hl(SM& sm, int buf, f32x4 S[8], f32x4 QS[4], bf16x8 BD[2],
                                               bf16x8 BDl[2], int wave, int li, int lq) {
    const int cw = 16 * wave + li;
    const __bf16* Ks = sm.Ks[buf];
    const __bf16* Qs = sm.Qs[buf];
    bf16x8 Bh[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Bh[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
    f32x4 KS[4];
#pragma unroll
    for (int mh = 0; mh < 4; mh += 2) {
        bf16x8 ak[2][4], aq[2][4];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = (16 * (mh + mm) + li) * kKsLd + 32 * ks + 8 * lq;
                ak[mm][ks] = lds_load8(&Ks[off]);
                aq[mm][ks] = lds_load8(&Qs[off]);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            f32x4 k = {0.f, 0.f, 0.f, 0.f}, q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                k = mfma16(ak[mm][ks], Bh[ks], k);
                q = mfma16(aq[mm][ks], Bh[ks], q);
            }
            KS[mh + mm] = k;
            QS[mh + mm] = q;
        }
    }
    f32x4 R[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = 16 * m + 4 * lq;
        const f32x4 sb = *reinterpret_cast<const f32x4*>(&sm.tokS[0][r0]);
        const f32x4 sr = *reinterpret_cast<const f32x4*>(&sm.tokS[1][r0]);
        const bf16x4 vv = lds_load4(&sm.Vt[buf][cw * kVtLd + r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) R[m][e] = sb[e] * float(vv[e]) - sr[e] * KS[m][e];
    }
    SubstFrags f;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
        const __bf16* an = (hl ? sm.AN_lo : sm.AN) + li * kKtLd + 8 * lq;
        f.d[hl][0] = lds_load4(an);
        f.d[hl][1] = lds_load4(an + 16 * kKtLd + 4);
        f.d[hl][2] = lds_load4(an + 32 * kKtLd + 32);
        f.d[hl][3] = lds_load4(an + 48 * kKtLd + 36);
        f.a10[hl] = lds_load4(an + 16 * kKtLd);
        f.a2x[hl] = lds_load8(an + 32 * kKtLd);
        f.a3x[hl] = lds_load8(an + 48 * kKtLd);
        f.a32[hl] = lds_load4(an + 48 * kKtLd + 32);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 Dl[4];
    bf16x4 Db[4], Dbl[4];
    delta_substitution_hl(R, f, Dl, Db, Dbl, [](int) {});
    BD[0] = cat4(Db[0], Db[1]);
    BD[1] = cat4(Db[2], Db[3]);
    BDl[0] = cat4(Dbl[0], Dbl[1]);
    BDl[1] = cat4(Dbl[2], Dbl[3]);
    f32x4 su[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) su[m] = *reinterpret_cast<const f32x4*>(&sm.tokS[3][16 * m + 4 * lq]);
    const float eC = expf(sm.gam[kC - 1]);
    bf16x8 BH[2], BL[2];
    split_hi_lo(su, Dl, BH, BL);
#pragma unroll
    for (int th = 0; th < 8; th += 4) {
        bf16x8 akt[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                akt[t][ks] = lds_load8(&sm.Kt[(16 * (th + t) + li) * kKtLd + 32 * ks + 8 * lq]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = S[th + t] * eC;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                acc = mfma16(akt[t][ks], BH[ks], acc);
                acc = mfma16(akt[t][ks], BL[ks], acc);
            }
            S[th + t] = acc;
        }
    }
}

// ---- B2: O = Gamma n_q (Q S0) + P Delta, staged (bf16) into the chunk's Q
// buffer, which no wave reads any more
template <bool PRECISE, class SM>
__device__ __forceinline__ void phase_out(SM& sm, int buf, const f32x4 QS[4], const bf16x8 BD[2], const bf16x8 BDl[2],
                                          int wave, int li, int lq) {
    constexpr int VLd = SM::VLd;
    const int cw = 16 * wave + li;
    __bf16* Os = sm.Qs[buf];
    f32x4 so[4];
    bf16x8 pa[6];
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        so[m] = *reinterpret_cast<const f32x4*>(&sm.tokS[2][16 * m + 4 * lq]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) pa[i++] = lds_load8(&sm.Ps[(16 * m + li) * kKtLd + 32 * ks + 8 * lq]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        f32x4 acc = so[m] * QS[m];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) {
                acc = mfma16(pa[i], BD[ks], acc);
                if constexpr (PRECISE) {
                    const bf16x8 pl = lds_load8(&sm.Ps_lo[(16 * m + li) * kKtLd + 32 * ks + 8 * lq]);
                    acc = mfma16(pl, BD[ks], acc);
                    acc = mfma16(pa[i], BDl[ks], acc);
                }
                ++i;
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) Os[(16 * m + 4 * lq + e) * VLd + cw] = __bf16(acc[e]);
    }
}

// ---- C: O rows -> HBM (16-byte stores); checkpoint slot when the chunk end
// is a multiple of the checkpoint interval
template <int NW, class SM>
__device__ __forceinline__ void phase_store(const PrefillParams& p, SM& sm, const Ctx& cx, int buf,
                                            const f32x4 S[8], int64_t kc, int64_t s_base, bool owns_qk_tail,
                                            int tid) {
    constexpr int NT = 64 * NW;
    constexpr int N = 16 * NW;
    constexpr int VLd = SM::VLd;
    constexpr int NCH = SM::NCH;
    const int lane = tid % 64, lq = lane / 16;
    const int64_t local0 = kc * kC - cx.sp;
    const __bf16* Os = sm.Qs[buf];
    constexpr int V8 = N / 8;
    uint16_t* out = static_cast<uint16_t*>(p.out);
    for (int e = tid; e < kC * V8; e += NT) {
        const int tau = e / V8, c8 = e % V8;
        const int64_t t = local0 + tau;
        if (t >= 0 && t < cx.L)
            *reinterpret_cast<uint4*>(out + (((int64_t)cx.b * cx.L + t) * p.num_v_heads + cx.h) * kD + cx.zcol0 + 8 * c8) =
                *reinterpret_cast<const uint4*>(&Os[tau * VLd + 8 * c8]);
    }
    const int64_t pe = (kc + 1) * kC;   // absolute end of this chunk
    if (p.ckpt_interval > 0 && pe % p.ckpt_interval == 0 && pe <= cx.sp + cx.L) {
        char* slot = p.ckpt_buf + (uint64_t)(pe / p.ckpt_interval - 1) * p.slot_bytes;
        float* rec = reinterpret_cast<float*>(slot + p.conv_slot_bytes);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[s_base + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
        uint16_t* ctail = reinterpret_cast<uint16_t*>(slot);
        for (int ch = tid; ch < NCH; ch += NT)
            if (ch >= 2 * kD || owns_qk_tail)
                write_tail(p, cx.b, pe - cx.sp, global_channel(ch, cx.kh, cx.h, cx.zcol0, p.num_k_heads), ctail);
    }
}

template <int NW, bool PRECISE>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(PrefillParams p) {
    constexpr int NT = 64 * NW;
    constexpr int N = 16 * NW;
    constexpr int S_SPLIT = kD / N;
    using SM = Smem<NW, PRECISE>;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS of one workgroup");
    constexpr int NCH = SM::NCH;
    static_assert(NCH % 4 == 0, "channel groups of 4");
    __shared__ SM sm;

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int li = lane % 16, lq = lane / 16;

    // ---- workgroup -> (b, key head, member).  The r*S_SPLIT workgroups of one
    // (b, key head) read the same q/k rows; give them one blockIdx % 8 so that
    // the round-robin dispatch puts them on one XCD and its L2.
    const int r = p.num_v_heads / p.num_k_heads;
    const int M = r * S_SPLIT;
    const int NG = p.batch * p.num_k_heads;
    const int bid = blockIdx.x;
    const int grp = (bid / 8 / M) * 8 + bid % 8;
    const int mem = (bid / 8) % M;
    if (grp >= NG) return;
    Ctx cx;
    cx.b = grp / p.num_k_heads;
    cx.kh = grp % p.num_k_heads;
    cx.h = cx.kh * r + mem / S_SPLIT;
    cx.zcol0 = (mem % S_SPLIT) * N;
    cx.L = p.seq_len;
    cx.sp = p.start_pos;
    cx.neg_A = -expf(p.A_log[cx.h]);
    cx.dt_h = p.dt_bias[cx.h];
    const bool owns_qk_tail = (mem == 0);

    // ---- one-time set-up: zero the upper tiles of P, conv taps -> LDS
    for (int e = tid; e < 6 * 256; e += NT) {
        const int t6 = e / 256, rr = (e / 16) % 16, cc = e % 16;
        const int m = t6 < 3 ? 0 : (t6 < 5 ? 1 : 2);
        const int pp = t6 < 3 ? t6 + 1 : (t6 < 5 ? t6 - 1 : 3);
        sm.Ps[(16 * m + rr) * kKtLd + pos(16 * pp + cc)] = __bf16(0.f);
        if constexpr (PRECISE) sm.Ps_lo[(16 * m + rr) * kKtLd + pos(16 * pp + cc)] = __bf16(0.f);
    }
    for (int e = tid; e < NCH * 4; e += NT) {
        // taps stored [tap][channel] so that four channels of one tap are one
        // conflict-free 16-byte read
        const int ch = e % NCH, j = e / NCH;
        const int64_t gc = global_channel(ch, cx.kh, cx.h, cx.zcol0, p.num_k_heads);
        sm.Ws[e] = bf16_bits_to_f32(static_cast<const uint16_t*>(p.conv_w)[gc * 4 + j]);
    }

    // ---- the state slice of this wave: S[16t + 4lq + e][zcol0 + 16 wave + li]
    const int64_t s_base = ((int64_t)cx.b * p.num_v_heads + cx.h) * kD * kD + cx.zcol0 + 16 * wave + li;
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[t][e] = p.rec_in ? p.rec_in[s_base + (int64_t)(16 * t + 4 * lq + e) * kD] : 0.f;

    const int64_t k_first = cx.sp / kC;
    const int64_t k_end = cx.L > 0 ? (cx.sp + cx.L - 1) / kC + 1 : k_first;
    __syncthreads();

    // ---- prologue: the S-independent work of the first chunk
    if (k_first < k_end) {
        const int64_t local0 = k_first * kC - cx.sp;
        phase_front<NW>(p, sm, cx, 0, local0, tid);
        __syncthreads();
        phase_rows<NW>(p, sm, cx, 0, 1, local0, tid);
        __syncthreads();
        phase_masks<NW, PRECISE>(sm, 0, 1, tid);
        __syncthreads();
        if (wave == 0) diag_solve<false, PRECISE>(sm, lane);
        __syncthreads();
    }

    // ---- software pipeline over chunks: the state phase of chunk kc runs
    // next to the S-independent work of chunk kc + 1 (other buffer).  Within
    // the first stage half the waves do the state products first and half the
    // front end first, so each SIMD pairs MFMA/LDS work with VALU work.
    for (int64_t kc = k_first; kc < k_end; ++kc) {
        const int buf = (int)((kc - k_first) & 1), nbuf = buf ^ 1;
        const bool next = kc + 1 < k_end;
        const int64_t nlocal0 = (kc + 1) * kC - cx.sp;
        f32x4 QS[4];
        bf16x8 BD[2], BDl[2];
        auto state = [&] {
            if constexpr (PRECISE) phase_state_hl(sm, buf, S, QS, BD, BDl, wave, li, lq);
            else phase_state(sm, buf, S, QS, BD, BDl, wave, li, lq);
        };
        if (wave < NW / 2 || !next) {
            state();
            if (next) phase_front<NW>(p, sm, cx, nbuf, nlocal0, tid);
        } else {
            phase_front<NW>(p, sm, cx, nbuf, nlocal0, tid);
            state();
        }
        __syncthreads();
        phase_out<PRECISE>(sm, buf, QS, BD, BDl, wave, li, lq);
        if (next) phase_rows<NW>(p, sm, cx, nbuf, buf, nlocal0, tid);
        __syncthreads();
        phase_store<NW>(p, sm, cx, buf, S, kc, s_base, owns_qk_tail, tid);
        if (next) phase_masks<NW, PRECISE>(sm, nbuf, buf, tid);
        __syncthreads();
        if (next) {
            if (wave == 0) diag_solve<false, PRECISE>(sm, lane);
            __syncthreads();
        }
    }

    // ---- final state and conv tail
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.rec_out[s_base + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
    for (int ch = tid; ch < NCH; ch += NT)
        if (ch >= 2 * kD || owns_qk_tail)
            write_tail(p, cx.b, cx.L, global_channel(ch, cx.kh, cx.h, cx.zcol0, p.num_k_heads),
                       static_cast<uint16_t*>(p.conv_out));
}

template <int NW, bool PRECISE = false>
hipError_t launch_nw(const PrefillParams& p, hipStream_t stream) {
    const int s_split = kD / (16 * NW);
    const int r = p.num_v_heads / p.num_k_heads;
    const int ng = p.batch * p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * s_split;
    hipLaunchKernelGGL((prefill_kernel<NW, PRECISE>), dim3(blocks), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int head_k_dim, int head_v_dim, int io_dtype, int conv_kernel, int chunk) {
    return head_k_dim == kD && head_v_dim == kD && io_dtype == GDN_BF16 && conv_kernel == 4 &&
           chunk == kC;
}

// Columns of S per workgroup.  One workgroup per (b, head) with all 128
// columns (8 waves) is fastest on every measured workload, including the
// 48-chain 16K prefill; 2 and 4 waves remain selectable for experiments
// through GDN_PREFILL_WAVES.
int prefill_waves() {
    if (const char* env = getenv("GDN_PREFILL_WAVES")) {
        const int v = atoi(env);
        if (v == 2 || v == 4 || v == 8) return v;
    }
    return 8;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    // the precise mode's lo parts of P and AN do not fit beside the 8-wave
    // layout: 4 waves (64 state columns) per workgroup
    if (p.precise) return launch_nw<4, true>(p, stream);
    switch (prefill_waves()) {
        case 8: return launch_nw<8>(p, stream);
        case 4: return launch_nw<4>(p, stream);
        default: return launch_nw<2>(p, stream);
    }
}

}  // namespace gdn
