// gdn_chunk_common.h -- device pieces shared by the chunked-prefill kernels
// (the fused single-pass kernel and the two-pass chunk-prep / state kernels).
//
// The rule computed is the gated delta rule of the cortex commit page
// "feat(stage-8c): linear-attention layer (Qwen3-Next GatedDeltaNet)"
// ("Block", "Discretisation", "Delta rule") in chunks of C = 64 tokens
// ("Performance note").  Within a chunk with rows r, incoming state S0,
// gamma = inclusive cumsum of g and Gamma = exp(gamma):
//   A[r,i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)      for i < r
//   T      = (I + A)^-1                       ("direct solve", the stable
//            variant of the Qwen3.6-27B PR, "Known limitations and follow-ups")
//   Delta  = T (diag(beta) V - diag(beta Gamma) K S0)
//   O      = diag(Gamma) Q S0 + (M .* Q K^T) Delta,  M[r,i] = exp(gamma_r - gamma_i), i <= r
//   S_C    = exp(gamma_C) S0 + (diag(exp(gamma_C - gamma)) K)^T Delta
// with q, k the unit-norm vectors.  They are kept as raw bf16 conv outputs
// (exact MFMA operands) and the norms are folded into fp32 row scales.
// Chunk boundaries sit at absolute multiples of 64; rows of a partial chunk
// outside the call have g = 0, beta = 0, q = k = v = 0, which leaves the
// result unchanged.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (lane l, i = l % 16,
// q = l / 16): A row i and B column i each hold 8 reduction slots of group
// q; D holds rows 4q..4q+3 of column i.  The reduction index a slot stands
// for only has to agree between A and B, so the accumulator layout of one
// product is reused as the B operand of the next without data movement.
#pragma once

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace chunked {

constexpr int kC = 64;              // chunk
constexpr int kD = 128;             // d_k = d_v
constexpr int kKsLd = kD + 8;       // bf16 row stride of Q, K in LDS (rows = tokens)
constexpr int kKtLd = kC + 8;       // bf16 row stride of K^T, P, AN in LDS
constexpr int kXLd = 17;            // fp32 row stride of the transposed diagonal blocks

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 (16 bytes) from LDS
__device__ __forceinline__ bf16x8 lds_load8(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_load4(const __bf16* p) {
    return *reinterpret_cast<const bf16x4*>(p);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b) {
    const f32x8 v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ f32x8 to_f32x8(bf16x8 v) { return __builtin_convertvector(v, f32x8); }

// bf16 hi + lo of fp32 values: hi = RNE(x), lo = RNE(x - hi); hi + lo carries
// about 16 significant bits (the operands of the precise mode)
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
    hi = __bf16(x);
    lo = __bf16(x - float(hi));
}

__device__ __forceinline__ void split_bf16x4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    hi = __builtin_convertvector(x, bf16x4);
    const f32x4 back = __builtin_convertvector(hi, f32x4);
    lo = __builtin_convertvector(x - back, bf16x4);
}

// Column order inside Q, K (d_k columns) and K^T, P, AN (token columns).  An
// index x = 32a + 16h + 4q + e is stored at 32a + 8q + 4h + e, so the eight
// reduction slots that lane group q of v_mfma_f32_16x16x32_bf16 needs for
// k-step a (indices 32a + 4q + {0..3} and 32a + 16 + 4q + {0..3}, the order
// in which an accumulator tile is reused as a B operand) are one contiguous
// 16-byte run, and runs of four consecutive indices stay contiguous.
__device__ __forceinline__ int pos(int x) {
    return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
}

// lower 16x16 tile pairs (m, p), p <= m, in a fixed order
__device__ __forceinline__ void tile_pair(int idx, int& m, int& p) {
    m = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
    p = idx - (m * (m + 1)) / 2;
}

__device__ __forceinline__ void unpack_bf16x4(uint2 raw, float x[4]) {
    x[0] = bf16_bits_to_f32(raw.x & 0xffffu);
    x[1] = bf16_bits_to_f32(raw.x >> 16);
    x[2] = bf16_bits_to_f32(raw.y & 0xffffu);
    x[3] = bf16_bits_to_f32(raw.y >> 16);
}

// Pre-conv inputs of channels gc..gc+3 at call-local token t < 0: the
// carried conv state for t >= -3 (zeros for a new request), else zeros.
__device__ __forceinline__ void load_x4_state(const PrefillParams& p, int b, int64_t t, int64_t gc,
                                              float x[4]) {
    const uint16_t* cs = static_cast<const uint16_t*>(p.conv_in);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        x[i] = (cs && t >= -3) ? bf16_bits_to_f32(cs[((int64_t)b * p.conv_dim + gc + i) * 3 + (3 + t)]) : 0.f;
}

// Copy the conv tail that ends just before call-local token `end` (the last
// three pre-conv inputs) for channel gc of sequence b into dst[b][gc][0..2].
__device__ __forceinline__ void write_tail(const PrefillParams& p, int b, int64_t end, int64_t gc,
                                           uint16_t* dst) {
    const uint16_t* qkv = static_cast<const uint16_t*>(p.qkv);
    const uint16_t* cs = static_cast<const uint16_t*>(p.conv_in);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t t = end - 3 + j;
        uint16_t v;
        if (t >= 0) v = qkv[((int64_t)b * p.seq_len + t) * p.conv_dim + gc];
        else v = cs ? cs[((int64_t)b * p.conv_dim + gc) * 3 + (3 + t)] : uint16_t(0);
        dst[((int64_t)b * p.conv_dim + gc) * 3 + j] = v;
    }
}

// Front end of one work item: channels gc..gc+3 of sequence b at the TT
// chunk rows tau0..tau0+TT-1 (call-local tokens local0 + tau): depthwise
// causal conv with taps w[j][i] (tap j of channel i; tap 3 multiplies the
// current token) in fp32, SiLU, bf16.  raw[k] holds the pre-conv inputs of
// the four channels at row tau0 - 3 + k.  conv_load issues the TT + 3 8-byte
// row loads together, so a caller can start the next item's loads before
// computing this one.  INTERIOR: every row lies inside the call.  Otherwise
// row indices are clamped into the call, rows before it are replaced by the
// carried conv state and rows outside it produce zeros.
template <bool INTERIOR, int TT = 8>
__device__ __forceinline__ void conv_load(const PrefillParams& p, int b, int64_t gc, int64_t local0, int tau0,
                                          uint2 raw[TT + 3]) {
    const int64_t L = p.seq_len;
    const int64_t t_first = local0 + tau0 - 3;
    if (INTERIOR) {
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) + ((int64_t)b * L + t_first) * p.conv_dim + gc;
        const int cd = (int)p.conv_dim;
#pragma unroll
        for (int j = 0; j < TT + 3; ++j) raw[j] = *reinterpret_cast<const uint2*>(src + j * cd);
    } else {
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) + (int64_t)b * L * p.conv_dim + gc;
#pragma unroll
        for (int j = 0; j < TT + 3; ++j) {
            const int64_t tc = min(max(t_first + j, (int64_t)0), L - 1);
            raw[j] = *reinterpret_cast<const uint2*>(src + tc * p.conv_dim);
        }
    }
}

template <bool INTERIOR, int TT = 8>
__device__ __forceinline__ void conv_compute(const PrefillParams& p, int b, int64_t gc, int64_t local0, int tau0,
                                             const float w[4][4], const uint2 raw[TT + 3], bf16x4 ub[TT]) {
    const int64_t L = p.seq_len;
    const int64_t t_first = local0 + tau0 - 3;
    float hist[3][4];
#pragma unroll
    for (int j = 0; j < 3; ++j) unpack_bf16x4(raw[j], hist[j]);
    if (!INTERIOR && t_first < 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (t_first + j < 0) load_x4_state(p, b, t_first + j, gc, hist[j]);
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t t = local0 + tau0 + tt;
        float x[4];
        unpack_bf16x4(raw[3 + tt], x);
        if (!INTERIOR && t < 0) load_x4_state(p, b, t, gc, x);
        const bool valid = INTERIOR || (t >= 0 && t < L);
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y = fmaf(w[3][i], x[i], fmaf(w[2][i], hist[2][i], fmaf(w[1][i], hist[1][i], w[0][i] * hist[0][i])));
            u[i] = valid ? silu_fast(y) : 0.f;
            hist[0][i] = hist[1][i];
            hist[1][i] = hist[2][i];
            hist[2][i] = x[i];
        }
        ub[tt] = __builtin_convertvector(u, bf16x4);
    }
}

template <bool INTERIOR>
__device__ __forceinline__ void conv_item(const PrefillParams& p, int b, int64_t gc, int64_t local0, int tau0,
                                          const float w[4][4], bf16x4 ub[8]) {
    uint2 raw[11];
    conv_load<INTERIOR>(p, b, gc, local0, tau0, raw);
    conv_compute<INTERIOR>(p, b, gc, local0, tau0, w, raw, ub);
}

// Gates of value head h for the 64 chunk rows (one full wave, lane = row):
// g = -exp(A_log) softplus(a + dt_bias) (neg_A = -exp(A_log)), beta =
// sigmoid(b), zeros for rows outside the call; gam = inclusive scan of g.
__device__ __forceinline__ void gates_scan(const PrefillParams& p, int b, int h, float neg_A, float dt_h,
                                           int64_t local0, int lane, float* gam, float* beta) {
    const int64_t t = local0 + lane;
    const bool valid = t >= 0 && t < p.seq_len;
    float gv = 0.f, bv = 0.f;
    if (valid) {
        const int64_t gi = ((int64_t)b * p.seq_len + t) * p.num_v_heads + h;
        const float av = bf16_bits_to_f32(static_cast<const uint16_t*>(p.a)[gi]);
        const float bb = bf16_bits_to_f32(static_cast<const uint16_t*>(p.b)[gi]);
        gv = neg_A * softplus_f32(av + dt_h);
        bv = sigmoid_f32(bb);
    }
    float s = gv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(s, off, 64);
        if (lane >= off) s += o;
    }
    gam[lane] = s;
    beta[lane] = bv;
}

// 1 / sqrt(sum x^2 + eps) * scale over one 128-wide bf16 LDS row
__device__ __forceinline__ float row_inv_norm(const __bf16* row, float scale, float eps) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kD; c += 8) {
        const f32x8 v = to_f32x8(lds_load8(row + c));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(v[i], v[i], acc);
    }
    return scale / sqrtf(acc + eps);
}

// Raw tile ti of K K^T (ti < 10) or Q K^T (ti >= 10) on the lower 16x16 tile
// pair tile_pair(ti % 10): bf16 operands straight from LDS (row stride
// kKsLd), fp32 accumulate.
__device__ __forceinline__ f32x4 gram_tile(const __bf16* Ks, const __bf16* Qs, int ti, int li, int lq) {
    int m, pp;
    tile_pair(ti >= 10 ? ti - 10 : ti, m, pp);
    const __bf16* arow = (ti >= 10 ? Qs : Ks) + (16 * m + li) * kKsLd + 8 * lq;
    const __bf16* brow = Ks + (16 * pp + li) * kKsLd + 8 * lq;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16(lds_load8(arow + 32 * ks), lds_load8(brow + 32 * ks), acc);
    return acc;
}

// Decay masks and row/column scales of one lower tile pair (lane l of the
// accumulator layout: column 16 pp + l % 16, rows 16 m + 4 (l / 16) + e):
//   A[r,i] = beta_r n_k[r] n_k[i] exp(gamma_r - gamma_i) (K K^T)[r,i], i < r
//     -> -A (bf16) off the diagonal blocks, fp32 transposed on them
//   P[r,i] = n_q[r] n_k[i] exp(gamma_r - gamma_i) (Q K^T)[r,i], i <= r (bf16)
// SM provides gam, beta, nq, nk [64] and Ps, AN [64 x kKtLd], AdT; with
// PRECISE also Ps_lo, AN_lo, which take the bf16 lo parts of P and -A.
template <bool PRECISE = false, class SM>
__device__ __forceinline__ void mask_pair(SM& sm, int pi, f32x4 g, f32x4 qk, int l) {
    const int li = l % 16, lq = l / 16;
    int m, pp;
    tile_pair(pi, m, pp);
    const int ii = 16 * pp + li, r0 = 16 * m + 4 * lq;
    const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.gam[r0]);
    const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[r0]);
    const f32x4 kr = *reinterpret_cast<const f32x4*>(&sm.nk[r0]);
    const f32x4 qr = *reinterpret_cast<const f32x4*>(&sm.nq[r0]);
    const float gi = sm.gam[ii], nki = sm.nk[ii];
    const int pii = pos(ii);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = r0 + e;
        const float dec = ii <= rr ? __expf(gr[e] - gi) * nki : 0.f;
        const float av = ii < rr ? br[e] * kr[e] * dec * g[e] : 0.f;
        if constexpr (PRECISE) {
            split_bf16(qr[e] * dec * qk[e], sm.Ps[rr * kKtLd + pii], sm.Ps_lo[rr * kKtLd + pii]);
            if (m == pp) sm.AdT[(m * 16 + li) * kXLd + 4 * lq + e] = av;
            else split_bf16(-av, sm.AN[rr * kKtLd + pii], sm.AN_lo[rr * kKtLd + pii]);
        } else {
            sm.Ps[rr * kKtLd + pii] = __bf16(qr[e] * dec * qk[e]);
            if (m == pp) sm.AdT[(m * 16 + li) * kXLd + 4 * lq + e] = av;
            else sm.AN[rr * kKtLd + pii] = __bf16(-av);
        }
    }
}

// Per-row scales of the state phase for row r = lane (one wave):
//   beta | beta Gamma n_k | Gamma n_q | exp(gamma_C - gamma) n_k
template <class SM>
__device__ __forceinline__ void row_scales(SM& sm, int r) {
    const float gl = sm.gam[r], gC = sm.gam[kC - 1];
    const float e = expf(gl), nkv = sm.nk[r], bv = sm.beta[r];
    sm.tokS[0][r] = bv;
    sm.tokS[1][r] = bv * e * nkv;
    sm.tokS[2][r] = e * sm.nq[r];
    sm.tokS[3][r] = expf(gC - gl) * nkv;
}

// Inverses of the four diagonal blocks, (I + A_mm)^-1 = I + N_mm, by
// substitution (one wave, lane = (block m, column c)); N_mm goes to the
// diagonal blocks of AN.  The off-diagonal coupling is applied in the state
// phase by blocked forward substitution, so no other part of (I + A)^-1 is
// formed.  Right-looking: once x[i] is final its contribution is subtracted
// from every later row (column i of A_mm is row i of AdT), so the dependent
// chain is one FMA per row.  Column i + 1 is loaded while column i is
// applied.  BOUNDED ties the address of column i + 1 to x[i] through an empty
// asm, so the compiler cannot hoist all 120 loads to the top (which costs
// ~200 registers); without it the loads are scheduled freely.
template <bool BOUNDED, bool PRECISE = false, class SM>
__device__ __forceinline__ void diag_solve(SM& sm, int lane) {
    const int m = lane / 16, c = lane % 16;
    const float* At = sm.AdT + m * 16 * kXLd;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = rr == c ? 1.f : 0.f;
    float col[2][16];   // column i of A_mm, loaded one step ahead
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) col[0][rr] = At[rr];
    int dep = 0;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        const float xi = x[i];
        if (BOUNDED) asm volatile("" : "+v"(dep) : "v"(xi));
        if (i + 1 < 15) {
#pragma unroll
            for (int rr = i + 2; rr < 16; ++rr) col[(i + 1) & 1][rr] = At[dep + (i + 1) * kXLd + rr];
        }
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr) x[rr] = fmaf(-col[i & 1][rr], xi, x[rr]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int o = (16 * m + rr) * kKtLd + pos(16 * m + c);
        if constexpr (PRECISE) split_bf16(rr == c ? 0.f : x[rr], sm.AN[o], sm.AN_lo[o]);
        else sm.AN[o] = __bf16(rr == c ? 0.f : x[rr]);
    }
}

// fp32 16x16 product on v_mfma_f32_16x16x4_f32 in the accumulator layout:
// lane l = (n = l % 16, q = l / 16), element e holds M[4q + e][n].  Step s
// takes reduction index 4q + s, so the A operand is element s of the left
// factor's transpose and the B operand element s of the right factor.
__device__ __forceinline__ f32x4 mm16_f32(f32x4 leftT, f32x4 right, f32x4 acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(leftT[s], right[s], acc, 0, 0, 0);
    return acc;
}

// The same diagonal-block inverse as diag_solve, by the faster form the
// Qwen3.6-27B PR names beside the direct solve ("Known limitations and
// follow-ups"): with X = -A_mm strictly lower triangular, X^16 = 0 and
//   (I + A_mm)^-1 = sum_{k<16} X^k = (I + X)(I + X^2)(I + X^4)(I + X^8),
// four squarings and three multiply-adds instead of a 15-step dependent
// chain.  One wave per block m.  Every factor is a polynomial in X, so the
// factors commute; each is kept with its transpose for use as a left
// factor.  Exact in exact arithmetic; in fp32 the powers X^k can be far
// larger than the inverse (keys that nearly coincide, beta near 1, slow
// decay), and their rounding then survives the cancellation.
template <bool PRECISE = false, class SM>
__device__ __forceinline__ void diag_neumann(SM& sm, int m, int lane) {
    const int n = lane % 16, q = lane / 16;
    const float* At = sm.AdT + m * 16 * kXLd;   // At[i * kXLd + r] = A_mm[r][i]
    f32x4 X, XT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        X[e] = -At[n * kXLd + 4 * q + e];
        XT[e] = -At[(4 * q + e) * kXLd + n];
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 X2 = mm16_f32(XT, X, z), X2T = mm16_f32(X, XT, z);
    const f32x4 X4 = mm16_f32(X2T, X2, z), X4T = mm16_f32(X2, X2T, z);
    f32x4 R = mm16_f32(X4T, X4, z);
#pragma unroll
    for (int e = 0; e < 4; ++e) R[e] += 4 * q + e == n ? 1.f : 0.f;
    R = mm16_f32(X4T, R, R);
    R = mm16_f32(X2T, R, R);
    R = mm16_f32(XT, R, R);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int o = (16 * m + 4 * q + e) * kKtLd + pos(16 * m + n);
        if constexpr (PRECISE) split_bf16(4 * q + e > n ? R[e] : 0.f, sm.AN[o], sm.AN_lo[o]);
        else sm.AN[o] = __bf16(4 * q + e > n ? R[e] : 0.f);
    }
}

// Blocked forward substitution for Delta of one wave's 16 columns:
// (I + A) Delta = R over the four 16-row blocks, Y_m = R_m - sum_{k<m} A_mk
// Delta_k, Delta_m = Y_m + N_mm Y_m.  The fp32 accumulator carries R and Y
// exactly; only the coupling terms see bf16 operands.  d[m] are this lane's
// A-operand slots of N_mm; a10, a2x, a3x, a32 those of -A_10, -[A_20 A_21],
// -[A_30 A_31], -A_32.
// hook(s), s = 0..7, runs right after the MFMAs of step s (two per block), so
// a caller can put independent work into the latency of this dependent chain.
template <class Hook>
__device__ __forceinline__ void delta_substitution(const f32x4 R[4], const bf16x4 d[4], bf16x4 a10, bf16x8 a2x,
                                                   bf16x8 a3x, bf16x4 a32, f32x4 Dl[4], bf16x4 Db[4], Hook&& hook) {
    const bf16x4 z4 = {__bf16(0.f), __bf16(0.f), __bf16(0.f), __bf16(0.f)};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 y = R[m];
        if (m == 1) y = mfma16(cat4(a10, z4), cat4(Db[0], z4), y);
        if (m == 2) y = mfma16(a2x, cat4(Db[0], Db[1]), y);
        if (m == 3) {
            y = mfma16(a3x, cat4(Db[0], Db[1]), y);
            y = mfma16(cat4(a32, z4), cat4(Db[2], z4), y);
        }
        hook(2 * m);
        const bf16x4 yb = __builtin_convertvector(y, bf16x4);
        Dl[m] = mfma16(cat4(d[m], z4), cat4(yb, z4), y);
        hook(2 * m + 1);
        Db[m] = __builtin_convertvector(Dl[m], bf16x4);
    }
}

__device__ __forceinline__ void delta_substitution(const f32x4 R[4], const bf16x4 d[4], bf16x4 a10, bf16x8 a2x,
                                                   bf16x8 a3x, bf16x4 a32, f32x4 Dl[4], bf16x4 Db[4]) {
    delta_substitution(R, d, a10, a2x, a3x, a32, Dl, Db, [](int) {});
}

// The same substitution with every coupling and diagonal product on bf16 hi
// + lo operands (X_hi Y_hi + X_lo Y_hi + X_hi Y_lo, the lo x lo term below
// fp32 rounding dropped): the precise mode.  The fragments come as {hi, lo}
// pairs; Db, Dbl are the hi and lo parts of Delta for the later products.
struct SubstFrags {
    bf16x4 d[2][4];
    bf16x4 a10[2];
    bf16x8 a2x[2], a3x[2];
    bf16x4 a32[2];
};

template <class Hook>
__device__ __forceinline__ void delta_substitution_hl(const f32x4 R[4], const SubstFrags& f, f32x4 Dl[4],
                                                      bf16x4 Db[4], bf16x4 Dbl[4], Hook&& hook) {
    const bf16x4 z4 = {__bf16(0.f), __bf16(0.f), __bf16(0.f), __bf16(0.f)};
    auto mm3 = [&](bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 acc) {
        acc = mfma16(ah, bh, acc);
        acc = mfma16(al, bh, acc);
        return mfma16(ah, bl, acc);
    };
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 y = R[m];
        if (m == 1)
            y = mm3(cat4(f.a10[0], z4), cat4(f.a10[1], z4), cat4(Db[0], z4), cat4(Dbl[0], z4), y);
        if (m == 2) y = mm3(f.a2x[0], f.a2x[1], cat4(Db[0], Db[1]), cat4(Dbl[0], Dbl[1]), y);
        if (m == 3) {
            y = mm3(f.a3x[0], f.a3x[1], cat4(Db[0], Db[1]), cat4(Dbl[0], Dbl[1]), y);
            y = mm3(cat4(f.a32[0], z4), cat4(f.a32[1], z4), cat4(Db[2], z4), cat4(Dbl[2], z4), y);
        }
        hook(2 * m);
        bf16x4 yh, yl;
        split_bf16x4(y, yh, yl);
        Dl[m] = mm3(cat4(f.d[0][m], z4), cat4(f.d[1][m], z4), cat4(yh, z4), cat4(yl, z4), y);
        hook(2 * m + 1);
        split_bf16x4(Dl[m], Db[m], Dbl[m]);
    }
}

// Delta' = exp(gamma_C - gamma) n_k Delta as bf16 hi + lo B operands of the
// state update (two k-steps of 32 tokens)
__device__ __forceinline__ void split_hi_lo(const f32x4 su[4], const f32x4 Dl[4], bf16x8 BH[2], bf16x8 BL[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 q0 = su[2 * ks] * Dl[2 * ks], q1 = su[2 * ks + 1] * Dl[2 * ks + 1];
        BH[ks] = to_bf16x8(q0, q1);
        const f32x8 back = to_f32x8(BH[ks]);
        const f32x4 l0 = {q0[0] - back[0], q0[1] - back[1], q0[2] - back[2], q0[3] - back[3]};
        const f32x4 l1 = {q1[0] - back[4], q1[1] - back[5], q1[2] - back[6], q1[3] - back[7]};
        BL[ks] = to_bf16x8(l0, l1);
    }
}

}  // namespace chunked
}  // namespace gdn
