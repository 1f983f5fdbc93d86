// gdn_prefill.hip -- fused chunked prefill of the Gated DeltaNet core (gfx950).
//
// What is computed: the per-token gated delta rule of the cortex commit page
// "feat(stage-8c): linear-attention layer (Qwen3-Next GatedDeltaNet)"
// ("Block", "Discretisation", "Delta rule"), evaluated in chunks of C = 64
// tokens ("Performance note").  Within a chunk with rows r, incoming state
// S0, gamma = inclusive cumsum of g and Gamma = exp(gamma), the rule unrolls
// to (derivation in the design notes; the pages only name the method):
//   A[r,i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)      for i < r
//   T      = (I + A)^-1                       ("direct solve", the stable
//            variant of the Qwen3.6-27B PR, "Known limitations and follow-ups")
//   Delta  = T (diag(beta) V - diag(beta Gamma) K S0)
//   O      = diag(Gamma) Q S0 + (M .* Q K^T) Delta,  M[r,i] = exp(gamma_r - gamma_i), i <= r
//   S_C    = exp(gamma_C) S0 + (diag(exp(gamma_C - gamma)) K)^T Delta
// with q, k the unit-norm vectors.  Here they are kept as raw bf16 conv
// outputs (exact MFMA operands) and the norms are folded into fp32 row scales.
//
// One workgroup owns (sequence b, value head h, a slice of N = 16*NW state
// columns); wave w owns 16 columns and keeps its 128 x 16 fp32 slice of S in
// MFMA accumulator registers for the whole call.  Per chunk:
//   A1  front end: raw qkv (+3-token halo, or the carried conv state) ->
//       depthwise conv (fp32) -> SiLU -> bf16 -> LDS (Q, K, K^T, V)
//   A2  gates g, beta (fp32), inclusive scan of g; L2 norms of q and k
//   A3  K K^T and Q K^T lower 16x16 tiles on MFMA (bf16 in, fp32 out),
//       decay masks -> A (fp32) and P (bf16)
//   A4  T = (I + A)^-1 by blocked forward substitution in fp32 (16x16
//       diagonal blocks by substitution, off-diagonal blocks by products)
//   B   per wave, on MFMA: K S0, Q S0 (S0 as bf16), R, Delta = R + (T-I) R,
//       O, and S <- exp(gamma_C) S + K^T Delta' with Delta' split into bf16
//       hi + lo (two MFMAs): the product that builds the state carries ~16
//       significant bits, everything else bf16 operands with fp32 accumulate.
//   C   O rows -> HBM (16-byte stores); checkpoint slots when the chunk end is
//       a multiple of the checkpoint interval.
// Chunk boundaries sit at absolute multiples of 64, so a partial first or
// last chunk is padded with rows that have g = 0, beta = 0, q = k = v = 0,
// which leaves the rule's result unchanged.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout used throughout (lane l, i =
// l % 16, q = l / 16): A row i and B column i each hold 8 reduction slots of
// group q; D holds rows 4q..4q+3 of column i.  The reduction index a slot
// stands for only has to agree between A and B, so the accumulator layout of
// one product is reused as the B operand of the next without data movement.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kC = 64;              // chunk
constexpr int kD = 128;             // d_k = d_v
constexpr int kKsLd = kD + 8;       // bf16 row stride of Q, K (rows = tokens)
constexpr int kKtLd = kC + 8;       // bf16 row stride of K^T, P, AN
constexpr int kXLd = 17;
constexpr int kVtLd = kC + 12;      // bf16 row stride of V^T

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

// two runs of 4 bf16 (8 bytes each): slots 0-3 from p, 4-7 from p + 16
__device__ __forceinline__ bf16x8 lds_load4x2(const __bf16* p) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

template <int NW>
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
    static_assert(kC * VLd <= kC * kKsLd, "output staging fits a Q buffer");
    static_assert(NW != 8 || (10 * 64 * 16 <= kC * kKsLd * 2 && 10 * 64 * 16 <= N * kVtLd * 2),
                  "raw Gram tiles fit the dead K and V^T buffers");
};

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

// Global channel of the WG's channel index ch (q: 0..127, k: 128..255, v: 256..)
__device__ __forceinline__ int64_t global_channel(int ch, int kh, int h, int zcol0, int Hk) {
    if (ch < kD) return (int64_t)kh * kD + ch;
    if (ch < 2 * kD) return (int64_t)Hk * kD + (int64_t)kh * kD + (ch - kD);
    return 2 * (int64_t)Hk * kD + (int64_t)h * kD + zcol0 + (ch - 2 * kD);
}

__device__ __forceinline__ void unpack_bf16x4(uint2 raw, float x[4]) {
    x[0] = bf16_bits_to_f32(raw.x & 0xffffu);
    x[1] = bf16_bits_to_f32(raw.x >> 16);
    x[2] = bf16_bits_to_f32(raw.y & 0xffffu);
    x[3] = bf16_bits_to_f32(raw.y >> 16);
}

// SiLU with the hardware exp2 and reciprocal (about 2 ulp of fp32; the
// result is rounded to bf16 right after).
__device__ __forceinline__ float silu_fast(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
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

// Per-workgroup constants.
struct Ctx {
    int b, kh, h, zcol0;
    int64_t L, sp;
    float neg_A, dt_h;
};

constexpr int kTilesPerWave = 4;   // 20 Gram tiles over waves 3..7

// Raw tile ti of K K^T (ti < 10) or Q K^T (ti >= 10) on the lower 16x16 tile
// pair tile_pair(ti % 10): bf16 operands straight from LDS, fp32 accumulate.
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
template <int NW>
__device__ __forceinline__ void mask_pair(Smem<NW>& sm, int pi, f32x4 g, f32x4 qk, int l) {
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
        sm.Ps[rr * kKtLd + pii] = __bf16(qr[e] * dec * qk[e]);
        if (m == pp) sm.AdT[(m * 16 + li) * kXLd + 4 * lq + e] = av;
        else sm.AN[rr * kKtLd + pii] = __bf16(-av);
    }
}

// Per-row scales of the state phase for row r = lane (one wave):
//   beta | beta Gamma n_k | Gamma n_q | exp(gamma_C - gamma) n_k
template <int NW>
__device__ __forceinline__ void row_scales(Smem<NW>& sm, int r) {
    const float gl = sm.gam[r], gC = sm.gam[kC - 1];
    const float e = expf(gl), nkv = sm.nk[r], bv = sm.beta[r];
    sm.tokS[0][r] = bv;
    sm.tokS[1][r] = bv * e * nkv;
    sm.tokS[2][r] = e * sm.nq[r];
    sm.tokS[3][r] = expf(gC - gl) * nkv;
}

// Front end of one work item: 4 channels x 8 tokens of the chunk.  The
// eleven 8-byte row loads (3 halo rows + 8) are issued together.  INTERIOR:
// every row lies inside the call.  Otherwise row indices are clamped into the
// call, rows before it are replaced by the carried conv state and rows outside
// it produce zeros.
template <bool INTERIOR, int NW>
__device__ __forceinline__ void front_item(const PrefillParams& p, Smem<NW>& sm, const Ctx& cx, int buf,
                                           int64_t local0, int item) {
    constexpr int NCH = Smem<NW>::NCH;
    constexpr int CG4 = NCH / 4;
    const int64_t L = cx.L;
    const int cg = item % CG4, seg = item / CG4;
    const int ch0 = cg * 4;
    const int64_t gc = global_channel(ch0, cx.kh, cx.h, cx.zcol0, p.num_k_heads);
    const int tau0 = seg * 8;
    const int64_t t_first = local0 + tau0 - 3;
    uint2 raw[11];
    if (INTERIOR) {
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) +
                              ((int64_t)cx.b * L + t_first) * p.conv_dim + gc;
        const int cd = (int)p.conv_dim;
#pragma unroll
        for (int j = 0; j < 11; ++j) raw[j] = *reinterpret_cast<const uint2*>(src + j * cd);
    } else {
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) + (int64_t)cx.b * L * p.conv_dim + gc;
#pragma unroll
        for (int j = 0; j < 11; ++j) {
            const int64_t tc = min(max(t_first + j, (int64_t)0), L - 1);
            raw[j] = *reinterpret_cast<const uint2*>(src + tc * p.conv_dim);
        }
    }
    float w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(&sm.Ws[j * NCH + ch0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[j][i] = wv[i];
    }
    float hist[3][4];
#pragma unroll
    for (int j = 0; j < 3; ++j) unpack_bf16x4(raw[j], hist[j]);
    if (!INTERIOR && t_first < 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (t_first + j < 0) load_x4_state(p, cx.b, t_first + j, gc, hist[j]);
    }
    const bool is_v = ch0 >= 2 * kD;
    __bf16* dst0 = ch0 < kD ? &sm.Qs[buf][pos(ch0)] : &sm.Ks[buf][pos(ch0 - kD)];
    bf16x8 vcol[4];   // v channels: 8 tokens of each of the 4 channels, stored as V^T rows
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int tau = tau0 + tt;
        const int64_t t = local0 + tau;
        float x[4];
        unpack_bf16x4(raw[3 + tt], x);
        if (!INTERIOR && t < 0) load_x4_state(p, cx.b, t, gc, x);
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
        const bf16x4 ub = __builtin_convertvector(u, bf16x4);
        if (is_v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vcol[i][tt] = ub[i];
        } else {
            *reinterpret_cast<bf16x4*>(dst0 + tau * kKsLd) = ub;
        }
    }
    if (is_v) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<bf16x8*>(&sm.Vt[buf][(ch0 - 2 * kD + i) * kVtLd + tau0]) = vcol[i];
    }
}

// ---- A1: front end of a chunk into Q, K, V^T buffer `buf`
template <int NW>
__device__ __forceinline__ void phase_front(const PrefillParams& p, Smem<NW>& sm, const Ctx& cx, int buf,
                                            int64_t local0, int tid) {
    constexpr int NT = 64 * NW;
    constexpr int CG4 = Smem<NW>::NCH / 4;
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
template <int NW>
__device__ __forceinline__ void phase_rows(const PrefillParams& p, Smem<NW>& sm, const Ctx& cx, int buf,
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
            const int tau = job;
            const int64_t t = local0 + tau;
            const bool valid = t >= 0 && t < cx.L;
            float gv = 0.f, bv = 0.f;
            if (valid) {
                const int64_t gi = ((int64_t)cx.b * cx.L + t) * p.num_v_heads + cx.h;
                const float av = bf16_bits_to_f32(static_cast<const uint16_t*>(p.a)[gi]);
                const float bb = bf16_bits_to_f32(static_cast<const uint16_t*>(p.b)[gi]);
                gv = cx.neg_A * softplus_f32(av + cx.dt_h);
                bv = sigmoid_f32(bb);
            }
            float s = gv;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(s, off, 64);
                if (lane >= off) s += o;
            }
            sm.gam[tau] = s;
            sm.beta[tau] = bv;
        } else {
            const bool isq = job < 2 * kC;
            const int tau = job % kC;
            const __bf16* row = (isq ? Qs : Ks) + tau * kKsLd;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < kD; c += 8) {
                const f32x8 v = to_f32x8(lds_load8(row + c));
#pragma unroll
                for (int i = 0; i < 8; ++i) acc = fmaf(v[i], v[i], acc);
            }
            const float n = (isq ? p.q_scale : 1.0f) / sqrtf(acc + p.l2_eps);
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
template <int NW>
__device__ __forceinline__ void phase_masks(Smem<NW>& sm, int buf, int gbuf, int tid) {
    constexpr int NT = 64 * NW;
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, lq = lane / 16;
    if constexpr (NW == 8) {
        // job = (tile pair, lane): both the K K^T and the Q K^T tile of one
        // lower tile pair, 640 jobs over 512 threads, branch-free within a wave
        const f32x4* G = reinterpret_cast<const f32x4*>(sm.Ks[gbuf]);
        const f32x4* GQ = reinterpret_cast<const f32x4*>(sm.Vt[gbuf]);
        for (int j = tid; j < 10 * 64; j += NT) mask_pair(sm, j >> 6, G[j], GQ[j], j & 63);
        if (wave == NW - 1) row_scales(sm, lane);
    } else {
        if (wave == 0) row_scales(sm, lane);
        for (int pi = wave - 1; pi >= 0 && pi < 10; pi += NW - 1)
            mask_pair(sm, pi, gram_tile(sm.Ks[buf], sm.Qs[buf], pi, li, lq),
                      gram_tile(sm.Ks[buf], sm.Qs[buf], 10 + pi, li, lq), lane);
    }
}

// ---- A4: inverses of the four diagonal blocks, (I + A_mm)^-1 = I + N_mm, by
// substitution (one wave, lane = (block m, column c)).  The off-diagonal
// coupling is applied in the state phase by blocked forward substitution, so
// no other part of (I + A)^-1 is formed.
template <int NW>
__device__ __forceinline__ void phase_diag(Smem<NW>& sm, int lane) {
    // right-looking: once x[i] is final, subtract its contribution from every
    // later row (column i of A_mm is row i of AdT), so the dependent chain is
    // one FMA per row
    const int m = lane / 16, c = lane % 16;
    const float* At = sm.AdT + m * 16 * kXLd;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = rr == c ? 1.f : 0.f;
    float col[2][16];   // column i of A_mm, loaded one step ahead
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) col[0][rr] = At[rr];
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        if (i + 1 < 15) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) col[(i + 1) & 1][rr] = At[(i + 1) * kXLd + rr];
        }
        const float xi = x[i];
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr) x[rr] = fmaf(-col[i & 1][rr], xi, x[rr]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
        sm.AN[(16 * m + rr) * kKtLd + pos(16 * m + c)] = __bf16(rr == c ? 0.f : x[rr]);
}

// ---- B1: state-dependent products of a chunk, per wave (16 state columns):
// K S0, Q S0, R, the blocked substitution for Delta, and the state update.
// Every block of LDS operands is loaded in one batch (fenced with a
// scheduling barrier) before the products that use it.  Returns Q S0 and
// Delta (bf16, as the B operands of P Delta) for B2.
template <int NW>
__device__ __forceinline__ void phase_state(Smem<NW>& sm, int buf, f32x4 S[8], f32x4 QS[4], bf16x8 BD[2],
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
    // (I + A) Delta = R by blocked forward substitution over the four 16-row
    // blocks: Y_m = R_m - sum_{k<m} A_mk Delta_k, then Delta_m = Y_m + N_mm Y_m.
    // The fp32 accumulator carries R and Y exactly; only the coupling terms
    // see bf16 operands.
    f32x4 Dl[4];
    bf16x4 Db[4];
    const bf16x4 z4 = {__bf16(0.f), __bf16(0.f), __bf16(0.f), __bf16(0.f)};
    const bf16x4 dg[4] = {d0, d1, d2, d3};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 y = R[m];
        if (m == 1) y = mfma16(cat4(a10, z4), cat4(Db[0], z4), y);
        if (m == 2) y = mfma16(a2x, cat4(Db[0], Db[1]), y);
        if (m == 3) {
            y = mfma16(a3x, cat4(Db[0], Db[1]), y);
            y = mfma16(cat4(a32, z4), cat4(Db[2], z4), y);
        }
        const bf16x4 yb = __builtin_convertvector(y, bf16x4);
        Dl[m] = mfma16(cat4(dg[m], z4), cat4(yb, z4), y);
        Db[m] = __builtin_convertvector(Dl[m], bf16x4);
    }
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
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 q0 = su[2 * ks] * Dl[2 * ks], q1 = su[2 * ks + 1] * Dl[2 * ks + 1];
        BH[ks] = to_bf16x8(q0, q1);
        const f32x8 back = to_f32x8(BH[ks]);
        const f32x4 l0 = {q0[0] - back[0], q0[1] - back[1], q0[2] - back[2], q0[3] - back[3]};
        const f32x4 l1 = {q1[0] - back[4], q1[1] - back[5], q1[2] - back[6], q1[3] - back[7]};
        BL[ks] = to_bf16x8(l0, l1);
    }
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

// ---- B2: O = Gamma n_q (Q S0) + P Delta, staged (bf16) into the chunk's Q
// buffer, which no wave reads any more
template <int NW>
__device__ __forceinline__ void phase_out(Smem<NW>& sm, int buf, const f32x4 QS[4], const bf16x8 BD[2],
                                          int wave, int li, int lq) {
    constexpr int VLd = Smem<NW>::VLd;
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
            if (ks == 0 || m >= 2) acc = mfma16(pa[i++], BD[ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) Os[(16 * m + 4 * lq + e) * VLd + cw] = __bf16(acc[e]);
    }
}

// ---- C: O rows -> HBM (16-byte stores); checkpoint slot when the chunk end
// is a multiple of the checkpoint interval
template <int NW>
__device__ __forceinline__ void phase_store(const PrefillParams& p, Smem<NW>& sm, const Ctx& cx, int buf,
                                            const f32x4 S[8], int64_t kc, int64_t s_base, bool owns_qk_tail,
                                            int tid) {
    constexpr int NT = 64 * NW;
    constexpr int N = 16 * NW;
    constexpr int VLd = Smem<NW>::VLd;
    constexpr int NCH = Smem<NW>::NCH;
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

template <int NW>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(PrefillParams p) {
    constexpr int NT = 64 * NW;
    constexpr int N = 16 * NW;
    constexpr int S_SPLIT = kD / N;
    using SM = Smem<NW>;
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
        phase_front(p, sm, cx, 0, local0, tid);
        __syncthreads();
        phase_rows(p, sm, cx, 0, 1, local0, tid);
        __syncthreads();
        phase_masks(sm, 0, 1, tid);
        __syncthreads();
        if (wave == 0) phase_diag(sm, lane);
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
        bf16x8 BD[2];
        if (wave < NW / 2 || !next) {
            phase_state(sm, buf, S, QS, BD, wave, li, lq);
            if (next) phase_front(p, sm, cx, nbuf, nlocal0, tid);
        } else {
            phase_front(p, sm, cx, nbuf, nlocal0, tid);
            phase_state(sm, buf, S, QS, BD, wave, li, lq);
        }
        __syncthreads();
        phase_out(sm, buf, QS, BD, wave, li, lq);
        if (next) phase_rows(p, sm, cx, nbuf, buf, nlocal0, tid);
        __syncthreads();
        phase_store(p, sm, cx, buf, S, kc, s_base, owns_qk_tail, tid);
        if (next) phase_masks(sm, nbuf, buf, tid);
        __syncthreads();
        if (next) {
            if (wave == 0) phase_diag(sm, lane);
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

template <int NW>
hipError_t launch_nw(const PrefillParams& p, hipStream_t stream) {
    const int s_split = kD / (16 * NW);
    const int r = p.num_v_heads / p.num_k_heads;
    const int ng = p.batch * p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * s_split;
    hipLaunchKernelGGL((prefill_kernel<NW>), dim3(blocks), dim3(64 * NW), 0, stream, p);
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
    switch (prefill_waves()) {
        case 8: return launch_nw<8>(p, stream);
        case 4: return launch_nw<4>(p, stream);
        default: return launch_nw<2>(p, stream);
    }
}

}  // namespace gdn
