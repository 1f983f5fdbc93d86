// gdn_prefill_split.hip -- two-pass chunked prefill of the Gated DeltaNet
// core (gfx950): the path taken when the caller passes a workspace.
//
// The chunked form (gdn_chunk_common.h) splits into work that does not
// depend on the state and the short recurrence over chunks that does.  The
// fused kernel does both in one workgroup per (sequence, value head), which
// leaves most of the chip idle when batch x heads is small.  Here:
//
//   prep  (one workgroup per sequence, key head and chunk; every chunk of a
//         segment in parallel): front end of the q, k channels of the key
//         head and the v channels of its value heads, K^T, L2 norms, the raw
//         K K^T / Q K^T tiles, and per value head the gates, decay masks,
//         row scales and the diagonal-block inverses.  Results go to
//         workspace records in the operand order of the state kernel.
//   state (one workgroup per sequence, value head and slice of 16*NW state
//         columns; chunks in order): per chunk only the state-dependent
//         products -- K S0, Q S0, R, Delta by blocked forward substitution,
//         O, and the state update -- with the next chunk's records copied
//         into the other LDS buffer by global_load_lds while this chunk
//         computes.
//
// A workspace smaller than the whole call is used segment by segment (prep
// then state for each run of chunks that fits); the state travels between
// segments through rec_state_out.  Every value the state kernel consumes is
// bit-identical to what the fused kernel computes in LDS, so the two paths
// agree to the last bit up to the compiler's instruction choice.
#include "gdn_chunk_common.h"

namespace gdn {

namespace {

using namespace chunked;

// ---- workspace records.  Matrices are row-major, columns in pos() order,
// unpadded.  Key record (sequence, key head, chunk): Q | K | K^T.  Value
// record (sequence, value head, chunk): P | AN | five rows of 64 fp32
// (beta | beta Gamma n_k | Gamma n_q | exp(gamma_C - gamma) n_k |
// exp(gamma_C), 0, ...) | V^T ([column][token], natural token order).
constexpr int kRecQ = 0;
constexpr int kRecK = kC * kD * 2;
constexpr int kRecKt = 2 * kC * kD * 2;
constexpr int kKeyRec = 3 * kC * kD * 2;            // 49152
constexpr int kRecP = 0;
constexpr int kRecAN = kC * kC * 2;
constexpr int kRecTok = 2 * kC * kC * 2;
constexpr int kTokBytes = 5 * kC * 4;
constexpr int kRecVt = kRecTok + kTokBytes;
constexpr int kValRec = kRecVt + kD * kC * 2;       // 34048
static_assert(kKeyRec % 256 == 0 && kValRec % 256 == 0, "records keep 256-byte alignment");

// State-kernel LDS buffer: the key record and the first three parts of the
// value record, back to back (Q | K | K^T | P | AN | rows).
constexpr int kBufQ = 0, kBufK = kRecK, kBufKt = kRecKt, kBufP = kKeyRec, kBufAN = kKeyRec + kRecAN,
              kBufTok = kKeyRec + kRecTok;
constexpr int kBufBytes = kKeyRec + kRecVt;         // 66816
constexpr int kPieces = (kBufBytes + 1023) / 1024;  // 1 KiB per wave-wide global_load_lds

constexpr int kMaxGroup = 8;                        // value heads per key head on this path

struct SplitParams {
    PrefillParams p;
    char* ws;
    int64_t k0;          // absolute index of the segment's first chunk
    int32_t nseg;        // chunks in the segment
    int32_t first_seg;   // state comes from rec_in (else from rec_out)
    int32_t last_seg;    // write the final conv tail
};

__device__ __forceinline__ char* key_rec(const SplitParams& s, int b, int kh, int j) {
    return s.ws + (((int64_t)b * s.p.num_k_heads + kh) * s.nseg + j) * kKeyRec;
}

__device__ __forceinline__ char* val_rec(const SplitParams& s, int b, int h, int j) {
    return s.ws + (int64_t)s.p.batch * s.p.num_k_heads * s.nseg * kKeyRec +
           (((int64_t)b * s.p.num_v_heads + h) * s.nseg + j) * kValRec;
}

// Byte offset of 16-byte granule g of row `row` in the state kernel's LDS
// copy of a 256-byte-row (Q, K) or 128-byte-row (K^T, P, AN) matrix: the
// granule index is XORed with row % 8, so the eight rows read by one phase
// of a ds_read_b128 hit eight different granule columns (no bank conflict).
__device__ __forceinline__ int swz256(int row, int g) { return row * 256 + 16 * (g ^ (row & 7)); }
__device__ __forceinline__ int swz128(int row, int g) { return row * 128 + 16 * (g ^ (row & 7)); }

// ============================================================ prep kernel
constexpr int kPrepWaves = 8;
constexpr int kPrepThreads = 64 * kPrepWaves;

struct alignas(16) PrepSmem {
    __bf16 Qs[kC * kKsLd];
    __bf16 Ks[kC * kKsLd];
    __bf16 Ps[kC * kKtLd];
    __bf16 AN[kC * kKtLd];
    float AdT[4 * 16 * kXLd];
    alignas(16) float beta[kC];
    alignas(16) float gam[kC];
    alignas(16) float nq[kC];
    alignas(16) float nk[kC];
    float tokS[5][kC];
    float Ws[4 * (2 + kMaxGroup) * kD];   // conv taps [tap][channel]: q, k, then the group's v
};

__device__ __forceinline__ void copy16(char* dst, const void* src) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

__global__ __launch_bounds__(kPrepThreads)
void prep_kernel(SplitParams sp) {
    const PrefillParams& p = sp.p;
    __shared__ PrepSmem sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int li = lane % 16, lq = lane / 16;
    const int Hk = p.num_k_heads, r = p.num_v_heads / Hk;
    const int j = blockIdx.x % sp.nseg;
    const int grp = blockIdx.x / sp.nseg;
    const int b = grp / Hk, kh = grp % Hk;
    const int64_t local0 = (sp.k0 + j) * kC - p.start_pos;
    char* krec = key_rec(sp, b, kh, j);
    const int nch = (2 + r) * kD;

    // ---- set-up: conv taps -> LDS; zero the upper tiles of P and AN (the
    // masks never write them) and the unused part of the fifth row
    for (int e = tid; e < nch * 4; e += kPrepThreads) {
        const int ch = e % nch, tap = e / nch;
        const int64_t gc = ch < 2 * kD ? (ch < kD ? (int64_t)kh * kD + ch : (int64_t)Hk * kD + (int64_t)kh * kD + ch - kD)
                                       : 2 * (int64_t)Hk * kD + (int64_t)kh * r * kD + (ch - 2 * kD);
        sm.Ws[tap * nch + ch] = bf16_bits_to_f32(static_cast<const uint16_t*>(p.conv_w)[gc * 4 + tap]);
    }
    for (int e = tid; e < 6 * 256; e += kPrepThreads) {
        const int t6 = e / 256, rr = (e / 16) % 16, cc = e % 16;
        const int m = t6 < 3 ? 0 : (t6 < 5 ? 1 : 2);
        const int pp = t6 < 3 ? t6 + 1 : (t6 < 5 ? t6 - 1 : 3);
        sm.Ps[(16 * m + rr) * kKtLd + pos(16 * pp + cc)] = __bf16(0.f);
        sm.AN[(16 * m + rr) * kKtLd + pos(16 * pp + cc)] = __bf16(0.f);
    }
    if (tid < kC) sm.tokS[4][tid] = 0.f;
    __syncthreads();

    // ---- front end: q, k -> LDS rows; v -> the V^T part of each value record
    {
        const int cg4 = nch / 4;
        const bool interior = local0 >= 3 && local0 + kC <= p.seq_len;
        for (int item = tid; item < cg4 * 8; item += kPrepThreads) {
            const int ch0 = (item % cg4) * 4, tau0 = (item / cg4) * 8;
            const int64_t gc = ch0 < 2 * kD ? (ch0 < kD ? (int64_t)kh * kD + ch0
                                                         : (int64_t)Hk * kD + (int64_t)kh * kD + ch0 - kD)
                                            : 2 * (int64_t)Hk * kD + (int64_t)kh * r * kD + (ch0 - 2 * kD);
            float w[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 wv = *reinterpret_cast<const f32x4*>(&sm.Ws[t * nch + ch0]);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[t][i] = wv[i];
            }
            bf16x4 ub[8];
            if (interior) conv_item<true>(p, b, gc, local0, tau0, w, ub);
            else conv_item<false>(p, b, gc, local0, tau0, w, ub);
            if (ch0 < 2 * kD) {
                __bf16* dst0 = ch0 < kD ? &sm.Qs[pos(ch0)] : &sm.Ks[pos(ch0 - kD)];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) *reinterpret_cast<bf16x4*>(dst0 + (tau0 + tt) * kKsLd) = ub[tt];
            } else {
                const int hh = (ch0 - 2 * kD) / kD, col = (ch0 - 2 * kD) % kD;
                char* vt = val_rec(sp, b, kh * r + hh, j) + kRecVt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16x8 v{ub[0][i], ub[1][i], ub[2][i], ub[3][i], ub[4][i], ub[5][i], ub[6][i], ub[7][i]};
                    *reinterpret_cast<bf16x8*>(vt + (col + i) * (kC * 2) + tau0 * 2) = v;
                }
            }
        }
    }
    __syncthreads();

    // ---- Q, K, K^T -> key record; L2 norms; raw Gram tiles (registers)
    for (int e = tid; e < 2 * kC * 16; e += kPrepThreads) {
        const int mat = e >> 10, row = (e >> 4) & 63, g = e & 15;
        copy16(krec + (mat ? kRecK : kRecQ) + row * 256 + 16 * g, (mat ? sm.Ks : sm.Qs) + row * kKsLd + 8 * g);
    }
    for (int e = tid; e < kD * 8; e += kPrepThreads) {
        // granule G of K^T row d holds tokens 32a + 4q + {0..3}, 32a + 16 + 4q + {0..3}
        const int d = e >> 3, G = e & 7;
        const int x0 = 32 * (G >> 2) + 4 * (G & 3);
        const int pd = pos(d);
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = sm.Ks[(x0 + i) * kKsLd + pd];
            v[4 + i] = sm.Ks[(x0 + 16 + i) * kKsLd + pd];
        }
        *reinterpret_cast<bf16x8*>(krec + kRecKt + d * (kC * 2) + 16 * G) = v;
    }
    if (tid < 2 * kC) {
        const bool isq = tid < kC;
        const int tau = tid % kC;
        const float n = row_inv_norm((isq ? sm.Qs : sm.Ks) + tau * kKsLd, isq ? p.q_scale : 1.0f, p.l2_eps);
        (isq ? sm.nq : sm.nk)[tau] = n;
    }
    // wave w keeps the K K^T and Q K^T tiles of lower tile pairs w and w + 8
    f32x4 gk[2], gq[2];
    gk[0] = gram_tile(sm.Ks, sm.Qs, wave, li, lq);
    gq[0] = gram_tile(sm.Ks, sm.Qs, 10 + wave, li, lq);
    if (wave < 2) {
        gk[1] = gram_tile(sm.Ks, sm.Qs, 8 + wave, li, lq);
        gq[1] = gram_tile(sm.Ks, sm.Qs, 18 + wave, li, lq);
    }
    __syncthreads();

    // ---- per value head of the group: gates, masks, row scales, diagonal
    // inverses -> value record
    for (int hh = 0; hh < r; ++hh) {
        const int h = kh * r + hh;
        char* vrec = val_rec(sp, b, h, j);
        if (wave == 0) {
            gates_scan(p, b, h, -expf(p.A_log[h]), p.dt_bias[h], local0, lane, sm.gam, sm.beta);
        } else if (hh > 0) {
            char* prev = val_rec(sp, b, h - 1, j) + kRecAN;
            for (int e = tid - 64; e < kC * 8; e += kPrepThreads - 64)
                copy16(prev + (e >> 3) * 128 + 16 * (e & 7), sm.AN + (e >> 3) * kKtLd + 8 * (e & 7));
        }
        __syncthreads();
        mask_pair(sm, wave, gk[0], gq[0], lane);
        if (wave < 2) mask_pair(sm, 8 + wave, gk[1], gq[1], lane);
        if (wave == kPrepWaves - 1) {
            row_scales(sm, lane);
            if (lane == 0) sm.tokS[4][0] = expf(sm.gam[kC - 1]);
        }
        __syncthreads();
        if (wave == 0) {
            diag_solve<true>(sm, lane);
        } else {
            for (int e = tid - 64; e < kC * 8 + kTokBytes / 16; e += kPrepThreads - 64) {
                if (e < kC * 8) copy16(vrec + kRecP + (e >> 3) * 128 + 16 * (e & 7), sm.Ps + (e >> 3) * kKtLd + 8 * (e & 7));
                else copy16(vrec + kRecTok + 16 * (e - kC * 8), &sm.tokS[0][0] + 4 * (e - kC * 8));
            }
        }
        __syncthreads();
    }
    char* last = val_rec(sp, b, kh * r + r - 1, j) + kRecAN;
    for (int e = tid; e < kC * 8; e += kPrepThreads)
        copy16(last + (e >> 3) * 128 + 16 * (e & 7), sm.AN + (e >> 3) * kKtLd + 8 * (e & 7));
}

// ============================================================ state kernel
#define LDS_PTR(x) ((__attribute__((address_space(3))) void*)(x))

// Start the copy of one chunk's records into an LDS buffer: 1 KiB pieces,
// one wave-wide global_load_lds_dwordx4 each, granules placed by swz256 /
// swz128.  Completion is awaited with the workgroup barrier.
template <int NW>
__device__ __forceinline__ void issue_chunk(char* lds, const char* krec, const char* vrec, int wave, int lane) {
    for (int pc = wave; pc < kPieces; pc += NW) {
        const int o = pc * 1024 + 16 * lane;
        const char* src;
        bool act = true;
        if (o < kBufKt) {
            const int row = (o >> 8) & (kC - 1), s = (o >> 4) & 15;
            src = krec + (o & ~255) + 16 * (s ^ (row & 7));
        } else if (o < kBufP) {
            const int l = o - kBufKt, row = l >> 7, s = (l >> 4) & 7;
            src = krec + kRecKt + (l & ~127) + 16 * (s ^ (row & 7));
        } else if (o < kBufTok) {
            const int l = o - kBufP, row = l >> 7, s = (l >> 4) & 7;
            src = vrec + (l & ~127) + 16 * (s ^ (row & 7));
        } else {
            const int l = o - kBufTok;
            act = l < kTokBytes;
            src = vrec + kRecTok + l;
        }
        if (act) __builtin_amdgcn_global_load_lds(src, LDS_PTR(lds + pc * 1024), 16, 0, 0);
    }
}

// V rows 16m + 4lq + {0..3} of this lane's column (registers)
__device__ __forceinline__ void load_v(const char* vrec, int col, int lq, bf16x4 vv[4]) {
    const char* base = vrec + kRecVt + col * (kC * 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) vv[m] = *reinterpret_cast<const bf16x4*>(base + (16 * m + 4 * lq) * 2);
}

__device__ __forceinline__ bf16x8 ld8(const char* buf, int off) { return *reinterpret_cast<const bf16x8*>(buf + off); }
__device__ __forceinline__ bf16x4 ld4(const char* buf, int off) { return *reinterpret_cast<const bf16x4*>(buf + off); }
__device__ __forceinline__ f32x4 ldf4(const char* buf, int off) { return *reinterpret_cast<const f32x4*>(buf + off); }

// State-dependent products of one chunk for this wave's 16 columns: K S0,
// Q S0, R = beta V - beta Gamma n_k (K S0), Delta, the state update.
// Returns Q S0 and Delta (bf16 B operands of P Delta).
__device__ __forceinline__ void state_products(const char* buf, f32x4 S[8], const bf16x4 vv[4], f32x4 QS[4],
                                               bf16x8 BD[2], int li, int lq) {
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
                const int off = swz256(16 * (mh + mm) + li, 4 * ks + lq);
                ak[mm][ks] = ld8(buf, kBufK + off);
                aq[mm][ks] = ld8(buf, kBufQ + off);
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
    // row scales for this lane's rows 16m + 4lq + e and the A-operand slots
    // of the substitution (token block k of an AN row sits in granule
    // 4 (k / 2) + lq, half k % 2)
    f32x4 sb[4], sr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = 16 * m + 4 * lq;
        sb[m] = ldf4(buf, kBufTok + 4 * (0 * kC + r0));
        sr[m] = ldf4(buf, kBufTok + 4 * (1 * kC + r0));
    }
    const bf16x4 d0 = ld4(buf, kBufAN + swz128(li, lq));
    const bf16x4 d1 = ld4(buf, kBufAN + swz128(16 + li, lq) + 8);
    const bf16x4 d2 = ld4(buf, kBufAN + swz128(32 + li, 4 + lq));
    const bf16x4 d3 = ld4(buf, kBufAN + swz128(48 + li, 4 + lq) + 8);
    const bf16x4 a10 = ld4(buf, kBufAN + swz128(16 + li, lq));
    const bf16x8 a2x = ld8(buf, kBufAN + swz128(32 + li, lq));
    const bf16x8 a3x = ld8(buf, kBufAN + swz128(48 + li, lq));
    const bf16x4 a32 = ld4(buf, kBufAN + swz128(48 + li, 4 + lq));
    __builtin_amdgcn_sched_barrier(0);
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
    // S <- exp(gamma_C) S + K^T Delta'  (Delta' as bf16 hi + lo)
    f32x4 su[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) su[m] = ldf4(buf, kBufTok + 4 * (3 * kC + 16 * m + 4 * lq));
    bf16x8 akt[8][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) akt[t][ks] = ld8(buf, kBufKt + swz128(16 * t + li, 4 * ks + lq));
    const float eC = *reinterpret_cast<const float*>(buf + kBufTok + 4 * 4 * kC);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 BH[2], BL[2];
    split_hi_lo(su, Dl, BH, BL);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t == 4) {
#pragma unroll
            for (int tt = 4; tt < 8; ++tt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) akt[tt][ks] = ld8(buf, kBufKt + swz128(16 * tt + li, 4 * ks + lq));
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

// O = Gamma n_q (Q S0) + P Delta for this wave's 16 columns -> Os (bf16)
template <int VLd>
__device__ __forceinline__ void out_tile(const char* buf, __bf16* Os, const f32x4 QS[4], const bf16x8 BD[2],
                                         int cw, int li, int lq) {
    f32x4 so[4];
    bf16x8 pa[6];
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        so[m] = ldf4(buf, kBufTok + 4 * (2 * kC + 16 * m + 4 * lq));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) pa[i++] = ld8(buf, kBufP + swz128(16 * m + li, 4 * ks + lq));
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

struct StateCtx {
    int b, kh, h, zcol0;
    bool owns_qk_tail;
    int64_t s_base;
};

// Global channel of the state workgroup's channel index ch (q: 0..127,
// k: 128..255, then its v columns)
__device__ __forceinline__ int64_t state_channel(const PrefillParams& p, const StateCtx& cx, int ch) {
    if (ch < kD) return (int64_t)cx.kh * kD + ch;
    if (ch < 2 * kD) return (int64_t)p.num_k_heads * kD + (int64_t)cx.kh * kD + (ch - kD);
    return 2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + (ch - 2 * kD);
}

// O rows of chunk kc (staged in Os) -> HBM, 16-byte stores, spread over
// `nthr` threads starting at thread `t0`
template <int NW>
__device__ __forceinline__ void store_rows(const PrefillParams& p, const StateCtx& cx, const __bf16* Os, int64_t kc,
                                           int t0, int nthr) {
    constexpr int N = 16 * NW, VLd = N + 8, V8 = N / 8;
    const int64_t local0 = kc * kC - p.start_pos;
    uint16_t* out = static_cast<uint16_t*>(p.out);
    for (int e = t0; e < kC * V8; e += nthr) {
        const int tau = e / V8, c8 = e % V8;
        const int64_t t = local0 + tau;
        if (t >= 0 && t < p.seq_len)
            *reinterpret_cast<uint4*>(out + (((int64_t)cx.b * p.seq_len + t) * p.num_v_heads + cx.h) * kD + cx.zcol0 + 8 * c8) =
                *reinterpret_cast<const uint4*>(&Os[tau * VLd + 8 * c8]);
    }
}

// Checkpoint slot when the end of chunk kc is a multiple of the checkpoint
// interval: this wave's state slice and (with the compute threads) the conv
// tails of the workgroup's channels
template <int NW>
__device__ __forceinline__ void checkpoint(const PrefillParams& p, const StateCtx& cx, const f32x4 S[8], int64_t kc,
                                           int tid) {
    constexpr int NT = 64 * NW, N = 16 * NW, NCH = 2 * kD + N;
    const int lq = (tid % 64) / 16;
    const int64_t pe = (kc + 1) * kC;
    if (p.ckpt_interval > 0 && pe % p.ckpt_interval == 0 && pe <= p.start_pos + p.seq_len) {
        char* slot = p.ckpt_buf + (uint64_t)(pe / p.ckpt_interval - 1) * p.slot_bytes;
        float* rec = reinterpret_cast<float*>(slot + p.conv_slot_bytes);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
        uint16_t* ctail = reinterpret_cast<uint16_t*>(slot);
        for (int ch = tid; ch < NCH; ch += NT)
            if (ch >= 2 * kD || cx.owns_qk_tail) write_tail(p, cx.b, pe - p.start_pos, state_channel(p, cx, ch), ctail);
    }
}

// Memory waves per state workgroup: eight waves in all
template <int NW> constexpr int kMemWaves = 8 - NW;

// One chunk of the state kernel.  Compute waves (0..NW-1): prefetch the next
// chunk's V rows, the state-dependent products, O -> Os[j % 2]; after the
// barrier the checkpoint.  Memory waves (NW..7): copy the next chunk's
// records into the other buffer, store the previous chunk's O rows, wait for
// the copies.  Every wave passes the same barrier outside the role branches.
template <int NW>
__device__ __forceinline__ void state_step(const SplitParams& sp, const StateCtx& cx, const char* cur, char* nxt,
                                           __bf16* Os, const __bf16* Os_prev, f32x4 S[8], bf16x4 vv[4], int j,
                                           int wave, int tid) {
    constexpr int VLd = 16 * NW + 8, NM = kMemWaves<NW>;
    const int lane = tid % 64, li = lane % 16, lq = lane / 16;
    const bool mem = wave >= NW;
    const bool more = j + 1 < sp.nseg;
    bf16x4 vn[4];
    if (mem) {
        if (more) issue_chunk<NM>(nxt, key_rec(sp, cx.b, cx.kh, j + 1), val_rec(sp, cx.b, cx.h, j + 1), wave - NW, lane);
        if (j > 0) store_rows<NW>(sp.p, cx, Os_prev, sp.k0 + j - 1, tid - 64 * NW, 64 * NM);
    } else {
        f32x4 QS[4];
        bf16x8 BD[2];
        if (more) load_v(val_rec(sp, cx.b, cx.h, j + 1), cx.zcol0 + 16 * wave + li, lq, vn);
        state_products(cur, S, vv, QS, BD, li, lq);
        out_tile<VLd>(cur, Os, QS, BD, 16 * wave + li, li, lq);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!mem) {
        if (more) {
#pragma unroll
            for (int m = 0; m < 4; ++m) vv[m] = vn[m];
        }
        checkpoint<NW>(sp.p, cx, S, sp.k0 + j, tid);
    }
}

// Waves 0..NW-1 own 16 state columns each; waves NW..7 move data.
template <int NW>
__global__ __launch_bounds__(512) void state_kernel(SplitParams sp) {
    static_assert(NW == 2 || NW == 4, "two or four compute waves");
    constexpr int NTALL = 512, N = 16 * NW, VLd = N + 8, NCH = 2 * kD + N, NM = kMemWaves<NW>;
    constexpr int S_SPLIT = kD / N;
    const PrefillParams& p = sp.p;
    __shared__ __attribute__((aligned(16))) char buf0[kBufBytes];
    __shared__ __attribute__((aligned(16))) char buf1[kBufBytes];
    __shared__ __attribute__((aligned(16))) __bf16 Os[2][kC * VLd];   // output staging, per chunk parity

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: role branches stay scalar
    const int li = lane % 16, lq = lane / 16;
    const bool mem = wave >= NW;
    // workgroup -> (b, key head, member); the r * S_SPLIT members of one
    // (b, key head) share a blockIdx % 8, so the round-robin dispatch puts
    // them on one XCD and its L2, where their common key records stay
    const int r = p.num_v_heads / p.num_k_heads;
    const int M = r * S_SPLIT;
    const int NG = p.batch * p.num_k_heads;
    const int bid = blockIdx.x;
    const int grp = (bid / 8 / M) * 8 + bid % 8;
    const int member = (bid / 8) % M;
    if (grp >= NG) return;
    StateCtx cx;
    cx.b = grp / p.num_k_heads;
    cx.kh = grp % p.num_k_heads;
    cx.h = cx.kh * r + member / S_SPLIT;
    cx.zcol0 = (member % S_SPLIT) * N;
    cx.owns_qk_tail = member == 0;
    cx.s_base = ((int64_t)cx.b * p.num_v_heads + cx.h) * kD * kD + cx.zcol0 + 16 * (mem ? 0 : wave) + li;

    const float* s_src = sp.first_seg ? p.rec_in : p.rec_out;
    f32x4 S[8];
    bf16x4 vv[4];
    if (!mem) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[t][e] = s_src ? s_src[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] : 0.f;
        if (sp.nseg > 0) load_v(val_rec(sp, cx.b, cx.h, 0), cx.zcol0 + 16 * wave + li, lq, vv);
    } else if (sp.nseg > 0) {
        issue_chunk<NM>(buf0, key_rec(sp, cx.b, cx.kh, 0), val_rec(sp, cx.b, cx.h, 0), wave - NW, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // two chunks per trip so that each LDS buffer is a distinct object: the
    // compiler then orders reads of one buffer only after its own copies
    for (int j = 0; j < sp.nseg; j += 2) {
        state_step<NW>(sp, cx, buf0, buf1, Os[0], Os[1], S, vv, j, wave, tid);
        if (j + 1 < sp.nseg) state_step<NW>(sp, cx, buf1, buf0, Os[1], Os[0], S, vv, j + 1, wave, tid);
    }
    if (mem && sp.nseg > 0) store_rows<NW>(p, cx, Os[(sp.nseg - 1) & 1], sp.k0 + sp.nseg - 1, tid - 64 * NW, 64 * NM);

    if (!mem) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.rec_out[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
    }
    if (sp.last_seg) {
        for (int ch = tid; ch < NCH; ch += NTALL)
            if (ch >= 2 * kD || cx.owns_qk_tail)
                write_tail(p, cx.b, p.seq_len, state_channel(p, cx, ch), static_cast<uint16_t*>(p.conv_out));
    }
}

template <int NW>
hipError_t launch_state(const SplitParams& sp, hipStream_t stream) {
    const int s_split = kD / (16 * NW);
    const int r = sp.p.num_v_heads / sp.p.num_k_heads;
    const int ng = sp.p.batch * sp.p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * s_split;
    hipLaunchKernelGGL((state_kernel<NW>), dim3(blocks), dim3(512), 0, stream, sp);
    return hipGetLastError();
}

// Compute waves (16 state columns each) per state workgroup.  One workgroup
// fits a CU (two 65 KiB LDS buffers), and a CU streams the records at a
// bounded rate, so with few (sequence, head) pairs the narrower workgroups
// spread the chains over more CUs.  GDN_PREFILL_STATE_WAVES (2 or 4)
// overrides the choice.
int state_waves(const PrefillParams& p) {
    if (const char* env = getenv("GDN_PREFILL_STATE_WAVES")) {
        const int v = atoi(env);
        if (v == 2 || v == 4) return v;
    }
    const int64_t heads = (int64_t)p.batch * p.num_v_heads;
    return heads * 4 <= 256 ? 2 : 4;
}

}  // namespace

bool prefill_split_supported(const PrefillParams& p) {
    const int r = p.num_v_heads / p.num_k_heads;
    return r >= 1 && r <= kMaxGroup;
}

uint64_t prefill_split_chunk_bytes(int batch, int num_k_heads, int num_v_heads) {
    return (uint64_t)batch * ((uint64_t)num_k_heads * kKeyRec + (uint64_t)num_v_heads * kValRec);
}

hipError_t launch_prefill_split(const PrefillParams& p, void* ws, uint64_t ws_bytes, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    const uint64_t per = prefill_split_chunk_bytes(p.batch, p.num_k_heads, p.num_v_heads);
    const int64_t k_first = p.start_pos / kC;
    const int64_t k_end = p.seq_len > 0 ? (p.start_pos + p.seq_len - 1) / kC + 1 : k_first;
    // segments of at most 2^30 / (B H_k) chunks keep the prep grid in range
    int64_t max_seg = (int64_t)(ws_bytes / per);
    const int64_t grid_cap = ((int64_t)1 << 30) / ((int64_t)p.batch * p.num_k_heads);
    if (max_seg > grid_cap) max_seg = grid_cap;
    const int nw = state_waves(p);
    SplitParams sp{};
    sp.p = p;
    sp.ws = static_cast<char*>(ws);
    sp.first_seg = 1;
    if (k_end == k_first) {
        sp.k0 = k_first;
        sp.nseg = 0;
        sp.last_seg = 1;
        return nw == 4 ? launch_state<4>(sp, stream) : launch_state<2>(sp, stream);
    }
    for (int64_t k0 = k_first; k0 < k_end; k0 += max_seg) {
        const int64_t n = k_end - k0 < max_seg ? k_end - k0 : max_seg;
        sp.k0 = k0;
        sp.nseg = (int32_t)n;
        sp.last_seg = k0 + n == k_end;
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(p.batch * p.num_k_heads * n)), dim3(kPrepThreads), 0, stream, sp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = nw == 4 ? launch_state<4>(sp, stream) : launch_state<2>(sp, stream);
        if (e != hipSuccess) return e;
        sp.first_seg = 0;
    }
    return hipSuccess;
}

}  // namespace gdn
