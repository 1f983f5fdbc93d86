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
//         head, L2 norms, the raw K K^T / Q K^T tiles, and per value head
//         of the group the gates, decay masks, row scales and the
//         diagonal-block inverses.  Results go to workspace records in the
//         operand order of the state kernel.
//   state (one workgroup per sequence, value head and slice of 16 * NW
//         state columns, NW = 2 or 4; chunks in order): NW compute waves do
//         only the state-dependent products of each chunk -- K S0, Q S0, R,
//         Delta by blocked forward substitution, the state update, O --
//         while 8 - NW memory waves store the previous chunk's O rows and
//         prepare the next chunk in the other LDS buffer: its records by
//         global_load_lds, K^T by an LDS transpose of K, and the front end of
//         the slice's v channels (conv + SiLU from a raw slab copied one chunk
//         earlier; the slice's own columns, so no value-head data goes
//         through the workspace).
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
// unpadded.  Key record (sequence, key head, chunk): Q | K.  Value record
// (sequence, value head, chunk): P | AN | five rows of 64 fp32
// (beta | beta Gamma n_k | Gamma n_q | exp(gamma_C - gamma) n_k |
// exp(gamma_C), 0, ...).
constexpr int kRecQ = 0;
constexpr int kRecK = kC * kD * 2;
constexpr int kKeyRec = 2 * kC * kD * 2;            // 32768
constexpr int kRecP = 0;
constexpr int kRecAN = kC * kC * 2;
constexpr int kRecTok = 2 * kC * kC * 2;
constexpr int kTokBytes = 5 * kC * 4;
constexpr int kValRec = kRecTok + kTokBytes;        // 17664
static_assert(kKeyRec % 256 == 0 && kValRec % 256 == 0, "records keep 256-byte alignment");

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

__device__ __forceinline__ void copy16(char* dst, const void* src) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// ============================================================ prep kernel
constexpr int kPrepWaves = 8;
constexpr int kPrepThreads = 64 * kPrepWaves;

struct alignas(16) PrepSmem {
    __bf16 Qs[kC * kKsLd];
    __bf16 Ks[kC * kKsLd];
    __bf16 Ps[kC * kKtLd];
    __bf16 AN[kC * kKtLd];
    float AdT[4 * 16 * kXLd];
    alignas(16) float beta[kMaxGroup][kC];   // per value head of the group
    alignas(16) float gam[kMaxGroup][kC];
    alignas(16) float nq[kC];
    alignas(16) float nk[kC];
    float tokS[5][kC];
    uint16_t Ws[4 * 2 * kD];   // conv taps (bf16 bits) [tap][channel]: q, then k
};

// One value head's view of the prep LDS, in the member names the shared
// mask, row-scale and solve helpers use.
struct PrepHeadView {
    float* gam;
    float* beta;
    float* nq;
    float* nk;
    __bf16* Ps;
    __bf16* AN;
    float* AdT;
    float (*tokS)[kC];
};

// Global channel of prep channel index ch: q then k of key head kh
__device__ __forceinline__ int64_t qk_channel(int ch, int kh, int Hk) {
    return ch < kD ? (int64_t)kh * kD + ch : (int64_t)Hk * kD + (int64_t)kh * kD + ch - kD;
}

// Front end of the q, k channels of a chunk -> LDS rows (4 channels x 8 rows
// per item, one item per thread)
template <bool INTERIOR>
__device__ __forceinline__ void prep_front(const PrefillParams& p, PrepSmem& sm, int b, int kh, int64_t local0,
                                           int tid) {
    static_assert(2 * kD / 4 * 8 == kPrepThreads, "one front-end item per thread");
    const int ch0 = (tid % 64) * 4, tau0 = (tid / 64) * 8;
    const int64_t gc = qk_channel(ch0, kh, p.num_k_heads);
    uint2 raw[11];
    conv_load<INTERIOR>(p, b, gc, local0, tau0, raw);
    float w[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) unpack_bf16x4(*reinterpret_cast<const uint2*>(&sm.Ws[t * 2 * kD + ch0]), w[t]);
    bf16x4 ub[8];
    conv_compute<INTERIOR>(p, b, gc, local0, tau0, w, raw, ub);
    __bf16* dst0 = ch0 < kD ? &sm.Qs[pos(ch0)] : &sm.Ks[pos(ch0 - kD)];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) *reinterpret_cast<bf16x4*>(dst0 + (tau0 + tt) * kKsLd) = ub[tt];
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

    // ---- set-up: gates of every value head of the group (wave hh: head
    // kh r + hh); conv taps -> LDS; zero the upper tiles of P and AN (the
    // masks never write them) and the unused part of the fifth row
    if (wave < r) {
        const int h = kh * r + wave;
        gates_scan(p, b, h, -expf(p.A_log[h]), p.dt_bias[h], local0, lane, sm.gam[wave], sm.beta[wave]);
    }
    for (int e = tid; e < 2 * kD * 4; e += kPrepThreads) {
        const int ch = e % (2 * kD), tap = e / (2 * kD);
        sm.Ws[e] = static_cast<const uint16_t*>(p.conv_w)[qk_channel(ch, kh, Hk) * 4 + tap];
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

    // ---- front end of q, k
    if (local0 >= 3 && local0 + kC <= p.seq_len) prep_front<true>(p, sm, b, kh, local0, tid);
    else prep_front<false>(p, sm, b, kh, local0, tid);
    __syncthreads();

    // ---- Q, K -> key record; L2 norms; raw Gram tiles (registers)
    for (int e = tid; e < 2 * kC * 16; e += kPrepThreads) {
        const int mat = e >> 10, row = (e >> 4) & 63, g = e & 15;
        copy16(krec + (mat ? kRecK : kRecQ) + row * 256 + 16 * g, (mat ? sm.Ks : sm.Qs) + row * kKsLd + 8 * g);
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

    // ---- per value head of the group: masks, row scales, diagonal
    // inverses -> value record
    for (int hh = 0; hh < r; ++hh) {
        char* vrec = val_rec(sp, b, kh * r + hh, j);
        PrepHeadView hv{sm.gam[hh], sm.beta[hh], sm.nq, sm.nk, sm.Ps, sm.AN, sm.AdT, sm.tokS};
        mask_pair(hv, wave, gk[0], gq[0], lane);
        if (wave < 2) mask_pair(hv, 8 + wave, gk[1], gq[1], lane);
        if (wave == kPrepWaves - 1) {
            row_scales(hv, lane);
            if (lane == 0) sm.tokS[4][0] = expf(sm.gam[hh][kC - 1]);
        }
        __syncthreads();
        if (wave == 0) {
            diag_solve<true>(hv, lane);
        } else {
            for (int e = tid - 64; e < kC * 8 + kTokBytes / 16; e += kPrepThreads - 64) {
                if (e < kC * 8) copy16(vrec + kRecP + (e >> 3) * 128 + 16 * (e & 7), sm.Ps + (e >> 3) * kKtLd + 8 * (e & 7));
                else copy16(vrec + kRecTok + 16 * (e - kC * 8), &sm.tokS[0][0] + 4 * (e - kC * 8));
            }
        }
        __syncthreads();
        for (int e = tid; e < kC * 8; e += kPrepThreads)
            copy16(vrec + kRecAN + (e >> 3) * 128 + 16 * (e & 7), sm.AN + (e >> 3) * kKtLd + 8 * (e & 7));
        if (hh + 1 < r) __syncthreads();
    }
}

// ============================================================ state kernel
#define LDS_PTR(x) ((__attribute__((address_space(3))) void*)(x))

// P and AN in LDS hold only their lower triangle of 16x16 tiles: rows 0..31
// keep granules 0..3 (64-byte rows), rows 32..63 all eight (128-byte rows).
// Granules are XOR-swizzled so that eight consecutive rows read by one phase
// of an LDS read hit eight different bank groups.
constexpr int kPaMat = 32 * 64 + 32 * 128;          // 6144 bytes per matrix
__device__ __forceinline__ int pa_off(int mat, int row, int g) {
    return mat * kPaMat + (row < 32 ? row * 64 + 16 * (g ^ ((row >> 1) & 3))
                                    : 2048 + (row - 32) * 128 + 16 * (g ^ (row & 7)));
}

// LDS buffer of one chunk: Q | K | K^T | P | AN | rows | V^T (V^T of the
// slice's columns, row stride kVtLd).  Once the chunk's products are done,
// its Q region stages the chunk's O rows ([64][slice] bf16).
constexpr int kVtLd = kC + 4;                       // bf16 row stride of V^T (conflict-free column reads)
constexpr int kBufQ = 0, kBufK = kC * kD * 2, kBufKt = 2 * kC * kD * 2, kBufPA = 3 * kC * kD * 2,
              kBufTok = kBufPA + 2 * kPaMat, kBufVt = kBufTok + kTokBytes;
static_assert(kBufPA % 1024 == 0 && kBufTok % 1024 == 0 && kBufVt % 16 == 0, "piece and row alignment");

// Record copies of one chunk: 1 KiB pieces, one wave-wide
// global_load_lds_dwordx4 each.  Pieces 0..15: Q, 16..31: K (256-byte rows),
// 32..43: P | AN triangles, 44..45: the rows of scales (1280 bytes).
constexpr int kPiecesK = 16, kPiecesPA = 32, kPiecesTok = 44, kPieces = 46;

__device__ __forceinline__ void issue_piece(char* lds, const char* krec, const char* vrec, int pc, int lane) {
    const char* src;
    int dst;
    bool act = true;
    if (pc < kPiecesPA) {
        const int o = (pc & 15) * 1024 + 16 * lane;   // offset inside Q or K
        const int row = o >> 8, s = (o >> 4) & 15;
        src = krec + (pc < kPiecesK ? kRecQ : kRecK) + row * 256 + 16 * (s ^ (row & 7));
        dst = (pc < kPiecesK ? kBufQ : kBufK) + o;
    } else if (pc < kPiecesTok) {
        const int o = (pc - kPiecesPA) * 1024 + 16 * lane;
        const int mat = o / kPaMat, l = o % kPaMat;
        int row, g;
        if (l < 2048) {
            row = l >> 6;
            g = ((l >> 4) & 3) ^ ((row >> 1) & 3);
        } else {
            row = 32 + ((l - 2048) >> 7);
            g = ((l >> 4) & 7) ^ (row & 7);
        }
        src = vrec + mat * (kC * kC * 2) + row * 128 + 16 * g;
        dst = kBufPA + o;
    } else {
        const int l = (pc - kPiecesTok) * 1024 + 16 * lane;
        act = l < kTokBytes;
        src = vrec + kRecTok + l;
        dst = kBufTok + l;
    }
    if (act) __builtin_amdgcn_global_load_lds(src, LDS_PTR(lds + (dst & ~1023)), 16, 0, 0);
}

// K^T granules G in [g0, g0 + 4) of every row d from the chunk's K: granule G
// of K^T row d holds tokens 32a + 4q + {0..3}, 32a + 16 + 4q + {0..3}
// (a = G / 4, q = G % 4), which all lie in K rows 32a .. 32a + 31.
__device__ __forceinline__ void transpose_k(char* buf, int g0, int lane) {
    for (int e = lane; e < kD * 4; e += 64) {
        const int d = e >> 2, G = g0 + (e & 3);
        const int x0 = 32 * (G >> 2) + 4 * (G & 3);
        const int pd = pos(d), gk = pd >> 3, ek = (pd & 7) * 2;
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = *reinterpret_cast<const __bf16*>(buf + kBufK + swz256(x0 + i, gk) + ek);
            v[4 + i] = *reinterpret_cast<const __bf16*>(buf + kBufK + swz256(x0 + 16 + i, gk) + ek);
        }
        *reinterpret_cast<bf16x8*>(buf + kBufKt + swz128(d, G)) = v;
    }
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
    const char* an = buf + kBufPA;
    const bf16x4 d0 = ld4(an, pa_off(1, li, lq));
    const bf16x4 d1 = ld4(an, pa_off(1, 16 + li, lq) + 8);
    const bf16x4 d2 = ld4(an, pa_off(1, 32 + li, 4 + lq));
    const bf16x4 d3 = ld4(an, pa_off(1, 48 + li, 4 + lq) + 8);
    const bf16x4 a10 = ld4(an, pa_off(1, 16 + li, lq));
    const bf16x8 a2x = ld8(an, pa_off(1, 32 + li, lq));
    const bf16x8 a3x = ld8(an, pa_off(1, 48 + li, lq));
    const bf16x4 a32 = ld4(an, pa_off(1, 48 + li, 4 + lq));
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

// O = Gamma n_q (Q S0) + P Delta for this wave's 16 columns (fp32 registers,
// rows 16m + 4lq + e)
__device__ __forceinline__ void out_tile(const char* buf, const f32x4 QS[4], const bf16x8 BD[2], f32x4 O[4], int li,
                                         int lq) {
    f32x4 so[4];
    bf16x8 pa[6];
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        so[m] = ldf4(buf, kBufTok + 4 * (2 * kC + 16 * m + 4 * lq));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) pa[i++] = ld8(buf + kBufPA, pa_off(0, 16 * m + li, 4 * ks + lq));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        f32x4 acc = so[m] * QS[m];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) acc = mfma16(pa[i++], BD[ks], acc);
        O[m] = acc;
    }
}

// O (bf16) -> the chunk's Q region as [64][N] rows.  Lanes 2i and 2i + 1
// (adjacent columns) swap values so that each writes two columns of two of
// its four rows as one 4-byte word.
template <int N>
__device__ __forceinline__ void stage_out(char* buf, const f32x4 O[4], int cw, int li, int lq) {
    const bool odd = li & 1;
    uint32_t* os = reinterpret_cast<uint32_t*>(buf + kBufQ) + (cw >> 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const float mine = odd ? O[m][2 + e2] : O[m][e2];
            const float give = odd ? O[m][e2] : O[m][2 + e2];
            const float got = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(give), 0xB1, 0xF, 0xF, false));
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 pr = __builtin_convertvector(
                (f32x4{odd ? got : mine, odd ? mine : got, 0.f, 0.f}).xy, bf16x2);
            const int row = 16 * m + 4 * lq + (odd ? 2 + e2 : e2);
            os[row * (N / 2)] = __builtin_bit_cast(uint32_t, pr);
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

// Layout and memory-wave roles of the state kernel with NW compute waves
// (16 state columns each) and 8 - NW memory waves.  Wave w runs on SIMD
// w % 4.
//   K waves (m 0, 1)   K rows 0..31 / 32..63, wait, K^T granules 0..3 / 4..7
//   V waves            the slice's v front end, one 4-channel x 4-row item
//                      per lane (NW = 4: every memory wave; NW = 2: waves 6, 7,
//                      on the SIMDs without a compute wave)
//   copy waves         the other record pieces and the raw slab, round robin
//   every memory wave  first stores its O pieces of the previous chunk from
//                      the Q region it is about to refill, then refills
//                      those Q pieces itself
template <int NW>
struct StateShape {
    static constexpr int NM = 8 - NW;
    static constexpr int N = 16 * NW;                        // state columns per workgroup
    static constexpr int SPLIT = kD / N;
    static constexpr int BUF = kBufVt + N * kVtLd * 2;
    static constexpr int SLAB_ROW = N * 2;                   // raw v slab: [67 rows][N channels] bf16
    static constexpr int SLAB = (kC + 3) * SLAB_ROW;
    static constexpr int SLAB_PIECES = (SLAB + 1023) / 1024;
    static constexpr int O_PIECES = kC * N * 2 / 1024;       // O staged in Q pieces 0 .. O_PIECES - 1
    static constexpr int NV = NW == 4 ? 4 : 2;               // V waves
    static constexpr int OTHER = (16 - O_PIECES) + 12 + 2 + SLAB_PIECES;
    static constexpr int NCOPY = NW == 4 ? 4 : 4;            // copy waves: NW = 4: m 0..3; NW = 2: m 2..5
    __device__ static bool is_v(int m) { return NW == 4 || m >= 4; }
    __device__ static int v_part(int m) { return NW == 4 ? m : m - 4; }
    __device__ static int copy_index(int m) { return NW == 4 ? m : m - 2; }   // < 0: not a copy wave
};

// Copy piece pc of a chunk's raw v slab (first row at call-local token
// local0 - 3) into `slab`
template <int NW>
__device__ __forceinline__ void issue_slab(const PrefillParams& p, const StateCtx& cx, char* slab, int64_t local0,
                                           int pc, int lane) {
    using SS = StateShape<NW>;
    const int o = pc * 1024 + 16 * lane;
    if (o < SS::SLAB) {
        const int row = o / SS::SLAB_ROW, g = (o % SS::SLAB_ROW) / 16;
        const int64_t t = min(max(local0 - 3 + row, (int64_t)0), p.seq_len - 1);
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) + ((int64_t)cx.b * p.seq_len + t) * p.conv_dim +
                              2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + 8 * g;
        __builtin_amdgcn_global_load_lds(src, LDS_PTR(slab + pc * 1024), 16, 0, 0);
    }
}

// Front end of part `part` of the slice's v channels for one chunk from its
// raw slab -> V^T in the chunk's buffer.  Items of 4 channels x 4 rows, one
// per lane: N / 4 channel groups x 16 row groups, 64 items per part.
template <int NW, bool INTERIOR>
__device__ __forceinline__ void v_front(const PrefillParams& p, const StateCtx& cx, const float* Wv, const char* slab,
                                        char* buf, int64_t local0, int part, int lane) {
    using SS = StateShape<NW>;
    constexpr int CG = SS::N / 4;
    const int item = 64 * part + lane;
    const int c0 = (item % CG) * 4, tau0 = (item / CG) * 4;
    const int64_t gc = 2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + c0;
    uint2 raw[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) raw[k] = *reinterpret_cast<const uint2*>(slab + (tau0 + k) * SS::SLAB_ROW + 2 * c0);
    float w[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[t][i] = Wv[t * SS::N + c0 + i];
    bf16x4 ub[4];
    conv_compute<INTERIOR, 4>(p, cx.b, gc, local0, tau0, w, raw, ub);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<bf16x4*>(buf + kBufVt + ((c0 + i) * kVtLd + tau0) * 2) = bf16x4{ub[0][i], ub[1][i], ub[2][i], ub[3][i]};
}

// O piece o of chunk kc (staged in buf's Q region) -> HBM: 16 bytes per lane
template <int NW>
__device__ __forceinline__ void store_out_piece(const PrefillParams& p, const StateCtx& cx, const char* buf,
                                                int64_t kc, int o, int lane) {
    using SS = StateShape<NW>;
    const int off = o * 1024 + 16 * lane;
    const int row = off / (SS::N * 2), c8 = (off % (SS::N * 2)) / 16;
    const uint4 v = *reinterpret_cast<const uint4*>(buf + kBufQ + off);
    const int64_t t = kc * kC - p.start_pos + row;
    if (t >= 0 && t < p.seq_len)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) +
                                  (((int64_t)cx.b * p.seq_len + t) * p.num_v_heads + cx.h) * kD + cx.zcol0 + 8 * c8) = v;
}

// Checkpoint slot when the end of chunk kc is a multiple of the checkpoint
// interval: this compute wave's state slice and (over the compute threads)
// the conv tails of the workgroup's channels
template <int NW>
__device__ __forceinline__ void checkpoint(const PrefillParams& p, const StateCtx& cx, const f32x4 S[8], int64_t kc,
                                           int tid) {
    constexpr int NT = 64 * NW, NCH = 2 * kD + 16 * NW;
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

// Memory wave m's share of one chunk: store the O pieces of chunk jn - 2
// (staged in buf's Q region) and refill buf with chunk jn: records, raw slab
// of chunk jn + 1 into slab_next, v front end from `slab`, K^T.
template <int NW>
__device__ __forceinline__ void mem_chunk(const SplitParams& sp, const StateCtx& cx, const float* Wv, char* buf,
                                          const char* slab, char* slab_next, int jn, bool store_prev, int m, int lane) {
    using SS = StateShape<NW>;
    const bool fill = jn < sp.nseg;
    // O pieces of the chunk that last used this buffer, then the same Q pieces
    if (store_prev)
        for (int o = m; o < SS::O_PIECES; o += SS::NM) store_out_piece<NW>(sp.p, cx, buf, sp.k0 + jn - 2, o, lane);
    if (!fill) return;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the O rows are in registers before the buffer is refilled
    const char* krec = key_rec(sp, cx.b, cx.kh, jn);
    const char* vrec = val_rec(sp, cx.b, cx.h, jn);
    for (int o = m; o < SS::O_PIECES; o += SS::NM) issue_piece(buf, krec, vrec, o, lane);
    if (m < 2)
        for (int pc = kPiecesK + 8 * m; pc < kPiecesK + 8 * m + 8; ++pc) issue_piece(buf, krec, vrec, pc, lane);
    const int ci = SS::copy_index(m);
    if (ci >= 0) {
        for (int i = ci; i < SS::OTHER; i += SS::NCOPY) {
            // other pieces: Q pieces O_PIECES..15, P | AN, scale rows, then the next slab
            if (i < 16 - SS::O_PIECES) issue_piece(buf, krec, vrec, SS::O_PIECES + i, lane);
            else if (i < 16 - SS::O_PIECES + 14) issue_piece(buf, krec, vrec, kPiecesPA + (i - (16 - SS::O_PIECES)), lane);
            else if (jn + 1 < sp.nseg)
                issue_slab<NW>(sp.p, cx, slab_next, (sp.k0 + jn + 1) * kC - sp.p.start_pos, i - (30 - SS::O_PIECES), lane);
        }
    }
    if (SS::is_v(m)) {
        const int64_t local0 = (sp.k0 + jn) * kC - sp.p.start_pos;
        if (local0 >= 3 && local0 + kC <= sp.p.seq_len) v_front<NW, true>(sp.p, cx, Wv, slab, buf, local0, SS::v_part(m), lane);
        else v_front<NW, false>(sp.p, cx, Wv, slab, buf, local0, SS::v_part(m), lane);
    }
    if (m < 2) {
        __builtin_amdgcn_s_waitcnt(0);
        transpose_k(buf, 4 * m, lane);
    }
}

// Waves 0..NW-1 own 16 state columns each; waves NW..7 move data.  Per chunk
// two barriers: E (the chunk's products are done and the next chunk's buffer
// is filled) and B (the chunk's O rows are staged in its Q region).
template <int NW>
__global__ __launch_bounds__(512) void state_kernel(SplitParams sp) {
    using SS = StateShape<NW>;
    constexpr int N = SS::N, NCH = 2 * kD + N;
    const PrefillParams& p = sp.p;
    __shared__ __attribute__((aligned(16))) char buf0[SS::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[SS::BUF];
    __shared__ __attribute__((aligned(16))) char slab0[SS::SLAB];   // raw v slabs, per chunk parity
    __shared__ __attribute__((aligned(16))) char slab1[SS::SLAB];
    __shared__ float Wv[4 * N];                                     // conv taps of the slice's v channels

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: role branches stay scalar
    const int li = lane % 16, lq = lane / 16;
    const bool compute = wave < NW;
    // workgroup -> (b, key head, member); the r * SPLIT members of one
    // (b, key head) share a blockIdx % 8, so the round-robin dispatch puts
    // them on one XCD and its L2, where their common key records stay
    const int r = p.num_v_heads / p.num_k_heads;
    const int M = r * SS::SPLIT;
    const int NG = p.batch * p.num_k_heads;
    const int bid = blockIdx.x;
    const int grp = (bid / 8 / M) * 8 + bid % 8;
    const int member = (bid / 8) % M;
    if (grp >= NG) return;
    StateCtx cx;
    cx.b = grp / p.num_k_heads;
    cx.kh = grp % p.num_k_heads;
    cx.h = cx.kh * r + member / SS::SPLIT;
    cx.zcol0 = (member % SS::SPLIT) * N;
    cx.owns_qk_tail = member == 0;
    cx.s_base = ((int64_t)cx.b * p.num_v_heads + cx.h) * kD * kD + cx.zcol0 + 16 * (compute ? wave : 0) + li;

    for (int e = tid; e < 4 * N; e += 512) {
        const int t = e / N, c = e % N;
        const int64_t gc = 2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + c;
        Wv[e] = bf16_bits_to_f32(static_cast<const uint16_t*>(p.conv_w)[gc * 4 + t]);
    }
    __syncthreads();

    // The two roles run separate loops with the same barriers (two in the
    // prologue, two per chunk), so their registers do not add up.
    if (compute) {
        const float* s_src = sp.first_seg ? p.rec_in : p.rec_out;
        f32x4 S[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[t][e] = s_src ? s_src[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] : 0.f;
        __syncthreads();
        __syncthreads();
        const int cw = 16 * wave + li;
        for (int j = 0; j < sp.nseg; ++j) {
            char* cur = (j & 1) ? buf1 : buf0;
            bf16x4 vv[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                vv[mb] = *reinterpret_cast<const bf16x4*>(cur + kBufVt + (cw * kVtLd + 16 * mb + 4 * lq) * 2);
            f32x4 QS[4], O[4];
            bf16x8 BD[2];
            state_products(cur, S, vv, QS, BD, li, lq);
            out_tile(cur, QS, BD, O, li, lq);
            // finish O before E (the compiler would otherwise sink it past
            // the barrier, where the memory waves wait for it)
            asm volatile("" ::"v"(O[0]), "v"(O[1]), "v"(O[2]), "v"(O[3]));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();   // E
            stage_out<N>(cur, O, cw, li, lq);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();   // B
            checkpoint<NW>(p, cx, S, sp.k0 + j, tid);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.rec_out[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
    } else {
        const int m = wave - NW;
        // raw slab of chunk 0, then chunk 0 into buf0 (and chunk 1's slab)
        if (sp.nseg > 0)
            for (int pc = m; pc < SS::SLAB_PIECES; pc += SS::NM) issue_slab<NW>(p, cx, slab0, sp.k0 * kC - p.start_pos, pc, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        mem_chunk<NW>(sp, cx, Wv, buf0, slab0, slab1, 0, false, m, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // Step j: store O of chunk j - 1 from the other buffer and refill it
        // with chunk j + 1.  Two chunks per trip so that each LDS buffer is a
        // distinct object: the compiler then orders reads of one buffer only
        // after its own copies.  Chunk c's slab lives in slab[c % 2].
        for (int j = 0; j < sp.nseg; j += 2) {
            mem_chunk<NW>(sp, cx, Wv, buf1, slab1, slab0, j + 1, j >= 1, m, lane);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();   // E
            __syncthreads();   // B
            if (j + 1 < sp.nseg) {
                mem_chunk<NW>(sp, cx, Wv, buf0, slab0, slab1, j + 2, true, m, lane);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();   // E
                __syncthreads();   // B
            }
        }
        // O of the last chunk
        if (sp.nseg > 0) {
            const char* last = ((sp.nseg - 1) & 1) ? buf1 : buf0;
            for (int o = m; o < SS::O_PIECES; o += SS::NM) store_out_piece<NW>(p, cx, last, sp.k0 + sp.nseg - 1, o, lane);
        }
    }
    if (sp.last_seg) {
        for (int ch = tid; ch < NCH; ch += 512)
            if (ch >= 2 * kD || cx.owns_qk_tail)
                write_tail(p, cx.b, p.seq_len, state_channel(p, cx, ch), static_cast<uint16_t*>(p.conv_out));
    }
}

template <int NW>
hipError_t launch_state(const SplitParams& sp, hipStream_t stream) {
    const int r = sp.p.num_v_heads / sp.p.num_k_heads;
    const int ng = sp.p.batch * sp.p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * StateShape<NW>::SPLIT;
    hipLaunchKernelGGL((state_kernel<NW>), dim3(blocks), dim3(512), 0, stream, sp);
    return hipGetLastError();
}

// Compute waves per state workgroup (16 state columns each).  A workgroup
// streams its chunk records at a bounded rate per CU, so with few
// (sequence, head) pairs the narrower workgroups spread the chains over more
// CUs; with many, the wider ones do more work per byte moved.
// GDN_PREFILL_STATE_WAVES (2 or 4) overrides the choice.
int state_waves(const PrefillParams& p) {
    if (const char* env = getenv("GDN_PREFILL_STATE_WAVES")) {
        const int v = atoi(env);
        if (v == 2 || v == 4) return v;
    }
    const int64_t heads = (int64_t)p.batch * p.num_v_heads;
    return heads * 4 <= 256 ? 2 : 4;
}

hipError_t launch_state_any(const SplitParams& sp, hipStream_t stream) {
    return state_waves(sp.p) == 4 ? launch_state<4>(sp, stream) : launch_state<2>(sp, stream);
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
    SplitParams sp{};
    sp.p = p;
    sp.ws = static_cast<char*>(ws);
    sp.first_seg = 1;
    if (k_end == k_first) {
        sp.k0 = k_first;
        sp.nseg = 0;
        sp.last_seg = 1;
        return launch_state_any(sp, stream);
    }
    for (int64_t k0 = k_first; k0 < k_end; k0 += max_seg) {
        const int64_t n = k_end - k0 < max_seg ? k_end - k0 : max_seg;
        sp.k0 = k0;
        sp.nseg = (int32_t)n;
        sp.last_seg = k0 + n == k_end;
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(p.batch * p.num_k_heads * n)), dim3(kPrepThreads), 0, stream, sp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_state_any(sp, stream);
        if (e != hipSuccess) return e;
        sp.first_seg = 0;
    }
    return hipSuccess;
}

}  // namespace gdn
