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
//         Delta by blocked forward substitution, the state update, O, which
//         they store straight from registers -- while 8 - NW memory waves
//         fill the LDS buffers of the next chunks (three buffers, records
//         requested two chunks ahead, where LDS allows; two otherwise): the
//         records by global_load_lds and the front end of the slice's v
//         channels (conv + SiLU from a raw slab the same wave copied ahead;
//         the slice's own columns, so no value-head data goes through the
//         workspace).  K^T is read from K with the transposing LDS reads.
//
// A workspace smaller than the whole call is used segment by segment (prep
// then state for each run of chunks that fits); the state travels between
// segments through rec_state_out.  Every value the state kernel consumes is
// bit-identical to what the fused kernel computes in LDS, so the two paths
// agree to the last bit up to the compiler's instruction choice.
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "gdn_chunk_common.h"

namespace gdn {

namespace {

using namespace chunked;

// P and AN hold only their lower triangle of 16x16 tiles: rows 0..31 keep
// granules 0..3 (64-byte rows), rows 32..63 all eight (128-byte rows).
// Granules are XOR-swizzled so that eight consecutive rows read by one phase
// of an LDS read hit eight different bank groups.  The value records store
// them in exactly this layout, so the state kernel copies them unchanged.
constexpr int kPaMat = 32 * 64 + 32 * 128;          // 6144 bytes per matrix
__device__ __forceinline__ int pa_off(int mat, int row, int g) {
    return mat * kPaMat + (row < 32 ? row * 64 + 16 * (g ^ ((row >> 1) & 3))
                                    : 2048 + (row - 32) * 128 + 16 * (g ^ (row & 7)));
}
// the inverse: byte l (a multiple of 16) of one matrix's layout holds row
// `row`, granule g (8 pos()-ordered columns)
__device__ __forceinline__ void pa_granule(int l, int& row, int& g) {
    if (l < 2048) {
        row = l >> 6;
        g = ((l >> 4) & 3) ^ ((row >> 1) & 3);
    } else {
        row = 32 + ((l - 2048) >> 7);
        g = ((l >> 4) & 7) ^ (row & 7);
    }
}

// ---- workspace records.  Q and K are row-major, columns in pos() order,
// unpadded.  Key record (sequence, key head, chunk): Q | K.  Value record
// (sequence, value head, chunk): P | AN (lower tiles, the layout above) |
// five rows of 64 fp32 (beta | beta Gamma n_k | Gamma n_q |
// exp(gamma_C - gamma) n_k | exp(gamma_C), 0, ...).
constexpr int kRecQ = 0;
constexpr int kRecK = kC * kD * 2;
constexpr int kKeyRec = 2 * kC * kD * 2;            // 32768
constexpr int kRecP = 0;
constexpr int kRecAN = kPaMat;
constexpr int kRecTok = 2 * kPaMat;
constexpr int kTokBytes = 5 * kC * 4;
constexpr int kValRec = kRecTok + kTokBytes;        // 13568
// precise mode (bf16 hi + lo operands): the rows of scales take a 2 KiB slot
// and the lo parts of P and AN follow, so that the whole value record has the
// layout of its LDS image
constexpr int kRecPlo = kRecTok + 2048;
constexpr int kValRecHL = kRecPlo + 2 * kPaMat;     // 26624
static_assert(kKeyRec % 256 == 0 && kValRec % 256 == 0 && kValRecHL % 256 == 0,
              "records keep 256-byte alignment");
constexpr int val_rec_bytes(bool precise) { return precise ? kValRecHL : kValRec; }

constexpr int kMaxGroup = 8;                        // value heads per key head on this path

struct SplitParams {
    PrefillParams p;
    char* ws;
    int32_t vrec_bytes;  // bytes of a value record (val_rec_bytes(p.precise))
    int64_t k0;          // absolute index of the segment's first chunk
    int32_t nseg;        // chunks in the segment
    int32_t first_seg;   // state comes from rec_in (else from rec_out)
    int32_t last_seg;    // write the final conv tail
    int32_t rec_stride;  // chunk records per (sequence, head) in the workspace
    int32_t rec_batch;   // sequences with records in the workspace
    int32_t pj;          // chunks per (sequence, key head) in a prep grid
    // Overlapped prep (null flags: off).  The prep launch on the caller's
    // stream covers chunks [0, n1); prep_kernel_tail publishes chunks n1..
    // one by one, concurrently with that launch and with the state kernel,
    // which waits for each chunk's flag.  Flags, claim counters and error
    // words carry the call's epoch, so nothing has to be cleared between
    // calls.
    uint64_t* flags;     // [B H_k][frow]: the epoch once a chunk's records are complete
    uint64_t* hdr;       // kOvlHdrWords: epoch-tagged claim counters per XCD, error words
    uint64_t epoch;      // this call's tag, never 0
    int32_t frow;        // flag words per row (a multiple of 32)
    int32_t n1;
    uint64_t wait_ticks; // bound of one wait, in ticks of the 100 MHz s_memrealtime clock
};

// ---- overlap header (64-bit word offsets; each XCD's counter on a 256-byte
// line of its own).  A counter holds a 40-bit epoch tag and a 24-bit count.
// An error word holds the epoch of the call that met the error: kHdrErrXcd
// an XCD id out of range, kHdrErrClaim more state workgroups on an XCD than
// its share of the work, kHdrErrWait a wait for a chunk that timed out.
constexpr int kOvlHdrWords = 1024;
constexpr int kHdrState = 0, kHdrPrep = 256, kHdrErrXcd = 512, kHdrErrClaim = 544, kHdrErrWait = 576;
constexpr int kOvlXcds = 8;
// persistent tail workgroups: as many as the tail stream's 64 CUs hold at
// once (two per CU; one in the precise mode, whose prep takes the LDS of two)
constexpr int ovl_tail_blocks(bool precise) { return precise ? 64 : 128; }

// The count before this claim of an epoch-tagged counter (0 for the call's
// first claim, whatever an earlier call left there)
__device__ __forceinline__ uint32_t claim_next(uint64_t* ctr, uint64_t epoch) {
    const uint64_t tag = (epoch & 0xffffffffffull) << 24;
    uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const bool cur = (old & ~0xffffffull) == tag;
        uint64_t seen = old;
        if (__hip_atomic_compare_exchange_strong(ctr, &seen, cur ? old + 1 : tag + 1, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return cur ? (uint32_t)(old & 0xffffff) : 0u;
        old = seen;
    }
}

__device__ __forceinline__ void ovl_error(uint64_t* hdr, int word, uint64_t epoch) {
    __hip_atomic_store(hdr + word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// XCD (accelerator complex die) of the calling wave, from the XCC_ID
// hardware register: the workgroups that share one XCD share its L2
__device__ __forceinline__ unsigned xcd_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)); }

// Records of record-sequence rb (the sequence's index among those of the
// launch), head and chunk j of the segment
__device__ __forceinline__ char* key_rec(const SplitParams& s, int rb, int kh, int j) {
    return s.ws + (((int64_t)rb * s.p.num_k_heads + kh) * s.rec_stride + j) * kKeyRec;
}

__device__ __forceinline__ char* val_rec(const SplitParams& s, int rb, int h, int j) {
    return s.ws + (int64_t)s.rec_batch * s.p.num_k_heads * s.rec_stride * kKeyRec +
           (((int64_t)rb * s.p.num_v_heads + h) * s.rec_stride + j) * s.vrec_bytes;
}

// ---- sequences of different lengths and start positions in one call
// (token-packed inputs and outputs, cu_seqlens).  One launch covers up to
// kVarlenGroup sequences, described in its kernel arguments; a segment is a
// run of chunks at the same offset j0 from each sequence's first chunk.
constexpr int kVarlenGroup = 64;

struct SeqDesc {
    int64_t tok0;    // first token of the sequence in the packed arrays
    int64_t start;   // absolute position of that token
    int64_t len;     // tokens of the sequence in this call
};

struct VarlenParams {
    SplitParams sp;      // shared fields; per-sequence ones come from seq[]
    int64_t j0;          // the segment's first chunk, relative to each sequence's first
    int32_t b0, nb;      // sequences b0 .. b0 + nb - 1 of the call
    SeqDesc seq[kVarlenGroup];
};

// The view of sequence b (entry i of the launch) as a one-sequence-per-row
// call: token-indexed pointers are shifted so that the kernels' row index
// b * len + t lands on token tok0 + t; state, conv-state and checkpoint
// arrays keep their index b.
__device__ __forceinline__ SplitParams seq_view(const VarlenParams& v, int i, int b) {
    SplitParams s = v.sp;
    const SeqDesc d = v.seq[i];
    const int64_t kf = d.start / kC;
    const int64_t n = d.len > 0 ? (d.start + d.len - 1) / kC + 1 - kf : 0;
    const int64_t shift = d.tok0 - (int64_t)b * d.len;
    const PrefillParams& p = v.sp.p;
    s.p.qkv = static_cast<const uint16_t*>(p.qkv) + shift * p.conv_dim;
    s.p.a = static_cast<const uint16_t*>(p.a) + shift * p.num_v_heads;
    s.p.b = static_cast<const uint16_t*>(p.b) + shift * p.num_v_heads;
    s.p.out = static_cast<uint16_t*>(p.out) + shift * p.num_v_heads * kD;
    s.p.seq_len = d.len;
    s.p.start_pos = d.start;
    s.k0 = kf + v.j0;
    const int64_t left = n - v.j0;
    s.nseg = left <= 0 ? 0 : (int32_t)(left < v.sp.rec_stride ? left : v.sp.rec_stride);
    s.first_seg = v.j0 == 0;
    s.last_seg = v.j0 + v.sp.rec_stride >= n;
    return s;
}

// Byte offset of 16-byte granule g of row `row` in the state kernel's LDS
// copy of a 256-byte-row matrix (Q, K): the granule index is XORed with
// row % 16, so the sixteen rows read by one phase of a ds_read_b128 hit
// sixteen different granule columns, and so do the sixteen rows of one
// transposing read of K (four lanes per row, granules 4u + 0..3).
__device__ __forceinline__ int swz256(int row, int g) { return row * 256 + 16 * (g ^ (row & 15)); }

__device__ __forceinline__ void copy16(char* dst, const void* src) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// ============================================================ prep kernel
constexpr int kPrepWaves = 8;
constexpr int kPrepThreads = 64 * kPrepWaves;

// One value head's masked matrices, diagonal blocks and row scales (and in
// the precise mode the lo parts of P and AN).
template <bool PRECISE>
struct alignas(16) PrepHeadBuf {
    static constexpr int LO = PRECISE ? kC * kKtLd : 8;
    __bf16 Ps[kC * kKtLd];
    __bf16 AN[kC * kKtLd];
    float AdT[4 * 16 * kXLd];
    float tokS[5][kC];
    __bf16 Ps_lo[LO];
    __bf16 AN_lo[LO];
};

// Q and K are dead once their record is written and the Gram tiles are in
// registers, so a second head buffer shares their space: one value head is
// solved while the next one's masks are formed.
template <bool PRECISE>
struct alignas(16) PrepSmem {
    union {
        struct {
            __bf16 Qs[kC * kKsLd];
            __bf16 Ks[kC * kKsLd];
        };
        PrepHeadBuf<PRECISE> hb1;
    };
    PrepHeadBuf<PRECISE> hb0;
    alignas(16) float beta[kMaxGroup][kC];   // per value head of the group
    alignas(16) float gam[kMaxGroup][kC];
    alignas(16) float nq[kC];
    alignas(16) float nk[kC];
    uint16_t Ws[4 * 2 * kD];   // conv taps (bf16 bits) [tap][channel]: q, then k
};
static_assert(sizeof(PrepHeadBuf<false>) <= 2 * kC * kKsLd * 2, "the second head buffer fits in Q and K");
static_assert(sizeof(PrepSmem<false>) <= 160 * 1024 / 2, "two prep workgroups per CU");

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
    __bf16* Ps_lo;
    __bf16* AN_lo;
};

// Global channel of prep channel index ch: q then k of key head kh
__device__ __forceinline__ int64_t qk_channel(int ch, int kh, int Hk) {
    return ch < kD ? (int64_t)kh * kD + ch : (int64_t)Hk * kD + (int64_t)kh * kD + ch - kD;
}

// Front end of the q, k channels of a chunk -> LDS rows (4 channels x 8 rows
// per item, one item per thread).  The raw rows are loaded first (by
// prep_front_load, at the start of the kernel, so that their latency
// overlaps the set-up), the conv runs once the taps are in LDS.
static_assert(2 * kD / 4 * 8 == kPrepThreads, "one front-end item per thread");

__device__ __forceinline__ void prep_front_load(const PrefillParams& p, int b, int kh, int64_t local0, bool interior,
                                                int tid, uint2 raw[11]) {
    const int ch0 = (tid % 64) * 4, tau0 = (tid / 64) * 8;
    const int64_t gc = qk_channel(ch0, kh, p.num_k_heads);
    if (interior) conv_load<true>(p, b, gc, local0, tau0, raw);
    else conv_load<false>(p, b, gc, local0, tau0, raw);
}

template <bool INTERIOR, class SMEM>
__device__ __forceinline__ void prep_front(const PrefillParams& p, SMEM& sm, int b, int kh, int64_t local0,
                                           int tid, const uint2 raw[11]) {
    const int ch0 = (tid % 64) * 4, tau0 = (tid / 64) * 8;
    const int64_t gc = qk_channel(ch0, kh, p.num_k_heads);
    float w[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) unpack_bf16x4(*reinterpret_cast<const uint2*>(&sm.Ws[t * 2 * kD + ch0]), w[t]);
    bf16x4 ub[8];
    conv_compute<INTERIOR>(p, b, gc, local0, tau0, w, raw, ub);
    __bf16* dst0 = ch0 < kD ? &sm.Qs[pos(ch0)] : &sm.Ks[pos(ch0 - kD)];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) *reinterpret_cast<bf16x4*>(dst0 + (tau0 + tt) * kKsLd) = ub[tt];
}

// Zero the upper tiles of a head buffer's P and AN (the masks never write
// them) and the unused part of its fifth row of scales.
template <bool PRECISE>
__device__ __forceinline__ void zero_upper(PrepHeadBuf<PRECISE>& hb, int tid) {
    for (int e = tid; e < 6 * 256; e += kPrepThreads) {
        const int t6 = e / 256, rr = (e / 16) % 16, cc = e % 16;
        const int m = t6 < 3 ? 0 : (t6 < 5 ? 1 : 2);
        const int pp = t6 < 3 ? t6 + 1 : (t6 < 5 ? t6 - 1 : 3);
        const int o = (16 * m + rr) * kKtLd + pos(16 * pp + cc);
        hb.Ps[o] = __bf16(0.f);
        hb.AN[o] = __bf16(0.f);
        if constexpr (PRECISE) {
            hb.Ps_lo[o] = __bf16(0.f);
            hb.AN_lo[o] = __bf16(0.f);
        }
    }
    if (tid < kC) hb.tokS[4][tid] = 0.f;
}

// Chunk j of the segment for sequence b (record-sequence rb) and key head kh
template <bool NEUMANN, bool PRECISE>
__device__ __forceinline__ void prep_body(const SplitParams& sp, int b, int rb, int kh, int j, int tid) {
    const PrefillParams& p = sp.p;
    using HB = PrepHeadBuf<PRECISE>;
    __shared__ PrepSmem<PRECISE> sm;
    // wave index in a scalar register: branches on it are uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
    const int li = lane % 16, lq = lane / 16;
    const int Hk = p.num_k_heads, r = p.num_v_heads / Hk;
    const int64_t local0 = (sp.k0 + j) * kC - p.start_pos;
    char* krec = key_rec(sp, rb, kh, j);
    const bool interior = local0 >= 3 && local0 + kC <= p.seq_len;
    uint2 raw[11];
    prep_front_load(p, b, kh, local0, interior, tid, raw);

    // ---- set-up: gates of every value head of the group (wave hh: head
    // kh r + hh); conv taps -> LDS; the first head buffer's zeros
    if (wave < r) {
        const int h = kh * r + wave;
        gates_scan(p, b, h, -expf(p.A_log[h]), p.dt_bias[h], local0, lane, sm.gam[wave], sm.beta[wave]);
    }
    for (int e = tid; e < 2 * kD * 4; e += kPrepThreads) {
        const int ch = e % (2 * kD), tap = e / (2 * kD);
        sm.Ws[e] = static_cast<const uint16_t*>(p.conv_w)[qk_channel(ch, kh, Hk) * 4 + tap];
    }
    zero_upper(sm.hb0, tid);
    __syncthreads();

    // ---- front end of q, k
    if (interior) prep_front<true>(p, sm, b, kh, local0, tid, raw);
    else prep_front<false>(p, sm, b, kh, local0, tid, raw);
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
    // The K K^T and Q K^T tiles of the ten lower tile pairs stay in the
    // registers of the waves that mask them.  Substitution: waves 1..7 hold
    // pairs wave - 1, waves 1..3 also pairs wave + 6, and wave 0, which
    // solves, none.  Neumann product (solved by waves 0..3): wave w holds
    // pair w, waves 0, 1 also pair w + 8.
    const bool has0 = NEUMANN || wave >= 1;
    const bool has1 = NEUMANN ? wave < 2 : (wave >= 1 && wave <= 3);
    const int pa0 = NEUMANN ? wave : wave - 1, pa1 = NEUMANN ? wave + 8 : wave + 6;
    f32x4 gk[2], gq[2];
    if (has0) {
        gk[0] = gram_tile(sm.Ks, sm.Qs, pa0, li, lq);
        gq[0] = gram_tile(sm.Ks, sm.Qs, 10 + pa0, li, lq);
    }
    if (has1) {
        gk[1] = gram_tile(sm.Ks, sm.Qs, pa1, li, lq);
        gq[1] = gram_tile(sm.Ks, sm.Qs, 10 + pa1, li, lq);
    }
    __syncthreads();

    auto view = [&](int hh, HB& hb) {
        return PrepHeadView{sm.gam[hh], sm.beta[hh], sm.nq, sm.nk, hb.Ps, hb.AN, hb.AdT, hb.tokS, hb.Ps_lo, hb.AN_lo};
    };
    // masks and row scales of value head hh of the group into a head buffer
    auto mask_head = [&](int hh, HB& hb) {
        PrepHeadView hv = view(hh, hb);
        if (has0) mask_pair<PRECISE>(hv, pa0, gk[0], gq[0], lane);
        if (has1) mask_pair<PRECISE>(hv, pa1, gk[1], gq[1], lane);
        if (wave == kPrepWaves - 1) {
            row_scales(hv, lane);
            if (lane == 0) hb.tokS[4][0] = expf(sm.gam[hh][kC - 1]);
        }
    };
    // P and the row scales of a head buffer -> value record (granules e0,
    // e0 + stride, ...), and AN; in the precise mode their lo parts too
    constexpr int kPaGran = kPaMat / 16;
    auto copy_p_tok = [&](char* vrec, const HB& hb, int e0, int stride) {
        for (int e = e0; e < kPaGran + kTokBytes / 16; e += stride) {
            if (e < kPaGran) {
                int row, g;
                pa_granule(16 * e, row, g);
                copy16(vrec + kRecP + 16 * e, hb.Ps + row * kKtLd + 8 * g);
                if constexpr (PRECISE) copy16(vrec + kRecPlo + 16 * e, hb.Ps_lo + row * kKtLd + 8 * g);
            } else {
                copy16(vrec + kRecTok + 16 * (e - kPaGran), &hb.tokS[0][0] + 4 * (e - kPaGran));
            }
        }
    };
    auto copy_an = [&](char* vrec, const HB& hb, int e0, int stride) {
        for (int e = e0; e < kPaGran; e += stride) {
            int row, g;
            pa_granule(16 * e, row, g);
            copy16(vrec + kRecAN + 16 * e, hb.AN + row * kKtLd + 8 * g);
            if constexpr (PRECISE) copy16(vrec + kRecPlo + kPaMat + 16 * e, hb.AN_lo + row * kKtLd + 8 * g);
        }
    };

    if (NEUMANN) {
        // per value head: masks, then the diagonal inverses on waves 0..3
        // while waves 4..7 copy P and the row scales, then AN
        for (int hh = 0; hh < r; ++hh) {
            char* vrec = val_rec(sp, rb, kh * r + hh, j);
            mask_head(hh, sm.hb0);
            __syncthreads();
            if (wave < 4) {
                PrepHeadView hv = view(hh, sm.hb0);
                diag_neumann<PRECISE>(hv, wave, lane);
            } else {
                copy_p_tok(vrec, sm.hb0, tid - 256, kPrepThreads - 256);
            }
            __syncthreads();
            copy_an(vrec, sm.hb0, tid, kPrepThreads);
            if (hh + 1 < r) __syncthreads();
        }
    } else {
        // software pipeline over the value heads, one barrier per head: wave
        // 0 solves head hh's diagonal blocks and copies its AN, while waves
        // 1..7 copy its P and row scales and form head hh + 1's masks in the
        // other buffer
        zero_upper(sm.hb1, tid);
        mask_head(0, sm.hb0);
        __syncthreads();
        for (int hh = 0; hh < r; ++hh) {
            HB& cur = hh & 1 ? sm.hb1 : sm.hb0;
            HB& nxt = hh & 1 ? sm.hb0 : sm.hb1;
            char* vrec = val_rec(sp, rb, kh * r + hh, j);
            if (wave == 0) {
                PrepHeadView hv = view(hh, cur);
                diag_solve<true, PRECISE>(hv, lane);
                // this wave's own LDS writes are read back in order; keep the
                // compiler from moving the reads above them
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
                copy_an(vrec, cur, lane, 64);
            } else {
                copy_p_tok(vrec, cur, tid - 64, kPrepThreads - 64);
                if (hh + 1 < r) mask_head(hh + 1, nxt);
            }
            if (hh + 1 < r) __syncthreads();
        }
    }
}

template <bool NEUMANN, bool PRECISE>
__global__ __launch_bounds__(kPrepThreads)
void prep_kernel(SplitParams sp) {
    const int j = blockIdx.x % sp.pj;
    const int grp = blockIdx.x / sp.pj;
    const int b = grp / sp.p.num_k_heads, kh = grp % sp.p.num_k_heads;
    prep_body<NEUMANN, PRECISE>(sp, b, b, kh, j, threadIdx.x);
}

// Tail of an overlapped call: persistent workgroups, as many as the tail
// stream's CUs hold at once (so none waits to be dispatched, and nothing
// dispatched after them waits behind them).  A workgroup takes the next item
// -- (group, chunk) of chunks n1.. -- of its own XCD, groups g with
// g % 8 == XCD, chunks in order, so that the state workgroups of the group,
// on the same XCD, read its records from the L2 they were written to.  Once
// every record store of an item has completed, its flag is set.
template <bool NEUMANN, bool PRECISE>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(PRECISE ? 2 : 4, PRECISE ? 2 : 4)))
void prep_kernel_tail(SplitParams sp) {
    __shared__ int next_item;
    const int tid0 = threadIdx.x;
    const unsigned x = xcd_id();
    if (x >= kOvlXcds) {
        if (tid0 == 0) ovl_error(sp.hdr, kHdrErrXcd, sp.epoch);
        return;
    }
    const int Hk = sp.p.num_k_heads, gx = sp.p.batch * Hk / kOvlXcds;
    const int items = gx * (sp.nseg - sp.n1);
    uint64_t* ctr = sp.hdr + kHdrPrep + 32 * x;
    if (tid0 == 0) next_item = (int)claim_next(ctr, sp.epoch);
    __syncthreads();
    int t = next_item;
    while (t < items) {
        // the thread index, opaque per item: the compiler cannot keep the
        // body's per-lane addresses live across the loop
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        int nxt = 0;
        if (tid0 == 0) nxt = (int)claim_next(ctr, sp.epoch);   // the next claim, during this item
        const int c = sp.n1 + t / gx, grp = (int)x + kOvlXcds * (t % gx);
        prep_body<NEUMANN, PRECISE>(sp, grp / Hk, grp / Hk, grp % Hk, c, tid);
        __builtin_amdgcn_s_waitcnt(0);   // this thread's record stores have completed
        __syncthreads();                 // ... and every other thread's
        if (tid0 == 0) {
            __hip_atomic_store(sp.flags + (int64_t)grp * sp.frow + c, sp.epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            next_item = nxt;
        }
        __syncthreads();
        t = next_item;
    }
}

// Varlen: blockIdx = (entry i, key head, chunk j of the segment); entries
// whose sequence has fewer chunks left leave at once
template <bool NEUMANN, bool PRECISE>
__global__ __launch_bounds__(kPrepThreads)
void prep_kernel_varlen(VarlenParams vp) {
    const int j = blockIdx.x % vp.sp.rec_stride;
    const int grp = blockIdx.x / vp.sp.rec_stride;
    const int i = grp / vp.sp.p.num_k_heads, kh = grp % vp.sp.p.num_k_heads;
    const SplitParams sp = seq_view(vp, i, vp.b0 + i);
    if (j >= sp.nseg) return;
    prep_body<NEUMANN, PRECISE>(sp, vp.b0 + i, i, kh, j, threadIdx.x);
}

// ============================================================ state kernel
// LDS pointer from a generic pointer into LDS by its low 32 bits (the LDS
// offset): no address-space cast, whose null check costs a compare and a
// select per copy

// LDS pointer from a generic pointer into LDS by its low 32 bits (the LDS
// offset): no address-space cast, whose null check costs a compare and a
// select per copy
#define LDS_PTR(x) ((__attribute__((address_space(3))) void*)(uintptr_t)(uint32_t)(uintptr_t)(x))

// LDS buffer of one chunk: Q | K | P | AN | rows [| P_lo | AN_lo] | V^T (V^T
// of the slice's columns, row stride kVtLd; the lo parts of P and AN in the
// precise mode only).  K^T is read from K by transposing LDS reads.
constexpr int kVtLd = kC + 4;                       // bf16 row stride of V^T (conflict-free column reads)
constexpr int kBufQ = 0, kBufK = kC * kD * 2, kBufPA = 2 * kC * kD * 2,
              kBufTok = kBufPA + 2 * kPaMat, kBufPAlo = kBufTok + 2048;
constexpr int buf_vt(bool precise) { return precise ? kBufPAlo + 2 * kPaMat : kBufTok + kTokBytes; }
static_assert(kBufPA % 1024 == 0 && kBufTok % 1024 == 0 && kBufPAlo % 1024 == 0 && kBufTok + kTokBytes <= kBufPAlo,
              "piece and row alignment");
static_assert(kBufTok - kBufPA == kRecTok && kBufPAlo - kBufPA == kRecPlo && kRecP == 0,
              "a value record is the LDS image from kBufPA on");

// Record copies of one chunk: 1 KiB pieces, one wave-wide
// global_load_lds_dwordx4 each.  Pieces 0..15: Q, 16..31: K (256-byte rows),
// 32..43: P | AN triangles, 44..45: the rows of scales (1280 bytes, padded
// to 2 KiB in the precise mode); in the precise mode 46..57: the lo parts of
// P | AN.
constexpr int kPiecesK = 16, kPiecesPA = 32, kPiecesLo = 46;
constexpr int num_pieces(bool precise) { return precise ? kPiecesLo + 12 : kPiecesLo; }

template <bool PRECISE>
__device__ __forceinline__ void issue_piece(char* lds, const char* krec, const char* vrec, int pc, int lane) {
    const char* src;
    int dst;
    bool act = true;
    if (pc < kPiecesPA) {
        const int o = (pc & 15) * 1024 + 16 * lane;   // offset inside Q or K
        const int row = o >> 8, s = (o >> 4) & 15;
        src = krec + (pc < kPiecesK ? kRecQ : kRecK) + swz256(row, s);
        dst = (pc < kPiecesK ? kBufQ : kBufK) + o;
    } else {
        // the value record is the image of LDS from kBufPA on
        const int o = (pc - kPiecesPA) * 1024 + 16 * lane;
        act = PRECISE || o < kRecTok + kTokBytes;
        src = vrec + o;
        dst = kBufPA + o;
    }
    if (act) __builtin_amdgcn_global_load_lds(src, LDS_PTR(lds + (dst & ~1023)), 16, 0, 0);
}

// A-operand fragment of K^T (rows d_k 16t..16t+15, reduction slots of token
// block ks) straight from the row-major K by two ds_read_b64_tr_b16: in each
// group of 16 lanes, lane j reads d_k columns 16t + 4(j % 4) + 0..3 of token
// row 32ks + 16h + 4q + j / 4 (q = lane group, h = half), and the read hands
// lane i of the group column 16t + i of those four rows -- tokens
// 32ks + 4q + 0..3 and 32ks + 16 + 4q + 0..3, the slot order of pos().
// Four consecutive d_k columns sit in one half (8 bytes) of a granule:
// granule 4(t / 2) + j % 4, half t % 2.
__device__ __forceinline__ bf16x8 kt_frag(const char* buf, int t, int ks, int li, int lq) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    bf16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int row = 32 * ks + 16 * hh + 4 * lq + li / 4;
        const int off = kBufK + swz256(row, 4 * (t / 2) + li % 4) + 8 * (t % 2);
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + off));
    }
    return cat4(h[0], h[1]);
}

__device__ __forceinline__ bf16x8 ld8(const char* buf, int off) { return *reinterpret_cast<const bf16x8*>(buf + off); }
__device__ __forceinline__ bf16x4 ld4(const char* buf, int off) { return *reinterpret_cast<const bf16x4*>(buf + off); }
__device__ __forceinline__ f32x4 ldf4(const char* buf, int off) { return *reinterpret_cast<const f32x4*>(buf + off); }

// One chunk for this wave's 16 state columns: K S0, R = beta V - beta
// Gamma n_k (K S0), Delta by blocked substitution with (Q S0)^T in its
// latency, O^T = (Q S0)^T diag(Gamma n_q) + (P Delta)^T (bf16 into Ob), then
// the state update S <- exp(gamma_C) S + K^T Delta' (Delta' as bf16 hi +
// lo).  Lane (i, q) of O tile m holds token 16m + i, columns 4q..4q+3: a
// transposed tile comes from the same operand registers with A and B
// swapped.  LDS operands are requested well ahead of their use: K and the
// substitution's operands first, Q and P next, the K^T fragments of two
// state tiles as each Q tile is retired.  store_prev() (the previous chunk's
// O stores) runs inside the substitution, where the wave mostly waits.
template <class StorePrev>
__device__ __forceinline__ void chunk_products(const char* buf, f32x4 S[8], const bf16x4 vv[4], bf16x4 Ob[4], int li,
                                               int lq, StorePrev&& store_prev) {
    // batch 1: K fragments, the row scales of R (this lane's rows
    // 16m + 4lq + e) and the substitution's A-operand slots (token block k
    // of an AN row sits in granule 4 (k / 2) + lq, half k % 2)
    bf16x8 ak[4][4], aq[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ak[m][ks] = ld8(buf, kBufK + swz256(16 * m + li, 4 * ks + lq));
    f32x4 sb[4], sr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = 16 * m + 4 * lq;
        sb[m] = ldf4(buf, kBufTok + 4 * (0 * kC + r0));
        sr[m] = ldf4(buf, kBufTok + 4 * (1 * kC + r0));
    }
    const char* an = buf + kBufPA;
    const bf16x4 dg[4] = {ld4(an, pa_off(1, li, lq)), ld4(an, pa_off(1, 16 + li, lq) + 8),
                          ld4(an, pa_off(1, 32 + li, 4 + lq)), ld4(an, pa_off(1, 48 + li, 4 + lq) + 8)};
    const bf16x4 a10 = ld4(an, pa_off(1, 16 + li, lq));
    const bf16x8 a2x = ld8(an, pa_off(1, 32 + li, lq));
    const bf16x8 a3x = ld8(an, pa_off(1, 48 + li, lq));
    const bf16x4 a32 = ld4(an, pa_off(1, 48 + li, 4 + lq));
    bf16x8 Bs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Bs[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
    __builtin_amdgcn_sched_barrier(0);
    // K S0 with the four row tiles' accumulation chains interleaved
    f32x4 KS[4], R[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) KS[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int m = 0; m < 4; ++m) KS[m] = mfma16(ak[m][ks], Bs[ks], KS[m]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) R[m][e] = sb[m][e] * float(vv[m][e]) - sr[m][e] * KS[m][e];
    // batch 2: Q and P fragments, the O scales of tokens 16m + li
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) aq[m][ks] = ld8(buf, kBufQ + swz256(16 * m + li, 4 * ks + lq));
    float so[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) so[m] = *reinterpret_cast<const float*>(buf + kBufTok + 4 * (2 * kC + 16 * m + li));
    const float eC = *reinterpret_cast<const float*>(buf + kBufTok + 4 * 4 * kC);
    bf16x8 pa[6];
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) pa[i++] = ld8(buf + kBufPA, pa_off(0, 16 * m + li, 4 * ks + lq));
    f32x4 Dl[4], QT[4];
    bf16x4 Db[4];
    bf16x8 akt[8][2];
#pragma unroll
    for (int m = 0; m < 4; ++m) QT[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    delta_substitution(R, dg, a10, a2x, a3x, a32, Dl, Db, [&](int s) {
        const int m = s / 2, k0 = 2 * (s % 2);
        QT[m] = mfma16(Bs[k0], aq[m][k0], QT[m]);
        QT[m] = mfma16(Bs[k0 + 1], aq[m][k0 + 1], QT[m]);
        if (s == 2) store_prev();
        if (s % 2 == 1)   // Q tile m retired: K^T fragments of state tiles 2m, 2m + 1
#pragma unroll
            for (int t = 2 * m; t < 2 * m + 2; ++t)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) akt[t][ks] = kt_frag(buf, t, ks, li, lq);
    });
    // the scales of the update
    f32x4 su[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) su[m] = ldf4(buf, kBufTok + 4 * (3 * kC + 16 * m + 4 * lq));
    const bf16x8 BD[2] = {cat4(Db[0], Db[1]), cat4(Db[2], Db[3])};
#pragma unroll
    for (int m = 0, i = 0; m < 4; ++m) {
        f32x4 acc = QT[m] * so[m];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) acc = mfma16(BD[ks], pa[i++], acc);
        Ob[m] = __builtin_convertvector(acc, bf16x4);
    }
    bf16x8 BH[2], BL[2];
    split_hi_lo(su, Dl, BH, BL);
    // the eight state tiles' accumulation chains interleaved
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] *= eC;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma16(akt[t][st / 2], (st % 2 ? BL : BH)[st / 2], S[t]);
}

// The precise mode's chunk: the substitution with the coupling and diagonal
// products on bf16 hi + lo (delta_substitution_hl), O's P Delta on hi + lo,
// and the state update as in chunk_products; K S0 and (Q S0)^T take S0
// rounded once to bf16, as in the default precision.  About 1.4x the MFMAs
// of the default; the operands are loaded in smaller batches (fewer
// registers, more exposed LDS latency).
template <class StorePrev>
__device__ __forceinline__ void chunk_products_hl(const char* buf, f32x4 S[8], const bf16x4 vv[4], bf16x4 Ob[4],
                                                  int li, int lq, StorePrev&& store_prev) {
    bf16x8 Bh[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Bh[ks] = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
    // K S0 in two halves of row tiles
    f32x4 KS[4];
#pragma unroll
    for (int mh = 0; mh < 4; mh += 2) {
        bf16x8 ak[2][4];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ak[mm][ks] = ld8(buf, kBufK + swz256(16 * (mh + mm) + li, 4 * ks + lq));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc = mfma16(ak[mm][ks], Bh[ks], acc);
            }
            KS[mh + mm] = acc;
        }
    }
    // R and the substitution's operands (hi from AN, lo from AN_lo)
    f32x4 R[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = 16 * m + 4 * lq;
        const f32x4 sb = ldf4(buf, kBufTok + 4 * (0 * kC + r0));
        const f32x4 sr = ldf4(buf, kBufTok + 4 * (1 * kC + r0));
#pragma unroll
        for (int e = 0; e < 4; ++e) R[m][e] = sb[e] * float(vv[m][e]) - sr[e] * KS[m][e];
    }
    SubstFrags f;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
        const char* an = buf + (hl ? kBufPAlo : kBufPA);
        f.d[hl][0] = ld4(an, pa_off(1, li, lq));
        f.d[hl][1] = ld4(an, pa_off(1, 16 + li, lq) + 8);
        f.d[hl][2] = ld4(an, pa_off(1, 32 + li, 4 + lq));
        f.d[hl][3] = ld4(an, pa_off(1, 48 + li, 4 + lq) + 8);
        f.a10[hl] = ld4(an, pa_off(1, 16 + li, lq));
        f.a2x[hl] = ld8(an, pa_off(1, 32 + li, lq));
        f.a3x[hl] = ld8(an, pa_off(1, 48 + li, lq));
        f.a32[hl] = ld4(an, pa_off(1, 48 + li, 4 + lq));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 Dl[4];
    bf16x4 Db[4], Dbl[4];
    delta_substitution_hl(R, f, Dl, Db, Dbl, [&](int st) {
        if (st == 2) store_prev();
    });
    __builtin_amdgcn_sched_barrier(0);
    // (Q S0)^T in two halves, then O^T = (Q S0)^T diag(Gamma n_q) + (P Delta)^T
    f32x4 QT[4];
#pragma unroll
    for (int mh = 0; mh < 4; mh += 2) {
        bf16x8 aq[2][4];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) aq[mm][ks] = ld8(buf, kBufQ + swz256(16 * (mh + mm) + li, 4 * ks + lq));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc = mfma16(Bh[k], aq[mm][k], acc);
            }
            QT[mh + mm] = acc;
        }
    }
    const bf16x8 BDh[2] = {cat4(Db[0], Db[1]), cat4(Db[2], Db[3])};
    const bf16x8 BDl[2] = {cat4(Dbl[0], Dbl[1]), cat4(Dbl[2], Dbl[3])};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float so = *reinterpret_cast<const float*>(buf + kBufTok + 4 * (2 * kC + 16 * m + li));
        f32x4 acc = QT[m] * so;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks == 0 || m >= 2) {
                const bf16x8 ph = ld8(buf + kBufPA, pa_off(0, 16 * m + li, 4 * ks + lq));
                const bf16x8 pl = ld8(buf + kBufPAlo, pa_off(0, 16 * m + li, 4 * ks + lq));
                acc = mfma16(BDh[ks], ph, acc);
                acc = mfma16(BDh[ks], pl, acc);
                acc = mfma16(BDl[ks], ph, acc);
            }
        Ob[m] = __builtin_convertvector(acc, bf16x4);
    }
    // the state update, as in chunk_products
    f32x4 su[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) su[m] = ldf4(buf, kBufTok + 4 * (3 * kC + 16 * m + 4 * lq));
    const float eC = *reinterpret_cast<const float*>(buf + kBufTok + 4 * 4 * kC);
    bf16x8 BH[2], BL[2];
    split_hi_lo(su, Dl, BH, BL);
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] *= eC;
#pragma unroll
    for (int th = 0; th < 8; th += 4) {
        bf16x8 akt[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) akt[t][ks] = kt_frag(buf, th + t, ks, li, lq);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                S[th + t] = mfma16(akt[t][st / 2], (st % 2 ? BL : BH)[st / 2], S[th + t]);
    }
}

struct StateCtx {
    int b, rb, kh, h, zcol0;   // rb: the sequence's index among the launch's records
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
// (16 state columns each) and 8 - NW memory waves (m = wave - NW; wave w
// runs on SIMD w % 4).  Memory wave m copies the record pieces
// [rec_lo(m), rec_hi(m)) of each chunk.  The V waves (NW = 4: every memory
// wave, which also copies record pieces; NW = 2: m = 4, 5, on the SIMDs
// without a compute wave, which copy none) run the front end of the slice's
// v channels, part v_part(m) of the chunk's rows, one 4-channel x 4-row item
// per lane, from a raw slab of exactly those rows (+ 3 rows of conv history)
// that the same wave copied into its own slab region two chunks earlier.
template <int NW, bool PRECISE = false>
struct StateShape {
    static constexpr int NM = 8 - NW;
    static constexpr int N = 16 * NW;                        // state columns per workgroup
    static constexpr int SPLIT = kD / N;
    static constexpr int VT = buf_vt(PRECISE);               // V^T offset in a buffer
    static constexpr int BUF = VT + N * kVtLd * 2;
    static constexpr int PIECES = num_pieces(PRECISE);
    static constexpr int NV = NW == 4 ? 4 : 2;               // V waves = parts of the chunk's rows
    static constexpr int SLAB_ROW = N * 2;                   // raw v slab: [rows][N channels] bf16
    static constexpr int PART_ROWS = kC / NV;
    static constexpr int SLAB_ROWS = PART_ROWS + 3;
    static constexpr int SLAB_PIECES = (SLAB_ROWS * SLAB_ROW + 1023) / 1024;
    // one part's slab region: the bytes copied (the last piece's lanes past
    // them are inactive and write nothing)
    static constexpr int SLAB = SLAB_ROWS * SLAB_ROW;
    static_assert(SLAB_PIECES == 3 && SLAB % 16 == 0, "three slab pieces per V wave");
    // chunk buffers: three (records requested two chunks ahead) where they
    // fit in LDS, else two
    static constexpr int NB = NW == 2 && !PRECISE ? 3 : 2;
    static_assert(NB * BUF + 2 * NV * SLAB + 16 * N <= 160 * 1024, "state kernel LDS");
    static constexpr bool is_v(int m) { return NW == 4 || m >= 4; }
    static constexpr int v_part(int m) { return NW == 4 ? m : m - 4; }
    // record pieces: NW = 2: 12, 12, 11, 11 for the copy waves m 0..3 and
    // none for the V waves; NW = 4: 12, 12, 11, 11 (precise: 15, 15, 14, 14
    // in both shapes)
    static constexpr int rec_lo(int m) {
        if (m >= 4) return PIECES;
        if constexpr (PRECISE) return m < 2 ? 15 * m : 30 + 14 * (m - 2);
        return m < 2 ? 12 * m : 24 + 11 * (m - 2);
    }
    static constexpr int rec_hi(int m) { return m + 1 == NM ? PIECES : rec_lo(m + 1); }
};

// Copy piece pc of the raw v slab of row part `part` of a chunk (slab row i
// = call-local token local0 - 3 + part * PART_ROWS + i) into `slab`
template <int NW>
__device__ __forceinline__ void issue_slab(const PrefillParams& p, const StateCtx& cx, char* slab, int64_t local0,
                                           int part, int pc, int lane) {
    using SS = StateShape<NW>;
    const int o = pc * 1024 + 16 * lane;
    if (o < SS::SLAB_ROWS * SS::SLAB_ROW) {
        const int row = o / SS::SLAB_ROW, g = (o % SS::SLAB_ROW) / 16;
        const int64_t t = min(max(local0 - 3 + part * SS::PART_ROWS + row, (int64_t)0), p.seq_len - 1);
        const uint16_t* src = static_cast<const uint16_t*>(p.qkv) + ((int64_t)cx.b * p.seq_len + t) * p.conv_dim +
                              2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + 8 * g;
        __builtin_amdgcn_global_load_lds(src, LDS_PTR(slab + pc * 1024), 16, 0, 0);
    }
}

// Front end of row part `part` of the slice's v channels for one chunk from
// its raw slab -> V^T in the chunk's buffer.  Items of 4 channels x 4 rows,
// one per lane: N / 4 channel groups x PART_ROWS / 4 row groups = 64 items.
template <int NW, bool INTERIOR, bool PRECISE>
__device__ __forceinline__ void v_front(const PrefillParams& p, const StateCtx& cx, const float* Wv, const char* slab,
                                        char* buf, int64_t local0, int part, int lane) {
    using SS = StateShape<NW, PRECISE>;
    constexpr int CG = SS::N / 4;
    static_assert(CG * (SS::PART_ROWS / 4) == 64, "one item per lane");
    const int c0 = (lane % CG) * 4, rt = (lane / CG) * 4;
    const int tau0 = part * SS::PART_ROWS + rt;
    const int64_t gc = 2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + c0;
    uint2 raw[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) raw[k] = *reinterpret_cast<const uint2*>(slab + (rt + k) * SS::SLAB_ROW + 2 * c0);
    float w[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[t][i] = Wv[t * SS::N + c0 + i];
    bf16x4 ub[4];
    conv_compute<INTERIOR, 4>(p, cx.b, gc, local0, tau0, w, raw, ub);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<bf16x4*>(buf + SS::VT + ((c0 + i) * kVtLd + tau0) * 2) = bf16x4{ub[0][i], ub[1][i], ub[2][i], ub[3][i]};
}

// O of chunk kc -> out (bf16): lane (i, q) of compute wave w writes columns
// 16w + 4q .. 16w + 4q + 3 of token 16m + i, one 8-byte store per tile.
// `obase` points at this lane's columns of call-local token i.
// x unchanged but hidden from the optimiser: the addresses formed from it
// are computed where they are used, not kept live across the chunk loop
// (which would spill them)
__device__ __forceinline__ int64_t opaque(int64_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ void store_o(const PrefillParams& p, uint16_t* obase, const bf16x4 O[4], int64_t kc, int li) {
    const int64_t row_stride = (int64_t)p.num_v_heads * kD;
    const int64_t t0 = kc * kC - p.start_pos;
    uint16_t* o = obase + t0 * row_stride;
    if (t0 >= 0 && t0 + kC <= p.seq_len) {
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<bf16x4*>(o + 16 * m * row_stride) = O[m];
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int64_t t = t0 + 16 * m + li;
            if (t >= 0 && t < p.seq_len) *reinterpret_cast<bf16x4*>(o + 16 * m * row_stride) = O[m];
        }
    }
}

// Checkpoint slot of chunk kc, whose end is a multiple of the checkpoint
// interval (the caller tracks that): this compute wave's state slice and
// (over the compute threads) the conv tails of the workgroup's channels
template <int NW>
__device__ __forceinline__ void checkpoint(const PrefillParams& p, const StateCtx& cx, const f32x4 S[8], int64_t kc,
                                           int tid) {
    constexpr int NT = 64 * NW, NCH = 2 * kD + 16 * NW;
    const int lq = (tid % 64) / 16;
    const int64_t pe = (kc + 1) * kC;
    if (pe <= p.start_pos + p.seq_len) {
        char* slot = p.ckpt_buf + (uint64_t)(pe / p.ckpt_interval - 1) * p.slot_bytes;
        float* rec = reinterpret_cast<float*>(slot + p.conv_slot_bytes);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[opaque(cx.s_base) + (int64_t)(16 * t + 4 * lq + e) * kD] = S[t][e];
        uint16_t* ctail = reinterpret_cast<uint16_t*>(slot);
        for (int ch = tid; ch < NCH; ch += NT)
            if (ch >= 2 * kD || cx.owns_qk_tail) write_tail(p, cx.b, pe - p.start_pos, state_channel(p, cx, ch), ctail);
    }
}

// vmcnt(n): wait until at most n vector-memory operations of this wave are
// outstanding (they complete in issue order).  LGKM: also wait for every LDS
// operation.
template <int n, bool LGKM = false>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt field");
    // vmcnt bits 3:0 and 15:14; expcnt: no wait
    __builtin_amdgcn_s_waitcnt((LGKM ? 0x0070 : 0x0f70) | (n & 15) | ((n >> 4) << 14));
}

// Workgroup barrier without the memory fences of __syncthreads: each wave
// first waits itself for the operations the others depend on (its LDS reads
// and writes, its LDS copies), so copies that no other wave reads before the
// next barrier (a V wave's next slab) stay in flight.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Overlapped call: chunk cr's records are complete once its flag holds the
// call's epoch.  `ready` holds the flag as loaded one step earlier; until it
// matches, the wave polls.  A wait gives up after 2 s (the error word
// kHdrErrWait, after which every wait of the call returns at once), so a
// wave never waits without bound; the compute waves then poison their
// slice of the call's outputs (ovl_failed).
__device__ __forceinline__ void await_chunk(const SplitParams& sp, const StateCtx& cx, int cr, uint64_t ready) {
    wait_vm<0>();   // the flag load of the previous step has returned
    if (__builtin_amdgcn_readfirstlane((uint32_t)(ready == sp.epoch))) return;
    const uint64_t* f = sp.flags + (int64_t)(cx.rb * sp.p.num_k_heads + cx.kh) * sp.frow + cr;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sp.epoch) return;
        if (__hip_atomic_load(sp.hdr + kHdrErrWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sp.epoch) return;
        if (__builtin_amdgcn_s_memrealtime() - t0 > sp.wait_ticks) {
            ovl_error(sp.hdr, kHdrErrWait, sp.epoch);
            return;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

// Whether an overlapped call met an error (a wait that timed out, or a
// workgroup placed outside its XCD's share): its outputs cannot be trusted
__device__ __forceinline__ bool ovl_failed(const SplitParams& sp) {
    if (!sp.flags) return false;
    bool bad = false;
#pragma unroll
    for (int w : {kHdrErrXcd, kHdrErrClaim, kHdrErrWait})
        bad |= __hip_atomic_load(sp.hdr + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sp.epoch;
    return bad;
}

__device__ __forceinline__ uint64_t load_flag(const SplitParams& sp, const StateCtx& cx, int cr) {
    asm volatile("" ::: "memory");   // issued after this step's record copies
    return __hip_atomic_load(sp.flags + (int64_t)(cx.rb * sp.p.num_k_heads + cx.kh) * sp.frow + cr, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Memory wave M's step c, run while the compute waves work on chunk c - 1
// (c = 0: before the first chunk).  It completes chunk c's buffer vbuf.  A
// copy wave requests its pieces of chunk c + NB - 2 into rbuf and waits for
// those of chunk c.  A V wave requests its pieces of chunk c, if it copies
// any (NW = 4), waits for chunk c's slab (in `slab`, requested two steps
// earlier), runs the front end into vbuf, then requests chunk c + 2's slab
// into the same region, which stays in flight across the barrier that
// follows.
template <int NW, int M, bool PRECISE>
__device__ __forceinline__ void mem_step(const SplitParams& sp, const StateCtx& cx, const float* Wv, char* rbuf,
                                          char* vbuf, char* slab, int c, int lane, uint64_t& ready) {
    using SS = StateShape<NW, PRECISE>;
    constexpr int LO = SS::rec_lo(M), HI = SS::rec_hi(M), AHEAD = SS::NB - 2;
    if constexpr (!SS::is_v(M)) {
        const int cr = c + AHEAD;
        if (cr < sp.nseg) {
            const bool ovl = sp.flags != nullptr;
            if (ovl && cr >= sp.n1) await_chunk(sp, cx, cr, ready);
            const char* krec = key_rec(sp, cx.rb, cx.kh, cr);
            const char* vrec = val_rec(sp, cx.rb, cx.h, cr);
#pragma unroll
            for (int pc = LO; pc < HI; ++pc) issue_piece<PRECISE>(rbuf, krec, vrec, pc, lane);
            if constexpr (AHEAD > 0)
                wait_vm<HI - LO, true>();   // chunk c's pieces, requested one step earlier, have landed
            else
                wait_vm<0, true>();
            if (ovl && cr + 1 < sp.nseg && cr + 1 >= sp.n1) ready = load_flag(sp, cx, cr + 1);
            return;
        }
        wait_vm<0, true>();
    } else {
        constexpr int P = HI - LO;   // record pieces a V wave copies (NW = 4; none at NW = 2)
        static_assert(P == 0 || AHEAD == 0, "V waves copy pieces only with two buffers");
        if (c < sp.nseg) {
            constexpr int part = SS::v_part(M);
            if constexpr (P > 0) {
                const char* krec = key_rec(sp, cx.rb, cx.kh, c);
                const char* vrec = val_rec(sp, cx.rb, cx.h, c);
#pragma unroll
                for (int pc = LO; pc < HI; ++pc) issue_piece<PRECISE>(rbuf, krec, vrec, pc, lane);
            }
            // outstanding, in issue order: the slabs of chunks c and (if any)
            // c + 1, then this step's pieces
            if (c + 1 < sp.nseg)
                wait_vm<SS::SLAB_PIECES + P>();
            else
                wait_vm<P>();
            const int64_t local0 = (sp.k0 + c) * kC - sp.p.start_pos;
            if (local0 >= 3 && local0 + kC <= sp.p.seq_len)
                v_front<NW, true, PRECISE>(sp.p, cx, Wv, slab, vbuf, local0, part, lane);
            else
                v_front<NW, false, PRECISE>(sp.p, cx, Wv, slab, vbuf, local0, part, lane);
            if (c + 2 < sp.nseg) {
                // the front end's reads of this region have returned
                __builtin_amdgcn_s_waitcnt(0xc07f);
                asm volatile("" ::: "memory");
#pragma unroll
                for (int pc = 0; pc < SS::SLAB_PIECES; ++pc)
                    issue_slab<NW>(sp.p, cx, slab, local0 + 2 * kC, part, pc, lane);
            }
            // this step's pieces have landed (chunk c + 2's slab may not have)
            if constexpr (P > 0) {
                if (c + 2 < sp.nseg)
                    wait_vm<SS::SLAB_PIECES>();
                else
                    wait_vm<0>();
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the V^T writes are done
    }
}

// Memory wave M over the whole segment, with the compute waves' barriers
// (two in the prologue, one per chunk).  Chunk c's buffer is
// buf[c % NB] and a V wave's slab of chunk c is slab[c % 2]; the loop is
// unrolled over a whole period of both so that every buffer and slab region
// is a distinct object at each step.
template <int NW, int M, bool PRECISE>
__device__ __forceinline__ void mem_role(const SplitParams& sp, const StateCtx& cx, const float* Wv, char* buf0,
                                          char* buf1, char* buf2, char* slab0, char* slab1, int lane) {
    using SS = StateShape<NW, PRECISE>;
    constexpr int NB = SS::NB, LO = SS::rec_lo(M), HI = SS::rec_hi(M);
    constexpr int PERIOD = NB == 3 ? 6 : 2;
    char* const bufs[3] = {buf0, buf1, buf2};
    char* const slabs[2] = {slab0, slab1};
    uint64_t ready = 0;   // copy waves of an overlapped call: the next chunk's flag
    if constexpr (SS::is_v(M)) {
        const int64_t l0 = sp.k0 * kC - sp.p.start_pos;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            if (c < sp.nseg)
#pragma unroll
                for (int pc = 0; pc < SS::SLAB_PIECES; ++pc)
                    issue_slab<NW>(sp.p, cx, slabs[c], l0 + c * kC, SS::v_part(M), pc, lane);
    } else if constexpr (NB == 3) {
        if (sp.nseg > 0) {   // chunk 0's pieces; step 0 requests chunk 1's
            const char* krec = key_rec(sp, cx.rb, cx.kh, 0);
            const char* vrec = val_rec(sp, cx.rb, cx.h, 0);
#pragma unroll
            for (int pc = LO; pc < HI; ++pc) issue_piece<PRECISE>(buf0, krec, vrec, pc, lane);
        }
    }
    wait_vm<0>();
    __syncthreads();
    mem_step<NW, M, PRECISE>(sp, cx, Wv, bufs[(NB - 2) % NB], buf0, slab0, 0, lane, ready);
    __syncthreads();
    for (int c = 1; c <= sp.nseg; c += PERIOD) {
#pragma unroll
        for (int i = 0; i < PERIOD; ++i) {
            if (c + i <= sp.nseg) {
                mem_step<NW, M, PRECISE>(sp, cx, Wv, bufs[(1 + i + NB - 2) % NB], bufs[(1 + i) % NB],
                                          slabs[(1 + i) % 2], c + i, lane, ready);
                lds_barrier();
            }
        }
    }
    wait_vm<0>();
}

__device__ __forceinline__ const SplitParams& base_of(const SplitParams& s) { return s; }
__device__ __forceinline__ const SplitParams& base_of(const VarlenParams& v) { return v.sp; }

// Waves 0..NW-1 own 16 state columns each; waves NW..7 move data.  One
// barrier per chunk: the chunk's products are done (its buffer may be
// refilled) and the next chunk's buffer is filled.  KP = SplitParams (one
// call's sequences share length and start) or VarlenParams (a group of
// sequences of their own; a sequence with no chunk in this segment is done,
// its state and conv tail written by the segment that held its last chunk,
// except in the first segment, where a sequence of no tokens copies its
// states).
template <int NW, bool PRECISE, class KP>
__global__ __launch_bounds__(512) void state_kernel(KP kp) {
    constexpr bool VARLEN = std::is_same<KP, VarlenParams>::value;
    using SS = StateShape<NW, PRECISE>;
    constexpr int N = SS::N, NCH = 2 * kD + N;
    const PrefillParams& p0 = base_of(kp).p;
    // separate arrays: the compiler keeps their accesses apart (one block
    // with computed offsets measured 10% slower)
    __shared__ __attribute__((aligned(16))) char buf0[SS::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[SS::BUF];
    __shared__ __attribute__((aligned(16))) char buf2[SS::NB == 3 ? SS::BUF : 16];
    __shared__ __attribute__((aligned(16))) char slab0[SS::NV * SS::SLAB];   // raw v slabs of the V waves,
    __shared__ __attribute__((aligned(16))) char slab1[SS::NV * SS::SLAB];   // per chunk parity
    __shared__ float Wv[4 * N];                                     // conv taps of the slice's v channels

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: role branches stay scalar
    const int li = lane % 16, lq = lane / 16;
    const bool compute = wave < NW;
    // workgroup -> (sequence, key head, member); the r * SPLIT members of
    // one (sequence, key head) share a blockIdx % 8, so the round-robin
    // dispatch puts them on one XCD and its L2, where their common key
    // records stay
    const int r = p0.num_v_heads / p0.num_k_heads;
    const int M = r * SS::SPLIT;
    int entries, b0 = 0;
    if constexpr (VARLEN) {
        entries = kp.nb;
        b0 = kp.b0;
    } else {
        entries = p0.batch;
    }
    const int NG = entries * p0.num_k_heads;
    int bid = blockIdx.x;
    if constexpr (!VARLEN) {
        if (kp.flags) {
            // overlapped call: take the next of this XCD's (group, member)
            // slots, groups g with g % 8 == XCD (those whose records the tail
            // prep writes into this XCD's L2); the slot count per XCD equals
            // the workgroups the round-robin dispatch puts there
            __shared__ int claim;
            if (tid == 0) {
                const unsigned x = xcd_id();
                const int share = NG / kOvlXcds * M;
                const int sl = x < kOvlXcds ? (int)claim_next(kp.hdr + kHdrState + 32 * x, kp.epoch) : share;
                if (sl >= share) ovl_error(kp.hdr, x < kOvlXcds ? kHdrErrClaim : kHdrErrXcd, kp.epoch);
                claim = sl < share ? kOvlXcds * sl + (int)x : -1;
            }
            __syncthreads();
            bid = claim;
            if (bid < 0) return;
        }
    }
    const int grp = (bid / 8 / M) * 8 + bid % 8;
    const int member = (bid / 8) % M;
    if (grp >= NG) return;
    StateCtx cx;
    cx.rb = grp / p0.num_k_heads;
    cx.b = b0 + cx.rb;
    cx.kh = grp % p0.num_k_heads;
    cx.h = cx.kh * r + member / SS::SPLIT;
    cx.zcol0 = (member % SS::SPLIT) * N;
    cx.owns_qk_tail = member == 0;
    cx.s_base = ((int64_t)cx.b * p0.num_v_heads + cx.h) * kD * kD + cx.zcol0 + 16 * (compute ? wave : 0) + li;
    SplitParams view;
    if constexpr (VARLEN) {
        view = seq_view(kp, cx.rb, cx.b);
        if (view.nseg == 0 && !view.first_seg) return;
    }
    const SplitParams& sp = VARLEN ? view : base_of(kp);
    const PrefillParams& p = sp.p;

    for (int e = tid; e < 4 * N; e += 512) {
        const int t = e / N, c = e % N;
        const int64_t gc = 2 * (int64_t)p.num_k_heads * kD + (int64_t)cx.h * kD + cx.zcol0 + c;
        Wv[e] = bf16_bits_to_f32(static_cast<const uint16_t*>(p.conv_w)[gc * 4 + t]);
    }
    __syncthreads();

    // The two roles run separate loops with the same barriers (two in the
    // prologue, one per chunk), so their registers do not add up.
    if (compute) {
        const float* s_src = sp.first_seg ? p.rec_in : p.rec_out;
        f32x4 S[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[t][e] = s_src ? s_src[cx.s_base + (int64_t)(16 * t + 4 * lq + e) * kD] : 0.f;
        // checkpoints every `every` chunks; `phase` counts chunk ends since
        // the last one (0: this chunk's end is a checkpoint position)
        const int64_t every = p.ckpt_interval / kC;
        int64_t phase = every > 0 ? (sp.k0 + 1) % every : 1;
        // the state loads complete here, so the chunk loop never waits on
        // the vector-memory counter (its O stores would hold it up)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        __syncthreads();
        const int cw = 16 * wave + li;
        uint16_t* obase = static_cast<uint16_t*>(p.out) + ((int64_t)cx.b * p.seq_len * p.num_v_heads + cx.h) * kD +
                          cx.zcol0 + 16 * wave + 4 * lq + (int64_t)li * p.num_v_heads * kD;
        bf16x4 Ob[4];   // O of the previous chunk, stored during the next one
        for (int j = 0, jb = 0; j < sp.nseg; ++j, jb = jb + 1 == SS::NB ? 0 : jb + 1) {
            const char* cur = jb == 0 ? buf0 : jb == 1 ? buf1 : buf2;
            bf16x4 vv[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                vv[mb] = *reinterpret_cast<const bf16x4*>(cur + SS::VT + (cw * kVtLd + 16 * mb + 4 * lq) * 2);
            bf16x4 On[4];
            auto store_prev = [&] {
                if (j > 0) store_o(p, obase, Ob, sp.k0 + j - 1, li);
            };
            if constexpr (PRECISE) chunk_products_hl(cur, S, vv, On, li, lq, store_prev);
            else chunk_products(cur, S, vv, On, li, lq, store_prev);
#pragma unroll
            for (int m = 0; m < 4; ++m) Ob[m] = On[m];
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): every LDS read of this buffer has returned
            lds_barrier();
            if (every > 0) {
                if (phase == 0) checkpoint<NW>(p, cx, S, sp.k0 + j, tid);
                phase = phase + 1 == every ? 0 : phase + 1;
            }
        }
        if (sp.nseg > 0) store_o(p, obase, Ob, sp.k0 + sp.nseg - 1, li);
        // an overlapped call whose prep did not keep up (its CUs held by
        // other work for the whole wait bound) computed from records that
        // were not complete: it fails loudly, with NaN in this wave's
        // columns of every output row of the segment and of the final state
        if (__builtin_amdgcn_readfirstlane((uint32_t)ovl_failed(sp))) {
            __builtin_amdgcn_s_waitcnt(0);
            const int64_t t_lo = std::max<int64_t>(sp.k0 * kC - p.start_pos, 0);
            const int64_t t_hi = std::min<int64_t>((sp.k0 + sp.nseg) * kC - p.start_pos, p.seq_len);
            uint16_t* ocol = static_cast<uint16_t*>(p.out) + ((int64_t)cx.b * p.seq_len * p.num_v_heads + cx.h) * kD +
                             cx.zcol0 + 16 * wave + 4 * (lane % 4);
            const bf16x4 qnan = {(__bf16)__builtin_nanf(""), (__bf16)__builtin_nanf(""), (__bf16)__builtin_nanf(""),
                                 (__bf16)__builtin_nanf("")};
            for (int64_t t = t_lo + lane / 4; t < t_hi; t += 16)
                *reinterpret_cast<bf16x4*>(ocol + t * p.num_v_heads * kD) = qnan;
#pragma unroll
            for (int t = 0; t < 8; ++t) S[t] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                     __builtin_nanf("")};
        }
        const int64_t sb = opaque(cx.s_base);
        const int64_t lq4 = opaque(4 * lq);   // the offsets of the state load are not kept across the loop
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.rec_out[sb + (16 * t + lq4 + e) * kD] = S[t][e];
    } else {
        // each V wave's slab region: part v_part(m) of the slab arrays
        const int m = wave - NW;
        const int vo = SS::is_v(m) ? SS::v_part(m) * SS::SLAB : 0;
        char* s0 = slab0 + vo;
        char* s1 = slab1 + vo;
        switch (m) {
            case 0: mem_role<NW, 0, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane); break;
            case 1: mem_role<NW, 1, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane); break;
            case 2: mem_role<NW, 2, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane); break;
            case 3: mem_role<NW, 3, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane); break;
            default:
                if constexpr (NW == 2) {
                    if (m == 4) mem_role<NW, 4, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane);
                    else mem_role<NW, 5, PRECISE>(sp, cx, Wv, buf0, buf1, buf2, s0, s1, lane);
                }
                break;
        }
    }
    if (sp.last_seg) {
        for (int ch = tid; ch < NCH; ch += 512)
            if (ch >= 2 * kD || cx.owns_qk_tail)
                write_tail(p, cx.b, p.seq_len, state_channel(p, cx, ch), static_cast<uint16_t*>(p.conv_out));
    }
}

template <int NW, bool PRECISE>
hipError_t launch_state(const SplitParams& sp, hipStream_t stream) {
    const int r = sp.p.num_v_heads / sp.p.num_k_heads;
    const int ng = sp.p.batch * sp.p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * StateShape<NW>::SPLIT;
    hipLaunchKernelGGL((state_kernel<NW, PRECISE, SplitParams>), dim3(blocks), dim3(512), 0, stream, sp);
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
    const bool w4 = state_waves(sp.p) == 4;
    if (sp.p.precise) return w4 ? launch_state<4, true>(sp, stream) : launch_state<2, true>(sp, stream);
    return w4 ? launch_state<4, false>(sp, stream) : launch_state<2, false>(sp, stream);
}

template <int NW, bool PRECISE>
hipError_t launch_state_varlen(const VarlenParams& vp, hipStream_t stream) {
    const int r = vp.sp.p.num_v_heads / vp.sp.p.num_k_heads;
    const int ng = vp.nb * vp.sp.p.num_k_heads;
    const int blocks = ((ng + 7) / 8) * 8 * r * StateShape<NW>::SPLIT;
    hipLaunchKernelGGL((state_kernel<NW, PRECISE, VarlenParams>), dim3(blocks), dim3(512), 0, stream, vp);
    return hipGetLastError();
}

template <class KP>
hipError_t launch_prep_any(const PrefillParams& p, const KP& kp, dim3 grid, hipStream_t stream);

template <bool NEUMANN, bool PRECISE>
hipError_t launch_tail(const SplitParams& sp, hipStream_t stream) {
    hipLaunchKernelGGL((prep_kernel_tail<NEUMANN, PRECISE>), dim3(ovl_tail_blocks(PRECISE)), dim3(kPrepThreads), 0,
                       stream, sp);
    return hipGetLastError();
}

hipError_t launch_tail_any(const SplitParams& sp, hipStream_t stream) {
    if (sp.p.precise) return sp.p.diag_neumann ? launch_tail<true, true>(sp, stream) : launch_tail<false, true>(sp, stream);
    return sp.p.diag_neumann ? launch_tail<true, false>(sp, stream) : launch_tail<false, false>(sp, stream);
}

// ---- overlapped calls.  Two library streams per device with disjoint CU
// masks: 24 of the 32 CUs of every XCD run the head prep and the state
// kernel, the other 8 the tail prep.  Bit i of a mask is CU i; under either
// order of CUs over XCDs (32 consecutive CUs per XCD, or CU i on XCD i % 8)
// the pattern (i / 8) % 4 splits every XCD 24 : 8, so the round-robin
// dispatch finds CUs on every XCD.  (An unmasked dispatch does not place its
// workgroups around a masked queue's: it waits for the CUs that queue holds,
// so the state kernel needs a mask of its own.)
struct OvlStreams {
    bool tried = false, ok = false;
    hipStream_t main = nullptr, tail = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, join_tail = nullptr;
};
constexpr int kOvlMaxDevices = 64;
std::mutex ovl_mutex;
OvlStreams ovl_dev[kOvlMaxDevices];
uint64_t ovl_epoch = 0;   // last epoch handed out (under ovl_mutex)

// The streams of device `dev` (the current device; created on first use,
// kept until the process ends), or null where the chip is not 8 XCDs of 32
// CUs.  Call with ovl_mutex held.
OvlStreams* ovl_streams(int dev) {
    if (dev < 0 || dev >= kOvlMaxDevices) return nullptr;
    OvlStreams& o = ovl_dev[dev];
    if (!o.tried) {
        o.tried = true;
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus != 256)
            return nullptr;
        uint32_t mm[8], mt[8];
        for (int w = 0; w < 8; ++w) {
            mm[w] = mt[w] = 0;
            for (int bit = 0; bit < 32; ++bit) ((((32 * w + bit) / 8) % 4 == 3) ? mt[w] : mm[w]) |= 1u << bit;
        }
        o.ok = hipExtStreamCreateWithCUMask(&o.main, 8, mm) == hipSuccess &&
               hipExtStreamCreateWithCUMask(&o.tail, 8, mt) == hipSuccess &&
               hipEventCreateWithFlags(&o.fork, hipEventDisableTiming) == hipSuccess &&
               hipEventCreateWithFlags(&o.join, hipEventDisableTiming) == hipSuccess &&
               hipEventCreateWithFlags(&o.join_tail, hipEventDisableTiming) == hipSuccess;
    }
    return o.ok ? &o : nullptr;
}

// prep launch for (Neumann diagonal solve, precise mode)
template <class KP>
hipError_t launch_prep_any(const PrefillParams& p, const KP& kp, dim3 grid, hipStream_t stream) {
    constexpr bool V = std::is_same<KP, VarlenParams>::value;
    if (p.precise) {
        if (p.diag_neumann) {
            if constexpr (V) hipLaunchKernelGGL((prep_kernel_varlen<true, true>), grid, dim3(kPrepThreads), 0, stream, kp);
            else hipLaunchKernelGGL((prep_kernel<true, true>), grid, dim3(kPrepThreads), 0, stream, kp);
        } else {
            if constexpr (V) hipLaunchKernelGGL((prep_kernel_varlen<false, true>), grid, dim3(kPrepThreads), 0, stream, kp);
            else hipLaunchKernelGGL((prep_kernel<false, true>), grid, dim3(kPrepThreads), 0, stream, kp);
        }
    } else {
        if (p.diag_neumann) {
            if constexpr (V) hipLaunchKernelGGL((prep_kernel_varlen<true, false>), grid, dim3(kPrepThreads), 0, stream, kp);
            else hipLaunchKernelGGL((prep_kernel<true, false>), grid, dim3(kPrepThreads), 0, stream, kp);
        } else {
            if constexpr (V) hipLaunchKernelGGL((prep_kernel_varlen<false, false>), grid, dim3(kPrepThreads), 0, stream, kp);
            else hipLaunchKernelGGL((prep_kernel<false, false>), grid, dim3(kPrepThreads), 0, stream, kp);
        }
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_split_supported(const PrefillParams& p) {
    const int r = p.num_v_heads / p.num_k_heads;
    return r >= 1 && r <= kMaxGroup;
}

uint64_t prefill_split_chunk_bytes(int batch, int num_k_heads, int num_v_heads, bool precise) {
    return (uint64_t)batch * ((uint64_t)num_k_heads * kKeyRec + (uint64_t)num_v_heads * val_rec_bytes(precise));
}

uint64_t prefill_overlap_bytes(int batch, int num_k_heads, int64_t chunks) {
    return 8 * ((uint64_t)batch * num_k_heads * (uint64_t)((chunks + 31) / 32 * 32) + kOvlHdrWords);
}

namespace {

// Chunks of an overlapped call that the head prep launch covers: enough that
// the tail prep, on a quarter of the CUs, stays ahead of the state kernel.
// A quarter of the chunks in the default precision; 30% in the precise mode,
// whose tail holds one prep workgroup per CU instead of two (both measured
// best on the 16k prefill).  GDN_PREFILL_OVERLAP_HEAD (a fraction)
// overrides the default.
int64_t overlap_head(int64_t n, bool precise) {
    double f = precise ? 0.30 : 0.25;
    if (const char* env = getenv("GDN_PREFILL_OVERLAP_HEAD")) {
        const double v = atof(env);
        if (v > 0.0 && v < 1.0) f = v;
    }
    int64_t n1 = (int64_t)std::ceil(f * (double)n);
    if (n1 < 1) n1 = 1;
    if (n1 > n - 1) n1 = n - 1;
    return n1;
}

// One segment of n chunks with the tail of the prep concurrent with the head
// prep and the state kernel (see SplitParams).  Both library streams wait for
// the caller's stream to reach this call (earlier calls on it may still read
// the workspace); the caller's stream then waits for both library streams.
// The tail is persistent (one workgroup per slot of its CUs), so no later
// dispatch waits behind unplaced tail workgroups.  Returns
// hipErrorNotSupported, with nothing enqueued, where the call does not
// qualify.
hipError_t launch_overlapped(SplitParams sp, int64_t n, uint64_t per, uint64_t ws_bytes, hipStream_t stream) {
    const PrefillParams& p = sp.p;
    const char* env = getenv("GDN_PREFILL_OVERLAP");
    if (env && env[0] == '0') return hipErrorNotSupported;
    const bool forced = env && env[0] == '1';
    const int64_t ng = (int64_t)p.batch * p.num_k_heads;
    const int r = p.num_v_heads / p.num_k_heads;
    // the state grid (24 workgroups per XCD at most, one per CU, beside the
    // tail's 8) and the per-XCD shares must come out even; short calls gain
    // nothing
    if (state_waves(p) != 2 || ng % kOvlXcds != 0 || ng * r * StateShape<2>::SPLIT > 24 * kOvlXcds || n < 2 ||
        (!forced && n < 64) || n > (1 << 20))
        return hipErrorNotSupported;
    if (ws_bytes < (uint64_t)n * per + prefill_overlap_bytes(p.batch, p.num_k_heads, n)) return hipErrorNotSupported;
    // The tail stream is a blocking stream (the only kind a CU mask comes
    // with): work on the NULL stream waits for it, so a call on the NULL
    // (legacy) stream would run the tail alone before its head and state
    // kernels.  Such calls, and calls being captured, take the serial path.
    if (stream == nullptr || stream == hipStreamLegacy || stream == hipStreamPerThread) return hipErrorNotSupported;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return hipErrorNotSupported;
    int dev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess || dev != cur)
        return hipErrorNotSupported;
    std::lock_guard<std::mutex> lock(ovl_mutex);
    OvlStreams* o = ovl_streams(dev);
    if (!o) return hipErrorNotSupported;
    if (ovl_epoch == 0) {
        // start from the clock, so that calls of different processes on one
        // workspace are unlikely to share an epoch
        ovl_epoch = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() & 0xffffffffffull;
    }
    ovl_epoch = ovl_epoch + 1 > 0xffffffffffull ? 1 : ovl_epoch + 1;
    sp.epoch = ovl_epoch;
    sp.frow = (int32_t)((n + 31) / 32 * 32);
    sp.flags = reinterpret_cast<uint64_t*>(sp.ws + (uint64_t)n * per);
    sp.hdr = sp.flags + ng * sp.frow;
    sp.n1 = (int32_t)overlap_head(n, p.precise);
    sp.pj = sp.n1;
    // 2 s by default; GDN_PREFILL_OVERLAP_WAIT_US sets another bound (tests)
    sp.wait_ticks = 200000000ull;
    if (const char* w = getenv("GDN_PREFILL_OVERLAP_WAIT_US")) {
        const long long us = atoll(w);
        if (us > 0) sp.wait_ticks = (uint64_t)us * 100;
    }
    // GDN_PREFILL_OVERLAP_SKIP_TAIL=1 leaves the tail prep out, so that its
    // chunks are never published: a test of the failure path (every wait
    // runs into its bound, the outputs come back NaN)
    const char* skip = getenv("GDN_PREFILL_OVERLAP_SKIP_TAIL");
    const bool skip_tail = skip && skip[0] == '1';
    hipError_t e = hipEventRecord(o->fork, stream);
    if (e != hipSuccess) return e;   // nothing enqueued
    e = hipStreamWaitEvent(o->tail, o->fork, 0);
    if (e == hipSuccess) e = hipStreamWaitEvent(o->main, o->fork, 0);
    if (e == hipSuccess) e = launch_prep_any(p, sp, dim3((unsigned)(ng * sp.n1)), o->main);
    if (e == hipSuccess && !skip_tail) e = launch_tail_any(sp, o->tail);
    if (e == hipSuccess) e = p.precise ? launch_state<2, true>(sp, o->main) : launch_state<2, false>(sp, o->main);
    // Join both library streams back into the caller's stream, after a failed
    // launch too: whatever the call enqueued is then ordered before the
    // caller's later work.  The tail stream is joined as well as the main
    // one: a tail workgroup dispatched late (its CUs held by other work) may
    // still claim from the workspace header after the state kernel is done.
    hipError_t j = hipEventRecord(o->join, o->main);
    if (j == hipSuccess) j = hipStreamWaitEvent(stream, o->join, 0);
    if (j == hipSuccess) j = hipEventRecord(o->join_tail, o->tail);
    if (j == hipSuccess) j = hipStreamWaitEvent(stream, o->join_tail, 0);
    return e != hipSuccess ? e : j;
}

}  // namespace

hipError_t launch_prefill_split(const PrefillParams& p, void* ws, uint64_t ws_bytes, hipStream_t stream,
                                bool allow_overlap) {
    if (p.batch == 0) return hipSuccess;
    const uint64_t per = prefill_split_chunk_bytes(p.batch, p.num_k_heads, p.num_v_heads, p.precise);
    const int64_t k_first = p.start_pos / kC;
    const int64_t k_end = p.seq_len > 0 ? (p.start_pos + p.seq_len - 1) / kC + 1 : k_first;
    // segments of at most 2^22 / (B H_k) chunks keep the prep grid's
    // work-items below 2^31 (B H_k <= 2^20, so a segment holds a chunk)
    int64_t max_seg = (int64_t)(ws_bytes / per);
    const int64_t grid_cap = ((int64_t)1 << 22) / ((int64_t)p.batch * p.num_k_heads);
    if (max_seg > grid_cap) max_seg = grid_cap;
    if (max_seg < 1) return hipErrorInvalidValue;
    SplitParams sp{};
    sp.p = p;
    sp.ws = static_cast<char*>(ws);
    sp.vrec_bytes = val_rec_bytes(p.precise);
    sp.first_seg = 1;
    if (k_end == k_first) {
        sp.k0 = k_first;
        sp.nseg = 0;
        sp.last_seg = 1;
        return launch_state_any(sp, stream);
    }
    sp.rec_batch = p.batch;
    if (allow_overlap && k_end - k_first <= max_seg) {
        const int64_t n = k_end - k_first;
        sp.k0 = k_first;
        sp.nseg = (int32_t)n;
        sp.rec_stride = (int32_t)n;
        sp.last_seg = 1;
        const hipError_t e = launch_overlapped(sp, n, per, ws_bytes, stream);
        if (e != hipErrorNotSupported) return e;
    }
    for (int64_t k0 = k_first; k0 < k_end; k0 += max_seg) {
        const int64_t n = k_end - k0 < max_seg ? k_end - k0 : max_seg;
        sp.k0 = k0;
        sp.nseg = (int32_t)n;
        sp.rec_stride = (int32_t)n;
        sp.pj = (int32_t)n;
        sp.last_seg = k0 + n == k_end;
        const dim3 grid((unsigned)(p.batch * p.num_k_heads * n));
        hipError_t e = launch_prep_any(p, sp, grid, stream);
        if (e != hipSuccess) return e;
        e = launch_state_any(sp, stream);
        if (e != hipSuccess) return e;
        sp.first_seg = 0;
    }
    return hipSuccess;
}

uint64_t prefill_varlen_group_bytes(int num_seqs, int num_k_heads, int num_v_heads, bool precise) {
    return prefill_split_chunk_bytes(num_seqs < kVarlenGroup ? num_seqs : kVarlenGroup, num_k_heads, num_v_heads,
                                     precise);
}

int prefill_varlen_group() { return kVarlenGroup; }

// Sequences of one call in groups of kVarlenGroup; per group, segments of
// as many chunks per sequence as the workspace holds for the whole group.
hipError_t launch_prefill_varlen(const PrefillParams& p, const int64_t* cu_seqlens, const int64_t* start_pos,
                                 void* ws, uint64_t ws_bytes, hipStream_t stream) {
    for (int g0 = 0; g0 < p.batch; g0 += kVarlenGroup) {
        const int G = p.batch - g0 < kVarlenGroup ? p.batch - g0 : kVarlenGroup;
        VarlenParams vp{};
        vp.sp.p = p;
        vp.sp.ws = static_cast<char*>(ws);
        vp.sp.vrec_bytes = val_rec_bytes(p.precise);
        vp.sp.rec_batch = G;
        vp.b0 = g0;
        vp.nb = G;
        int64_t max_n = 0;
        for (int i = 0; i < G; ++i) {
            const int64_t t0 = cu_seqlens[g0 + i], len = cu_seqlens[g0 + i + 1] - t0, st = start_pos[g0 + i];
            vp.seq[i] = SeqDesc{t0, st, len};
            const int64_t n = len > 0 ? (st + len - 1) / kC + 1 - st / kC : 0;
            if (n > max_n) max_n = n;
        }
        int64_t seg = (int64_t)(ws_bytes / prefill_split_chunk_bytes(G, p.num_k_heads, p.num_v_heads, p.precise));
        const int64_t grid_cap = ((int64_t)1 << 22) / ((int64_t)G * p.num_k_heads);
        if (seg > max_n) seg = max_n;
        if (seg > grid_cap) seg = grid_cap;
        if (seg < 1) seg = 1;
        vp.sp.rec_stride = (int32_t)seg;
        PrefillParams pg = p;
        pg.batch = G;
        const int nw = state_waves(pg);
        for (int64_t j0 = 0; j0 == 0 || j0 < max_n; j0 += seg) {
            vp.j0 = j0;
            if (max_n > 0) {
                const dim3 grid((unsigned)(G * p.num_k_heads * seg));
                const hipError_t e = launch_prep_any(p, vp, grid, stream);
                if (e != hipSuccess) return e;
            }
            const hipError_t e = p.precise ? (nw == 4 ? launch_state_varlen<4, true>(vp, stream)
                                                      : launch_state_varlen<2, true>(vp, stream))
                                           : (nw == 4 ? launch_state_varlen<4, false>(vp, stream)
                                                      : launch_state_varlen<2, false>(vp, stream));
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace gdn
