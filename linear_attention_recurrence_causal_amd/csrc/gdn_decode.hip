// gdn_decode.hip -- one recurrent decode step of the Gated DeltaNet core (gfx950).
//
// Rule (cortex commit "feat(stage-8c): linear-attention layer (Qwen3-Next
// GatedDeltaNet)", passages "Block", "Discretisation", "Delta rule"): for the
// new token of sequence b and value head h,
//   u = SiLU(causal conv over [conv_state_in | x]) rounded to the io dtype,
//   q = l2norm(u_q) * q_scale, k = l2norm(u_k), v = u_v,
//   g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b),
//   S' = exp(g) S; delta = beta (v - S'^T k); S = S' + k delta^T;
//   o = S^T q = S'^T q + delta (k . q).
//
// Memory-bound by design: the fp32 state (d_k x d_v per head, 64 KiB at 128)
// is read once and written once; everything else is < 3% of the bytes.  The
// few front-end inputs are requested before the state, so the conv, norms and
// gates are done by the time the state arrives.
// One workgroup owns a (b, h, NCOL-column slice) of S.  Columns of S are
// independent given (q, k, beta, g), so slicing d_v multiplies parallelism;
// each slice recomputes the (cheap) conv of its head's q and k channels.
//
// With the output gate (GATE; "Output": RMSNormGated(o, z), per token and
// head over d_v) a workgroup owns all d_v columns of its head, so the row's
// sum of squares stays on chip and y = w o / sqrt(mean(o^2) + eps) silu(z)
// is formed from the fp32 o before any rounding.
//
// Thread layout (256 threads, 512 for 128-column slices): thread = (cq, rg),
// cq = column quad (4
// consecutive fp32 columns = one 16-byte load), rg = row group; thread owns
// rows rg, rg + NRG, ... so that for each row step the whole workgroup reads
// NRG full row segments with 16-byte coalesced loads.  S' lives in registers
// between the read and the write.  Reductions over rows use a fixed
// butterfly + fixed cross-wave order (deterministic, no atomics).
#include <cstdlib>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kDecodeThreads = 256;

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// Buffer resource over one head's slice [base, base + bytes) of a state
// snapshot, with raw byte offsets: one 32-bit offset per lane inside the
// d_k x d_v slice (64 KiB at d = 128), whatever the snapshot's total size.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t snap_rsrc(const float* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}

// A wave-uniform 64-bit value in scalar registers (the compiler forms some
// 64-bit products of uniform values on the vector unit, one copy per lane)
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// MAXT: tokens per call the kernel is built for (1: the one-token step,
// whose 64-column split fits seven waves per SIMD; kMaxDecodeTokens: the
// multi-token step, four waves per SIMD).  Every token's conv, norms and
// gates are formed before the token loop, into LDS.  The arithmetic per
// token is the same in both, so T tokens in one call equal T one-token calls
// bit for bit.  GATE: also write the gated output (NCOL must be d_v).
template <typename IO, int DK, int NCOL, int MAXT, bool GATE, int THREADS = kDecodeThreads>
__global__ __launch_bounds__(THREADS, MAXT > 1 ? (THREADS == 512 && !GATE ? 6 : 4)
                                               : (THREADS == 512 ? 6 : (NCOL == 64 && !GATE ? 7 : (NCOL == 128 ? 4 : 1))))
void decode_step_kernel(DecodeParams p) {
    using T = io_traits<IO>;
    constexpr int NCQ = NCOL / 4;                 // column quads per slice
    constexpr int NRG = THREADS / NCQ;            // row groups
    constexpr int RPT = DK / NRG;                 // rows per thread
    static_assert(RPT * NRG == DK && NCQ * NRG == THREADS, "bad decode tiling");
    constexpr int NCH = 2 * DK + NCOL;            // conv channels this slice needs
    constexpr int NWAVES = THREADS / 64;
    constexpr int CPT = (NCH + THREADS - 1) / THREADS;   // channels per thread

    __shared__ float u_s[MAXT][NCH];              // conv+SiLU outputs (io-rounded) per token
    __shared__ float red_s[2][NWAVES][NCOL];      // cross-wave partial sums
    __shared__ __align__(16) float delta_s[NCOL];
    __shared__ float scal_s[MAXT][4];             // per token: q.q, k.k, k.q (unnormalised), g
    __shared__ float beta_s[MAXT];
    __shared__ float gsum_s[NWAVES];              // gate: per-wave sums of o^2
    __shared__ float gzw_s[GATE ? MAXT : 1][GATE ? NCOL : 1];   // gate: w silu(z) per token and column

    const int tid = threadIdx.x;
    const int z = blockIdx.x;                     // column slice
    const int h = blockIdx.y;                     // value head
    const int b = blockIdx.z;                     // sequence
    const int r = p.num_v_heads / p.num_k_heads;
    const int kh = h / r;
    const int dv = p.head_v_dim;
    const int64_t conv_dim = p.conv_dim;
    const int col0 = z * NCOL;
    const int ntok = MAXT == 1 ? 1 : p.num_tokens;   // the one-token kernel runs straight through
    float* const rec_snap = MAXT == 1 ? nullptr : p.rec_snap;
    void* const conv_snap = MAXT == 1 ? nullptr : p.conv_snap;
    const int cq = tid % NCQ;
    const int rg = tid / NCQ;
    const int wave = tid / 64, lane = tid % 64;

    // ---- 1. front-end inputs of the slice's channels for every token: few
    // bytes, requested first so that they return (in issue order) ahead of
    // the state, and token 0's conv, norms and gates run while the state is
    // still in flight
    const bool write_qk_tail = (h % r == 0) && (z == 0);
    float hist[CPT][3];              // the last three pre-conv inputs (carried conv state)
    float taps[CPT][4];
    float xin[CPT][MAXT];
    int64_t fcs[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int i = tid + k * THREADS;
        if (i < NCH) {
            int64_t c;
            if (i < DK) c = (int64_t)kh * DK + i;
            else if (i < 2 * DK) c = (int64_t)p.num_k_heads * DK + (int64_t)kh * DK + (i - DK);
            else c = 2 * (int64_t)p.num_k_heads * DK + (int64_t)h * dv + col0 + (i - 2 * DK);
            const int64_t cs = ((int64_t)b * conv_dim + c) * 3;
            fcs[k] = cs;
#pragma unroll
            for (int j = 0; j < 3; ++j) hist[k][j] = p.conv_in ? T::load(p.conv_in, cs + j) : 0.f;
#pragma unroll
            for (int t = 0; t < MAXT; ++t)
                if (t < ntok) xin[k][t] = T::load(p.qkv, ((int64_t)b * ntok + t) * conv_dim + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) taps[k][j] = T::load(p.conv_w, c * 4 + j);
        }
    }
    float gate_a[MAXT], gate_b[MAXT];
    if (wave == 3 && lane == 0) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t)
            if (t < ntok) {
                const int64_t gi = ((int64_t)b * ntok + t) * p.num_v_heads + h;
                gate_a[t] = T::load(p.a, gi);
                gate_b[t] = T::load(p.b, gi);
            }
    }
    const float neg_A = -expf(p.A_log[h]), dt_h = p.dt_bias[h];
    // gate inputs of this thread's column (threads tid < NCOL = d_v)
    float zin[MAXT], gw = 0.f;
    if (GATE && tid < NCOL) {
        gw = T::load(p.gate_w, tid);
#pragma unroll
        for (int t = 0; t < MAXT; ++t)
            if (t < ntok) zin[t] = T::load(p.gate_z, (((int64_t)b * ntok + t) * p.num_v_heads + h) * dv + tid);
    }

    // ---- 2. the state slice (the bytes that matter), kept in registers for
    // all the tokens.  The one-token build requests it here, behind the
    // front-end inputs, so that its front end runs while the state is in
    // flight; the multi-token build requests it after its tokens' conv
    // (below), so that the tokens' inputs and the state are not in registers
    // together.
    // This thread's state elements: the head's d_k x d_v slice (a uniform
    // base) plus a 32-bit offset inside it, row i at + i NRG dv.
    const int64_t head_base = uniform64(((int64_t)b * p.num_v_heads + h) * DK * dv);
    const int lane_off = col0 + cq * 4 + rg * dv;
    const int64_t state_elems = (int64_t)p.batch * p.num_v_heads * DK * dv;
    float4 S[RPT];
    // the one-token build keeps a per-lane 64-bit base (fewer registers
    // there); the multi-token build a uniform base and 32-bit offsets
    const int64_t s_base = head_base + col0 + cq * 4;
    auto elem = [&](const float* base, int i) {
        return MAXT == 1 ? base + s_base + (int64_t)(rg + i * NRG) * dv
                         : (base + head_base) + (lane_off + i * NRG * dv);
    };
    auto load_state = [&] {
        if (p.rec_in) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) S[i] = *reinterpret_cast<const float4*>(elem(p.rec_in, i));
        } else {
#pragma unroll
            for (int i = 0; i < RPT; ++i) S[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if (MAXT == 1) load_state();

    // the gate factors w silu(z) go to LDS once, so that no gate input stays
    // in a register through the state arithmetic
    if (GATE && tid < NCOL) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t)
            if (t < ntok) gzw_s[t][tid] = gw * silu_f32(zin[t]);
    }

    // ---- 3. every token's front end, none of which depends on the state, so
    // it runs while the state is in flight and leaves two barriers per token
    // to the token loop.  Conv + SiLU of the slice's channels (io-rounded)
    // into u_s[t]; the carried tail moves on token by token (to that token's
    // conv snapshot, and after the last token to conv_out).
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        if (t >= ntok) break;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int i = tid + k * THREADS;
            if (i < NCH) {
                const float x = xin[k][t];
                const float y = fmaf(taps[k][3], x, fmaf(taps[k][2], hist[k][2],
                                                         fmaf(taps[k][1], hist[k][1], taps[k][0] * hist[k][0])));
                u_s[t][i] = T::round(silu_f32(y));
                hist[k][0] = hist[k][1];
                hist[k][1] = hist[k][2];
                hist[k][2] = x;
                if (i >= 2 * DK || write_qk_tail) {
                    if (conv_snap) {
                        const int64_t cs = (int64_t)t * p.batch * conv_dim * 3 + fcs[k];
#pragma unroll
                        for (int j = 0; j < 3; ++j) T::store(conv_snap, cs + j, hist[k][j]);
                    }
                    if (t == ntok - 1)
#pragma unroll
                        for (int j = 0; j < 3; ++j) T::store(p.conv_out, fcs[k] + j, hist[k][j]);
                }
            }
        }
    }
    if (MAXT > 1) load_state();
    __syncthreads();
    // q.q, k.k and k.q of every token (item 3t + kind, one wave each, fixed
    // order), and the gates (the lane that loaded them)
    for (int it = wave; it < 3 * ntok; it += NWAVES) {
        const int t = it / 3, kind = it % 3;
        float acc = 0.f;
        for (int i = lane; i < DK; i += 64) {
            const float qv = u_s[t][i], kv = u_s[t][DK + i];
            acc = fmaf(kind == 1 ? kv : qv, kind == 0 ? qv : kv, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) scal_s[t][kind] = acc;
    }
    if (wave == 3 && lane == 0) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t)
            if (t < ntok) {
                scal_s[t][3] = neg_A * softplus_f32(gate_a[t] + dt_h);
                beta_s[t] = sigmoid_f32(gate_b[t]);
            }
    }
    __syncthreads();

    for (int t = 0; t < ntok; ++t) {
        const float n_q = p.q_scale / sqrtf(scal_s[t][0] + p.l2_eps);
        const float n_k = 1.0f / sqrtf(scal_s[t][1] + p.l2_eps);
        const float kq = scal_s[t][2] * n_q * n_k;     // k_hat . q_hat
        const float decay = expf(scal_s[t][3]);
        const float beta = beta_s[t];

        // ---- 4. S' = exp(g) S; partial S'^T k and S'^T q over this thread's rows
        float kv[4] = {0.f, 0.f, 0.f, 0.f}, oq[4] = {0.f, 0.f, 0.f, 0.f};
        float krow[MAXT == 1 ? RPT : 1];   // the multi-token build forms k again in step 6
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + i * NRG;
            const float kk = u_s[t][DK + row] * n_k;
            const float qq = u_s[t][row] * n_q;
            if (MAXT == 1) krow[i] = kk;
            S[i].x *= decay; S[i].y *= decay; S[i].z *= decay; S[i].w *= decay;
            kv[0] = fmaf(S[i].x, kk, kv[0]); kv[1] = fmaf(S[i].y, kk, kv[1]);
            kv[2] = fmaf(S[i].z, kk, kv[2]); kv[3] = fmaf(S[i].w, kk, kv[3]);
            oq[0] = fmaf(S[i].x, qq, oq[0]); oq[1] = fmaf(S[i].y, qq, oq[1]);
            oq[2] = fmaf(S[i].z, qq, oq[2]); oq[3] = fmaf(S[i].w, qq, oq[3]);
        }
        // reduce over the row groups of this wave (lanes differing in the rg bits)
#pragma unroll
        for (int m = NCQ; m < 64; m <<= 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kv[j] += __shfl_xor(kv[j], m, 64);
                oq[j] += __shfl_xor(oq[j], m, 64);
            }
        }
        if (lane < NCQ) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                red_s[0][wave][cq * 4 + j] = kv[j];
                red_s[1][wave][cq * 4 + j] = oq[j];
            }
        }
        __syncthreads();

        // ---- 5. delta and o per column
        const int64_t oi = (((int64_t)b * ntok + t) * p.num_v_heads + h) * dv + col0 + tid;
        float o = 0.f;
        if (tid < NCOL) {
            float skv = 0.f, soq = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) { skv += red_s[0][w][tid]; soq += red_s[1][w][tid]; }
            const float vv = u_s[t][2 * DK + tid];
            const float d = beta * (vv - skv);
            delta_s[tid] = d;
            o = fmaf(d, kq, soq);
            if (!GATE || p.out) T::store(p.out, oi, o);
        }
        if (GATE) {
            // sum of o^2 over the head's d_v columns (waves 0 .. NCOL/64)
            const float sq = wave_sum(o * o);
            if (lane == 0) gsum_s[wave] = sq;
        }
        __syncthreads();
        if (GATE && tid < NCOL) {
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < (NCOL + 63) / 64; ++w) ss += gsum_s[w];
            const float inv = 1.0f / sqrtf(ss * (1.0f / NCOL) + p.gate_eps);
            T::store(p.gate_y, oi, (o * inv) * gzw_s[t][tid]);
        }

        // ---- 6. S = S' + k delta^T (this token's snapshot, if asked for)
        const float4 dl = *reinterpret_cast<const float4*>(&delta_s[cq * 4]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kk = MAXT == 1 ? krow[i] : u_s[t][DK + rg + i * NRG] * n_k;   // the same product
            S[i].x = fmaf(kk, dl.x, S[i].x); S[i].y = fmaf(kk, dl.y, S[i].y);
            S[i].z = fmaf(kk, dl.z, S[i].z); S[i].w = fmaf(kk, dl.w, S[i].w);
        }
        if (rec_snap) {
            // snapshot t through a buffer resource: a uniform base and one
            // 32-bit offset per lane, rather than a 64-bit address per row
            const __amdgpu_buffer_rsrc_t rs = snap_rsrc(rec_snap + t * state_elems + head_base, DK * dv * 4);
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const v4u32*>(&S[i]), rs,
                                                       (lane_off + i * NRG * dv) * 4, 0, 0);
        }
    }

    // ---- 7. the state, once
#pragma unroll
    for (int i = 0; i < RPT; ++i) *reinterpret_cast<float4*>(const_cast<float*>(elem(p.rec_out, i))) = S[i];
}

// 128-column workgroups (the gated step's, and GDN_DECODE_COLS=128) take 512
// threads, so that each thread holds as few state rows as in the 64-column
// step and the CU keeps more waves resident; gated and ungated 128-column
// steps then sum their rows in the same order.
template <typename IO, int DK, int NCOL, bool GATE>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
    constexpr int TH = NCOL == 128 ? 512 : kDecodeThreads;
    dim3 grid(p.head_v_dim / NCOL, p.num_v_heads, p.batch);
    if (p.num_tokens == 1 && !p.rec_snap && !p.conv_snap)
        hipLaunchKernelGGL((decode_step_kernel<IO, DK, NCOL, 1, GATE, TH>), grid, dim3(TH), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_step_kernel<IO, DK, NCOL, kMaxDecodeTokens, GATE, TH>), grid, dim3(TH), 0, stream,
                           p);
    return hipGetLastError();
}

// Columns of S per workgroup: all d_v by default (a workgroup owns a head;
// at d_v = 128, 512 threads with eight state rows each; on the 32 x 48 head
// decode measured at least as fast as 64 columns for 1..8 tokens, and
// faster with the Infinity Cache cold); GDN_DECODE_COLS = 32 / 64 / 128
// selects another split.  The gated step always takes all d_v columns.
template <typename IO, int DK>
hipError_t launch_dk(const DecodeParams& p, hipStream_t stream) {
    if (p.gate_y) {
        switch (p.head_v_dim) {
            case 32: return launch_typed<IO, DK, 32, true>(p, stream);
            case 64: return launch_typed<IO, DK, 64, true>(p, stream);
            case 128: return launch_typed<IO, DK, 128, true>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    int cols = p.head_v_dim;
    if (const char* env = getenv("GDN_DECODE_COLS")) {
        const int v = atoi(env);
        if ((v == 32 || v == 64 || v == 128) && v <= p.head_v_dim) cols = v;
    }
    switch (cols) {
        case 32: return launch_typed<IO, DK, 32, false>(p, stream);
        case 64: return launch_typed<IO, DK, 64, false>(p, stream);
        case 128: return launch_typed<IO, DK, 128, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename IO>
hipError_t launch_io(const DecodeParams& p, hipStream_t stream) {
    switch (p.head_k_dim) {
        case 32: return launch_dk<IO, 32>(p, stream);
        case 64: return launch_dk<IO, 64>(p, stream);
        case 128: return launch_dk<IO, 128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int head_k_dim, int head_v_dim, int io_dtype) {
    auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
    return ok(head_k_dim) && ok(head_v_dim) && (io_dtype == GDN_F32 || io_dtype == GDN_BF16);
}

hipError_t launch_decode_step(const DecodeParams& p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    return p.io_dtype == GDN_BF16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace gdn
