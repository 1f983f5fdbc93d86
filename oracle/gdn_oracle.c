/*
 * gdn_oracle.c -- plain fp64 CPU reference of the Gated DeltaNet core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * the seeded input generators, which hold none of the method's arithmetic.
 *
 * Sources (all three are web pages; cited by title and passage):
 *   [GDN]   commit page "feat(stage-8c): linear-attention layer (Qwen3-Next
 *           GatedDeltaNet)" of the cortex repository -- passages "Block",
 *           "Discretisation", "Delta rule", "State", "Config extended",
 *           "Performance note", "8 unit tests".
 *   [QPR]   "Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and vLLM
 *           serving path" -- "Summary", "Why this is larger than a normal
 *           contrib model" (recurrent + conv checkpoints for prefix reuse).
 *   [CNPR]  "Add Qwen3-Coder-Next contrib model (80B/3B hybrid
 *           DeltaNet+MoE)" -- "Model Architecture" table (16 qk / 32 v heads).
 *
 * What is computed, per sequence b and value head h (key head h / (Hv/Hk),
 * the repeat-interleave sharing of [GDN] "8 unit tests"):
 *   front end  ([GDN] "Block"): depthwise causal conv of width K over the
 *              packed [q | k | v] channel stream, prepending the carried
 *              conv state; SiLU; optional rounding of the result to the
 *              I/O dtype; split per head; q and k scaled to unit L2 norm
 *              x * (sum x^2 + eps)^(-1/2).
 *   gates      ([GDN] "Discretisation"): g = -exp(A_log) * softplus(a + dt_bias),
 *              beta = sigmoid(b).
 *   recurrence ([GDN] "Delta rule"), token by token:
 *              S <- exp(g) S;  kv = S^T k;  delta = beta (v - kv);
 *              S <- S + k delta^T;  o = S^T q.
 *   state      ([GDN] "State"): conv tail = last K-1 pre-conv inputs, and
 *              the d_k x d_v recurrent state per value head.
 *   checkpoints ([QPR] "Summary"): the recurrent state and conv tail after
 *              every absolute position that is a multiple of the interval.
 *   output gate ([GDN] "Output"): RMSNormGated of the core output with z,
 *              applied to given o, z and norm weights (oracle_output_gate).
 *
 * Every quantity is carried in fp64.  The only rounding to a narrower type
 * is the optional rounding of the conv+SiLU output to bf16 (round to
 * nearest, ties to even, 8 significant bits), done by rounding_to_bf16()
 * below from the definition of the format.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t batch;        /* B                                             */
    int64_t seq_len;      /* L: tokens in this call                        */
    int64_t num_k_heads;  /* H_k                                           */
    int64_t num_v_heads;  /* H_v, a multiple of H_k                        */
    int64_t head_k_dim;   /* d_k                                           */
    int64_t head_v_dim;   /* d_v                                           */
    int64_t conv_kernel;  /* K (4 on the pages)                            */
    int64_t start_pos;    /* absolute position of the call's first token   */
    int64_t ckpt_interval;/* 0 = no checkpoints                            */
    int32_t io_bf16;      /* 1: io tensors are bf16 bit patterns, 0: fp32  */
    int32_t round_conv;   /* 1: round the conv+SiLU output to the io dtype */
    double q_scale;       /* multiplies the unit-norm query (1 = literal)   */
    double l2_eps;        /* epsilon inside the L2 norm                    */
} oracle_dims;

/* ---- scalar helpers, each from its textbook definition ----------------- */

static double io_read(const void* p, int bf16, int64_t i) {
    if (bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)p)[i];
}

static void io_copy(void* dst, int64_t di, const void* src, int64_t si, int bf16) {
    if (bf16) ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
    else ((float*)dst)[di] = ((const float*)src)[si];
}

/* Round to the nearest bf16 value (8 significant bits, exponent range of
 * fp32, ties to even).  x = m 2^e with 0.5 <= |m| < 1, so the spacing of
 * bf16 values around x is 2^(e-8), floored at the subnormal spacing 2^-133. */
double rounding_to_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);
    int q = e - 8;
    if (q < -133) q = -133;
    double y = ldexp(nearbyint(ldexp(x, -q)), q);
    if (fabs(y) > 3.3895313892515355e38) y = copysign(INFINITY, x);
    return y;
}

/* Round to the nearest fp32 value (the C cast is round-to-nearest-even). */
static double rounding_to_f32(double x) { return (double)(float)x; }

double oracle_softplus(double x) {
    /* log(1 + e^x) written so that neither branch overflows or cancels */
    return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

double oracle_silu(double x) { return x * oracle_sigmoid(x); }

/* x <- scale * x / sqrt(sum x^2 + eps): the l2norm of [GDN] "Block"; a zero
 * vector stays zero ([GDN] "8 unit tests" checks exactly that case). */
void oracle_l2_normalize(double* x, int64_t n, double eps, double scale) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    const double inv = scale / sqrt(ss + eps);
    for (int64_t i = 0; i < n; ++i) x[i] *= inv;
}

/* Output gate of [GDN] "Output": RMSNormGated(core output, z), per row of n
 * channels (one token and value head over d_v):
 *   y = w * o / sqrt(mean(o^2) + eps) * silu(z)
 * The page names the gated norm beside a plain norm written (1 + w) * x; the
 * gated one is read as scaling by w itself.  rows x n arrays, row-major. */
void oracle_output_gate(int64_t rows, int64_t n, const double* o, const double* z, const double* w,
                        double eps, double* y) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* orow = o + r * n;
        double ss = 0.0;
        for (int64_t j = 0; j < n; ++j) ss += orow[j] * orow[j];
        const double inv = 1.0 / sqrt(ss / (double)n + eps);
        for (int64_t j = 0; j < n; ++j) y[r * n + j] = w[j] * orow[j] * inv * oracle_silu(z[r * n + j]);
    }
}

/* g of [GDN] "Discretisation" */
double oracle_gate_g(double A_log, double a, double dt_bias) {
    return -exp(A_log) * oracle_softplus(a + dt_bias);
}

/* ---- front end for one channel at one token ----------------------------
 * Output at call-local token t of channel c: the causal cross-correlation
 *   y = sum_{j=0}^{K-1} w[c][j] * xt[t + j]
 * over the extended stream xt = conv_state_in[c][0..K-2] (oldest first)
 * followed by the call's tokens, so w[c][K-1] weights the current token.
 * Then u = SiLU(y), rounded to the io dtype when requested.            */
static double xt_at(const oracle_dims* d, const void* qkv, const void* conv_state_in,
                    int64_t b, int64_t c, int64_t idx /* into xt */) {
    const int64_t K1 = d->conv_kernel - 1;
    const int64_t H_k = d->num_k_heads, H_v = d->num_v_heads;
    const int64_t conv_dim = 2 * H_k * d->head_k_dim + H_v * d->head_v_dim;
    if (idx < K1) {
        if (!conv_state_in) return 0.0;
        return io_read(conv_state_in, d->io_bf16, (b * conv_dim + c) * K1 + idx);
    }
    return io_read(qkv, d->io_bf16, (b * d->seq_len + (idx - K1)) * conv_dim + c);
}

static double conv_silu(const oracle_dims* d, const void* qkv, const void* conv_w,
                        const void* conv_state_in, int64_t b, int64_t c, int64_t t) {
    const int64_t K = d->conv_kernel;
    double y = 0.0;
    for (int64_t j = 0; j < K; ++j)
        y += io_read(conv_w, d->io_bf16, c * K + j) * xt_at(d, qkv, conv_state_in, b, c, t + j);
    double u = oracle_silu(y);
    if (d->round_conv) u = d->io_bf16 ? rounding_to_bf16(u) : rounding_to_f32(u);
    return u;
}

/* Features of token t for sequence b and value head h:
 * qh[d_k], kh[d_k] (unit-normed), v[d_v], and the two gates. */
static void token_features(const oracle_dims* d, const void* qkv, const void* a, const void* bb,
                           const void* conv_w, const float* A_log, const float* dt_bias,
                           const void* conv_state_in, int64_t b, int64_t h, int64_t t,
                           double* qh, double* kh, double* v, double* g, double* beta) {
    const int64_t H_k = d->num_k_heads, H_v = d->num_v_heads;
    const int64_t dk = d->head_k_dim, dv = d->head_v_dim;
    const int64_t kh_idx = h / (H_v / H_k);
    const int64_t q_base = kh_idx * dk;
    const int64_t k_base = H_k * dk + kh_idx * dk;
    const int64_t v_base = 2 * H_k * dk + h * dv;
    for (int64_t i = 0; i < dk; ++i) {
        qh[i] = conv_silu(d, qkv, conv_w, conv_state_in, b, q_base + i, t);
        kh[i] = conv_silu(d, qkv, conv_w, conv_state_in, b, k_base + i, t);
    }
    oracle_l2_normalize(qh, dk, d->l2_eps, d->q_scale);
    oracle_l2_normalize(kh, dk, d->l2_eps, 1.0);
    for (int64_t j = 0; j < dv; ++j) v[j] = conv_silu(d, qkv, conv_w, conv_state_in, b, v_base + j, t);
    const int64_t gi = (b * d->seq_len + t) * H_v + h;
    *g = oracle_gate_g((double)A_log[h], io_read(a, d->io_bf16, gi), (double)dt_bias[h]);
    *beta = oracle_sigmoid(io_read(bb, d->io_bf16, gi));
}

/* One token of [GDN] "Delta rule" on a row-major d_k x d_v state S. */
static void delta_rule_token(int64_t dk, int64_t dv, double* S, const double* q, const double* k,
                             const double* v, double g, double beta, double* o, double* tmp) {
    const double decay = exp(g);
    for (int64_t i = 0; i < dk * dv; ++i) S[i] *= decay;
    for (int64_t j = 0; j < dv; ++j) tmp[j] = 0.0;            /* kv = S^T k   */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) tmp[j] += S[i * dv + j] * k[i];
    for (int64_t j = 0; j < dv; ++j) tmp[j] = beta * (v[j] - tmp[j]);   /* delta */
    for (int64_t i = 0; i < dk; ++i)                           /* S += k delta^T */
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += k[i] * tmp[j];
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;              /* o = S^T q   */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) o[j] += S[i * dv + j] * q[i];
}

/* Slots this call emits: absolute positions p in (start_pos, start_pos+L]
 * with p % interval == 0; slot index p / interval - 1. */
static int64_t first_slot(const oracle_dims* d) {
    return d->ckpt_interval > 0 ? d->start_pos / d->ckpt_interval : 0;
}
int64_t oracle_ckpt_count(const oracle_dims* d) {
    if (d->ckpt_interval <= 0) return 0;
    return (d->start_pos + d->seq_len) / d->ckpt_interval - d->start_pos / d->ckpt_interval;
}

/* ---- the whole layer for a selection of value heads --------------------
 * Inputs (io dtype = bf16 bits or fp32 per dims->io_bf16):
 *   qkv [B, L, conv_dim], a, b [B, L, H_v], conv_w [conv_dim, K],
 *   A_log, dt_bias [H_v] fp32, conv_state_in [B, conv_dim, K-1] or NULL (zeros),
 *   S0 [B, H_v, d_k, d_v] fp64 or NULL (zeros).
 *   heads[nsel]: value heads to compute (NULL = all, nsel = H_v).
 * Outputs (fp64, compact over the selection):
 *   out [B, L, nsel, d_v], S_out [B, nsel, d_k, d_v],
 *   ckpt_S [n_ckpt, B, nsel, d_k, d_v] (NULL to skip).
 * Returns 0, or -1 on a bad argument. */
int oracle_layer(const oracle_dims* d, const void* qkv, const void* a, const void* bb,
                 const void* conv_w, const float* A_log, const float* dt_bias,
                 const void* conv_state_in, const double* S0, const int64_t* heads, int64_t nsel,
                 double* out, double* S_out, double* ckpt_S) {
    const int64_t B = d->batch, L = d->seq_len, H_v = d->num_v_heads;
    const int64_t dk = d->head_k_dim, dv = d->head_v_dim;
    if (B < 0 || L < 0 || d->num_k_heads <= 0 || H_v % d->num_k_heads || dk <= 0 || dv <= 0 ||
        d->conv_kernel < 1 || nsel < 0)
        return -1;
    if (!heads) nsel = H_v;
    for (int64_t si = 0; heads && si < nsel; ++si)
        if (heads[si] < 0 || heads[si] >= H_v) return -1;
    const int64_t s0 = first_slot(d);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t si = 0; si < nsel; ++si) {
            const int64_t h = heads ? heads[si] : si;
            double* S = (double*)malloc(sizeof(double) * (dk * dv + 2 * dk + 3 * dv));
            double* q = S + dk * dv;
            double* k = q + dk;
            double* v = k + dk;
            double* o = v + dv;
            double* tmp = o + dv;
            for (int64_t i = 0; i < dk * dv; ++i)
                S[i] = S0 ? S0[((b * H_v + h) * dk * dv) + i] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double g, beta;
                token_features(d, qkv, a, bb, conv_w, A_log, dt_bias, conv_state_in, b, h, t,
                               q, k, v, &g, &beta);
                delta_rule_token(dk, dv, S, q, k, v, g, beta, o, tmp);
                double* od = out + ((b * L + t) * nsel + si) * dv;
                for (int64_t j = 0; j < dv; ++j) od[j] = o[j];
                const int64_t p = d->start_pos + t + 1;
                if (ckpt_S && d->ckpt_interval > 0 && p % d->ckpt_interval == 0) {
                    const int64_t slot = p / d->ckpt_interval - 1 - s0;
                    double* cd = ckpt_S + ((slot * B + b) * nsel + si) * dk * dv;
                    memcpy(cd, S, sizeof(double) * dk * dv);
                }
            }
            memcpy(S_out + (b * nsel + si) * dk * dv, S, sizeof(double) * dk * dv);
            free(S);
        }
    }
    return 0;
}

/* ---- carried conv state -------------------------------------------------
 * conv_state_out[b][c][j] = xt[L + j] for j < K-1: the last K-1 pre-conv
 * inputs of the extended stream, copied bit for bit ([GDN] "State").
 * ckpt_conv [n_ckpt, B, conv_dim, K-1]: the same tail at each checkpoint
 * position (NULL to skip). */
int oracle_conv_tail(const oracle_dims* d, const void* qkv, const void* conv_state_in,
                     void* conv_state_out, void* ckpt_conv) {
    const int64_t B = d->batch, L = d->seq_len, K1 = d->conv_kernel - 1;
    const int64_t conv_dim = 2 * d->num_k_heads * d->head_k_dim + d->num_v_heads * d->head_v_dim;
    const int64_t n_ck = oracle_ckpt_count(d), s0 = first_slot(d);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < conv_dim; ++c)
            for (int64_t j = 0; j < K1; ++j) {
                /* xt index of the tail entry j after consuming n tokens is n + j */
                const int64_t dst = (b * conv_dim + c) * K1 + j;
                for (int64_t s = -1; s < n_ck; ++s) {
                    int64_t n;
                    void* target;
                    int64_t di = dst;
                    if (s < 0) { n = L; target = conv_state_out; }
                    else {
                        if (!ckpt_conv) break;
                        n = (s0 + s + 1) * d->ckpt_interval - d->start_pos;
                        target = ckpt_conv;
                        di = s * B * conv_dim * K1 + dst;
                    }
                    if (!target) continue;
                    const int64_t idx = n + j;
                    if (idx < K1) {
                        if (conv_state_in) io_copy(target, di, conv_state_in, (b * conv_dim + c) * K1 + idx, d->io_bf16);
                        else if (d->io_bf16) ((uint16_t*)target)[di] = 0;
                        else ((float*)target)[di] = 0.0f;
                    } else {
                        io_copy(target, di, qkv, (b * L + (idx - K1)) * conv_dim + c, d->io_bf16);
                    }
                }
            }
    return 0;
}

/* ---- front end alone, materialised (for pins and kernel debugging) ------
 * q_hat, k_hat [B, L, H_k, d_k]; v [B, L, H_v, d_v]; g, beta [B, L, H_v]. */
int oracle_frontend(const oracle_dims* d, const void* qkv, const void* a, const void* bb,
                    const void* conv_w, const float* A_log, const float* dt_bias,
                    const void* conv_state_in, double* q_hat, double* k_hat, double* v,
                    double* g, double* beta) {
    const int64_t B = d->batch, L = d->seq_len, H_k = d->num_k_heads, H_v = d->num_v_heads;
    const int64_t dk = d->head_k_dim, dv = d->head_v_dim, r = H_v / H_k;
    if (H_v % H_k) return -1;
    double* qt = (double*)malloc(sizeof(double) * (2 * dk + dv));
    double* kt = qt + dk;
    double* vt = kt + dk;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < L; ++t)
            for (int64_t h = 0; h < H_v; ++h) {
                double gg, bt;
                token_features(d, qkv, a, bb, conv_w, A_log, dt_bias, conv_state_in, b, h, t,
                               qt, kt, vt, &gg, &bt);
                const int64_t bth = (b * L + t) * H_v + h;
                g[bth] = gg;
                beta[bth] = bt;
                memcpy(v + bth * dv, vt, sizeof(double) * dv);
                if (h % r == 0) {
                    const int64_t btk = (b * L + t) * H_k + h / r;
                    memcpy(q_hat + btk * dk, qt, sizeof(double) * dk);
                    memcpy(k_hat + btk * dk, kt, sizeof(double) * dk);
                }
            }
    free(qt);
    return 0;
}

/* ---- the recurrence alone on given features ------------------------------
 * q_hat, k_hat [B, L, H_k, d_k]; v [B, L, H_v, d_v]; g, beta [B, L, H_v];
 * S0 [B, H_v, d_k, d_v] or NULL.  out [B, L, H_v, d_v]; S_out [B, H_v, d_k, d_v]. */
int oracle_core(const oracle_dims* d, const double* q_hat, const double* k_hat, const double* v,
                const double* g, const double* beta, const double* S0, double* out, double* S_out) {
    const int64_t B = d->batch, L = d->seq_len, H_k = d->num_k_heads, H_v = d->num_v_heads;
    const int64_t dk = d->head_k_dim, dv = d->head_v_dim;
    if (H_v % H_k) return -1;
    const int64_t r = H_v / H_k;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H_v; ++h) {
            double* S = S_out + (b * H_v + h) * dk * dv;
            double* tmp = (double*)malloc(sizeof(double) * dv);
            for (int64_t i = 0; i < dk * dv; ++i) S[i] = S0 ? S0[(b * H_v + h) * dk * dv + i] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t btk = (b * L + t) * H_k + h / r, bth = (b * L + t) * H_v + h;
                delta_rule_token(dk, dv, S, q_hat + btk * dk, k_hat + btk * dk, v + bth * dv,
                                 g[bth], beta[bth], out + bth * dv, tmp);
            }
            free(tmp);
        }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
