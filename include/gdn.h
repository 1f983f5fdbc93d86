/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet core library (libgdn.so).
 *
 * The operation ("the GDN core") is the per-head gated delta rule with its
 * front end, as stated on the cortex commit page "feat(stage-8c):
 * linear-attention layer (Qwen3-Next GatedDeltaNet)":
 *   - "Block": depthwise causal Conv1d (kernel 4) over the packed projected
 *     q|k|v stream, prepending the carried conv state; SiLU; split into
 *     heads; L2 normalisation of q and k.
 *   - "Discretisation": g = -exp(A_log) * softplus(a + dt_bias) and
 *     beta = sigmoid(b), both in fp32.
 *   - "Delta rule": per token, S <- exp(g) S; kv = S^T k; delta = beta (v - kv);
 *     S <- S + k delta^T; o = S^T q (with the updated S).
 *   - "State": the carried conv tail and the d_k x d_v recurrent state per
 *     value head; a new request starts from cleared (zero) state.
 *   - "Performance note": prefill evaluates the same rule in chunks of 64.
 * Checkpoints of the recurrent and conv state at fixed positions make a
 * prefix resumable ("Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and
 * vLLM serving path", "Summary" and "Why this is larger than a normal
 * contrib model").
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is caller-owned device memory (HIP, the current
 *     device) unless marked "host".  The library never allocates, frees or
 *     synchronises; it enqueues kernels on `stream` (a hipStream_t, NULL =
 *     the null stream) and returns.  It keeps no global mutable state.
 *   - Arguments are validated before anything is enqueued.  On a validation
 *     error (GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EALIAS, GDN_ESPACE) nothing is
 *     enqueued and no output is touched.  No C++ exception crosses this
 *     boundary.
 *   - GDN_EHIP means the HIP runtime refused a launch.  A call that launches
 *     several kernels (a prefill run segment by segment through a small
 *     workspace, a varlen prefill over several groups) stops at the first
 *     refused launch and returns GDN_EHIP; the kernels launched before it
 *     stay enqueued, so the outputs are then partly written and must be
 *     treated as undefined.
 *   - Tensors are dense, row-major, with the shapes given below.  Every
 *     pointer needs the alignment of its element type; in addition qkv and
 *     out of gdn_prefill_chunked and both recurrent states of gdn_decode_step
 *     must be 16-byte aligned, and ckpt_buf 256-byte aligned.
 *   - Packed channel order (conv_dim = 2*H_k*d_k + H_v*d_v): all q channels
 *     (key head major), then all k channels, then all v channels (value head
 *     major).  conv_w rows follow the same order.
 *   - Value head h reads key head h / (H_v / H_k) (repeat-interleave).
 *   - io dtype (qkv, a, b, conv_w, conv_state, out): GDN_F32 or GDN_BF16.
 *     A_log, dt_bias and the recurrent state are always fp32.
 *   - conv_state [B, conv_dim, K-1]: per channel the last K-1 pre-conv inputs,
 *     oldest first.  (The cortex state keeps K columns; its oldest is never
 *     read by a width-K causal conv of the next token, so K-1 are stored.)
 *   - rec_state [B, H_v, d_k, d_v] fp32, d_v contiguous.
 *
 * Environment overrides (read at each call; for tests and tuning, the
 * defaults are the measured best):
 *   GDN_PREFILL_PATH=fused|split   prefill path when a workspace is given
 *   GDN_PREFILL_STATE_WAVES=2|4     compute waves per two-pass state workgroup
 *   GDN_PREFILL_WAVES=2|4|8         waves per fused prefill workgroup
 *   GDN_DIAG_SOLVE=neumann          diagonal-block inverses by the Neumann
 *                                   product (two-pass path)
 *   GDN_DECODE_COLS=32|64|128       state columns per decode workgroup (the
 *                                   gated step always takes all d_v)
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gdn_status;
enum {
    GDN_OK = 0,
    GDN_EINVAL = 1,       /* null / misaligned pointer, bad size or config   */
    GDN_EUNSUPPORTED = 2, /* valid but no kernel for this shape / dtype      */
    GDN_EALIAS = 3,       /* forbidden overlap between an output and input   */
    GDN_ESPACE = 4,       /* checkpoint buffer / entry array / workspace too small */
    GDN_EHIP = 5          /* the HIP runtime reported a launch error         */
};

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Operand precision of the chunked prefill's MFMA products (the decode step
 * is fp32 throughout and ignores it).
 *   GDN_PRECISION_DEFAULT: raw bf16 q/k/v are exact MFMA operands, norms,
 *     beta and decays are fp32 row scales, the product that builds the state
 *     takes Delta as bf16 hi + lo; the other state-path operands (S0 in K S0
 *     and Q S0, the triangular solve's coupling and diagonal blocks, P and
 *     Delta in P Delta) are single bf16.
 *   GDN_PRECISION_HILO: the triangular solve's coupling and diagonal
 *     blocks and P and Delta in P Delta as bf16 hi + lo (about 16
 *     significant bits; three MFMAs per product), for inputs where the
 *     triangular solve cancels heavily (keys that nearly coincide, beta near
 *     1, slow decay); S0 stays single bf16, as in the default, which measured
 *     no worse on those inputs.  About 1.4x the state-path MFMA work, and
 *     12.75 KiB more workspace per value head and chunk.
 * The solve is the stable direct one of the Qwen3.6-27B PR ("Known
 * limitations and follow-ups") in both. */
typedef enum { GDN_PRECISION_DEFAULT = 0, GDN_PRECISION_HILO = 1 } gdn_precision;

/* Layer shape and numerics.  Supported today: conv_kernel 4, chunk 64;
 * prefill: d_k = d_v = 128, io GDN_BF16, B * H_v <= 2^20; decode: d_k, d_v
 * in {32, 64, 128}, io GDN_F32 or GDN_BF16, B and H_v <= 65535.  Larger
 * shapes get GDN_EUNSUPPORTED (they would exceed a launch's grid). */
typedef struct gdn_config {
    int32_t batch;        /* B >= 0                                          */
    int32_t num_k_heads;  /* H_k >= 1                                        */
    int32_t num_v_heads;  /* H_v, a positive multiple of H_k                 */
    int32_t head_k_dim;   /* d_k                                             */
    int32_t head_v_dim;   /* d_v                                             */
    int32_t conv_kernel;  /* K                                               */
    int32_t chunk;        /* prefill chunk length C                          */
    int32_t io_dtype;     /* gdn_dtype                                       */
    float q_scale;        /* factor on the unit-norm query; 1 = the pages' rule */
    float l2_eps;         /* epsilon in x * (sum x^2 + eps)^(-1/2), >= 0      */
    int32_t precision;    /* gdn_precision of the prefill (0 = default)        */
} gdn_config;

/* One emitted checkpoint slot.  Slot j holds the state after absolute
 * position (j+1)*interval; its conv tail sits at ckpt_buf + conv_offset
 * ([B, conv_dim, K-1], io dtype) and its recurrent state at ckpt_buf +
 * rec_offset ([B, H_v, d_k, d_v], fp32). */
typedef struct gdn_ckpt_entry {
    int64_t slot;
    int64_t position;
    uint64_t conv_offset;
    uint64_t rec_offset;
} gdn_ckpt_entry;

/* Checkpoint plan of a prefill call (host only, touches no device).
 *   The call covers absolute positions [start_pos, start_pos + seq_len); it
 *   emits slot j for every position p = (j+1)*interval in
 *   (start_pos, start_pos + seq_len].  slot_bytes = align256(B*conv_dim*(K-1)*
 *   io_size) + align256(B*H_v*d_k*d_v*4); conv_offset = slot*slot_bytes;
 *   rec_offset = conv_offset + align256(B*conv_dim*(K-1)*io_size).
 *   *count      (host, required): slots emitted.
 *   *buffer_bytes (host, required): bytes a ckpt_buf needs for this call,
 *                 (last emitted slot + 1) * slot_bytes, 0 if none.
 *   entries     (host, nullable): filled with up to `capacity` entries.
 * Errors: GDN_EINVAL (bad config, start_pos/seq_len < 0, interval < 0 or not
 * a multiple of cfg->chunk, null count/buffer_bytes); GDN_ESPACE when
 * entries != NULL and capacity < *count (count and bytes are still set). */
gdn_status gdn_state_checkpoint(const gdn_config* cfg, int64_t start_pos, int64_t seq_len,
                                int64_t interval, gdn_ckpt_entry* entries, int64_t capacity,
                                int64_t* count, uint64_t* buffer_bytes);

/* Workspace for the two-pass prefill (host only): the bytes with which a call
 * of seq_len tokens per sequence (any start_pos) runs each pass once,
 *   B * n * (H_k * 32768 + H_v * 13568)  (n: chunks the call can span)
 * plus, from n = 2 on, 8 * (B * H_k * roundup(n, 32) + 1024) for the ready
 * flags of the overlapped prep (see gdn_prefill_chunked).
 * The chunked form splits into per-chunk work that does not depend on the
 * state and a short recurrence over chunks that does ("Performance note");
 * with a workspace the first part runs for every chunk in parallel and only
 * the second runs chunk by chunk, which is the faster path at every batch
 * size measured.  A smaller workspace, down to one chunk's worth (the value
 * for seq_len = 1), is used segment by segment.  With less than that, or
 * NULL, or a head group H_v / H_k above 8, gdn_prefill_chunked runs a fused
 * single-pass kernel that keeps every intermediate on chip (the environment
 * variable GDN_PREFILL_PATH=split or =fused overrides the choice).  Both
 * paths compute the same values in the same precision. */
gdn_status gdn_prefill_workspace_bytes(const gdn_config* cfg, int64_t seq_len, uint64_t* bytes);

/* Chunked prefill of seq_len tokens per sequence ("Performance note":
 * chunk 64; the result is that of the per-token rule up to rounding).
 *   qkv           [B, L, conv_dim] io        pre-conv projected stream
 *   a, b          [B, L, H_v] io             gate inputs
 *   conv_w        [conv_dim, K] io           depthwise taps; tap K-1 weights
 *                                            the current token
 *   A_log, dt_bias [H_v] fp32
 *   conv_state_in [B, conv_dim, K-1] io, or NULL for a new request (zeros)
 *   conv_state_out [B, conv_dim, K-1] io     must not overlap conv_state_in
 *   rec_state_in  [B, H_v, d_k, d_v] fp32, or NULL for zeros
 *   rec_state_out [B, H_v, d_k, d_v] fp32    may equal rec_state_in exactly
 *   out           [B, L, H_v, d_v] io
 *   start_pos     absolute position of the first token; chunk boundaries
 *                 sit at absolute multiples of `chunk`, so a call resumed at
 *                 a checkpoint repeats the uninterrupted call bit for bit
 *   ckpt_buf, ckpt_buf_bytes, ckpt_interval: see gdn_state_checkpoint;
 *                 interval 0 = none (ckpt_buf may then be NULL)
 *   workspace, workspace_bytes: scratch device memory for the two-pass path
 *                 (see gdn_prefill_workspace_bytes), 256-byte aligned, not
 *                 overlapping any other buffer; its contents are clobbered.
 *                 NULL / 0 selects the fused path.
 * With seq_len == 0 only the states are copied (qkv, a, b, out may be NULL).
 * The conv+SiLU output is rounded to the io dtype before the L2 norm, as the
 * stream it comes from is stored in that dtype.
 * The diagonal 16x16 blocks of (I + A)^-1 are formed by forward substitution
 * (the "direct solve" of the Qwen3.6-27B PR, "Known limitations and
 * follow-ups").  On the two-pass path the environment variable
 * GDN_DIAG_SOLVE=neumann selects the product form of the Neumann series
 * instead (the faster-style variant the same passage names), read at each
 * call; it is less accurate where keys nearly coincide.
 * Overlapped prep: with the whole call in one segment plus the flag bytes
 * above, a state kernel of 16-column waves on at most 24 workgroups per XCD,
 * B * H_k a multiple of 8, 64 chunks or more, a GPU of 8 XCDs x 32 CUs, and
 * a created stream (not the NULL, legacy or per-thread stream, not being
 * captured), the call runs the prep of its later chunks concurrently with
 * the state kernel, on two library-owned streams of the device with disjoint
 * CU masks (24 and 8 CUs of every XCD), forked from `stream` at the call and
 * joined back into it at the end; the results are bit for bit those of the
 * serial path.  The library streams are blocking streams: work the caller
 * puts on the NULL stream meanwhile waits for them.  The state kernel waits
 * for each later chunk's records with a bound of 2 s: if the concurrent prep
 * cannot run that long (its CUs held by other work), the call fails loudly
 * rather than returning wrong values: every state workgroup that met the
 * timeout or started waiting after it writes NaN into its columns of
 * rec_state_out and of every out row of the call, so the final state of at
 * least the affected heads is NaN (the checkpoint slots the call wrote are
 * then invalid too); the caller's stream sees no error code.  GDN_PREFILL_OVERLAP=0 turns the
 * overlap off, =1 takes it from 2 chunks on. */
gdn_status gdn_prefill_chunked(const gdn_config* cfg, int64_t seq_len, int64_t start_pos,
                               const void* qkv, const void* a, const void* b, const void* conv_w,
                               const float* A_log, const float* dt_bias,
                               const void* conv_state_in, void* conv_state_out,
                               const float* rec_state_in, float* rec_state_out, void* out,
                               void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval,
                               void* workspace, uint64_t workspace_bytes, void* stream);

/* gdn_prefill_chunked without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc)
 * but want the two-pass path rather than the fused kernel.  Arguments,
 * results and errors are those of gdn_prefill_chunked; the chunk records live
 * in a static device array of GDN_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library's code object holds on every device it is loaded on, until the
 * process ends.  A call whose records exceed it runs in segments, as with a
 * small workspace.
 *   - GDN_ESPACE if one chunk's records do not fit the array: B * (H_k *
 *     32768 + H_v * 13568) bytes (26624 per value head in the precise mode)
 *     above 64 MiB, e.g. B above 57 with 16 key and 48 value heads.
 *   - The array's address is looked up (hipGetSymbolAddress) on the first
 *     call on a device, with that device current; GDN_EHIP if that fails.
 *   - Every call on one device shares its array: calls that overlap in time
 *     on one device (two streams, two threads) race and give wrong results.
 *     Consecutive calls on one stream are safe.  Nothing in the array has to
 *     start at zero: each segment's first pass writes every record its
 *     second pass reads.
 *   - A head group H_v / H_k above 8 or GDN_PREFILL_PATH=fused runs the
 *     fused kernel, which needs no scratch. */
#define GDN_NOALLOC_SCRATCH_BYTES ((uint64_t)64 << 20)
gdn_status gdn_prefill_chunked_noalloc(const gdn_config* cfg, int64_t seq_len, int64_t start_pos,
                                       const void* qkv, const void* a, const void* b, const void* conv_w,
                                       const float* A_log, const float* dt_bias,
                                       const void* conv_state_in, void* conv_state_out,
                                       const float* rec_state_in, float* rec_state_out, void* out,
                                       void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval,
                                       void* stream);

/* Workspace for gdn_prefill_varlen (host only): the bytes with which every
 * group of up to 64 sequences runs each pass once,
 *   max over groups of (sequences of the group) * (chunks its longest
 *   sequence spans) * (H_k * 32768 + H_v * 13568).
 * cu_seqlens, start_pos: host arrays as for gdn_prefill_varlen. */
gdn_status gdn_prefill_varlen_workspace_bytes(const gdn_config* cfg, const int64_t* cu_seqlens,
                                              const int64_t* start_pos, uint64_t* bytes);

/* Chunked prefill of B = cfg->batch sequences of different lengths and
 * start positions in one call, packed along the token axis (continuous
 * batching; the Qwen3.6-27B PR lists batching past one sequence and prefix
 * caching under "Known limitations and follow-ups" and "Summary").  Per
 * sequence the result is bit for bit that of gdn_prefill_chunked with that
 * sequence alone (same start_pos, same checkpoints).
 *   cu_seqlens   (host) [B + 1] int64, cu_seqlens[0] = 0, non-decreasing:
 *                sequence i owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
 *                (T = cu_seqlens[B] tokens in all; empty sequences allowed,
 *                they copy their states)
 *   start_pos    (host) [B] int64 >= 0: absolute position of each
 *                sequence's first token (chunk boundaries at absolute
 *                multiples of 64, as in gdn_prefill_chunked)
 *   qkv          [T, conv_dim] io, 16-byte aligned; a, b [T, H_v] io
 *   out          [T, H_v, d_v] io, 16-byte aligned
 *   conv_state_in/out [B, conv_dim, K-1], rec_state_in/out [B, H_v, d_k, d_v]:
 *                per sequence, as in gdn_prefill_chunked (NULL inputs =
 *                new requests)
 *   ckpt_buf, ckpt_buf_bytes, ckpt_interval: slots laid out as in
 *                gdn_state_checkpoint with batch B; sequence i writes its
 *                part of slot j for every position (j+1)*interval in
 *                (start_pos[i], start_pos[i] + len_i] and leaves the others
 *                alone.  The buffer must hold the furthest slot any
 *                sequence writes.
 *   workspace    required (this path is two-pass only): at least one chunk
 *                of records for the largest group of sequences,
 *                min(B, 64) * (H_k * 32768 + H_v * 13568) bytes, else
 *                GDN_ESPACE; gdn_prefill_varlen_workspace_bytes gives the
 *                size that runs every group in one segment.
 * Supported: as gdn_prefill_chunked's two-pass path (bf16 io, d = 128,
 * H_v / H_k <= 8). */
gdn_status gdn_prefill_varlen(const gdn_config* cfg, const int64_t* cu_seqlens, const int64_t* start_pos,
                              const void* qkv, const void* a, const void* b, const void* conv_w,
                              const float* A_log, const float* dt_bias, const void* conv_state_in,
                              void* conv_state_out, const float* rec_state_in, float* rec_state_out, void* out,
                              void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval, void* workspace,
                              uint64_t workspace_bytes, void* stream);

/* Prefix-cache lookup (host only): for a request of which the first
 * cached_tokens tokens are known (a prefix hit), the checkpoint to resume
 * from -- the slot of the largest multiple of interval not above
 * cached_tokens -- and the offsets of sequence seq_index's conv tail and
 * recurrent state inside ckpt_buf (layout of gdn_state_checkpoint with
 * cfg->batch sequences).  Resume with start_pos = entry->position and the
 * tokens from there on.  entry->slot = -1 (position 0, offsets 0) when no
 * checkpoint lies in the prefix: start a new request.  Whether the slot
 * was written is the caller's bookkeeping ("Summary" of the Qwen3.6-27B
 * PR: recurrent and conv checkpoints for prefix reuse). */
gdn_status gdn_ckpt_lookup(const gdn_config* cfg, int64_t interval, int64_t cached_tokens, int32_t seq_index,
                           gdn_ckpt_entry* entry);

/* One recurrent decode step: one new token per sequence ("Delta rule").
 *   qkv [B, conv_dim], a, b [B, H_v], out [B, H_v, d_v] (io dtype); the
 *   other arguments as in gdn_prefill_chunked.  conv_state_out must not
 *   overlap conv_state_in; rec_state_out may equal rec_state_in exactly. */
gdn_status gdn_decode_step(const gdn_config* cfg, const void* qkv, const void* a, const void* b,
                           const void* conv_w, const float* A_log, const float* dt_bias,
                           const void* conv_state_in, void* conv_state_out,
                           const float* rec_state_in, float* rec_state_out, void* out,
                           void* stream);

/* T = num_tokens consecutive decode tokens per sequence in one call, for
 * multi-token verification in speculative decoding: the same rule as T
 * calls of gdn_decode_step ("Delta rule", "State"), and bit for bit the same
 * results, with the state read and written once per call instead of once per
 * token.
 *   num_tokens     T, 1 .. 8
 *   qkv            [B, T, conv_dim] io; a, b [B, T, H_v] io
 *   out            [B, T, H_v, d_v] io
 *   conv_state_out, rec_state_out: the states after the last token
 *   rec_snapshots  [T, B, H_v, d_k, d_v] fp32, or NULL: the recurrent state
 *                  after each token (roll back to an accepted prefix of t + 1
 *                  tokens by resuming from snapshot t); 16-byte aligned
 *   conv_snapshots [T, B, conv_dim, K-1] io, or NULL: the conv tail after
 *                  each token
 * The other arguments are those of gdn_decode_step.  The snapshots must not
 * overlap any other buffer.  GDN_EINVAL for T outside 1 .. 8. */
gdn_status gdn_decode_multi(const gdn_config* cfg, int32_t num_tokens, const void* qkv, const void* a,
                            const void* b, const void* conv_w, const float* A_log, const float* dt_bias,
                            const void* conv_state_in, void* conv_state_out, const float* rec_state_in,
                            float* rec_state_out, void* out, float* rec_snapshots, void* conv_snapshots,
                            void* stream);

/* gdn_decode_multi with the output gate of gdn_output_gate fused in: y is
 * formed per token and value head from the fp32 core output before it is
 * rounded, by a workgroup that owns all d_v columns of its head.
 *   out        [B, T, H_v, d_v] io, or NULL to write only y
 *   z          [B, T, H_v, d_v] io, the gate input
 *   norm_w     [d_v] io
 *   gate_eps   >= 0, finite
 *   y          [B, T, H_v, d_v] io, the gated output (required); must not
 *              overlap any other buffer
 * The other arguments and the T-token semantics are those of
 * gdn_decode_multi; out, states and snapshots are bitwise those of
 * gdn_decode_multi run with all d_v columns per workgroup (the environment
 * variable GDN_DECODE_COLS = d_v), whose row sums are taken in the same
 * order.  Supported: d_v in {32, 64, 128}. */
gdn_status gdn_decode_gated(const gdn_config* cfg, int32_t num_tokens, const void* qkv, const void* a,
                            const void* b, const void* conv_w, const float* A_log, const float* dt_bias,
                            const void* conv_state_in, void* conv_state_out, const float* rec_state_in,
                            float* rec_state_out, void* out, const void* z, const void* norm_w, float gate_eps,
                            void* y, float* rec_snapshots, void* conv_snapshots, void* stream);

/* Output gate of the block ("Output": RMSNormGated of the core output with
 * the gate z, before out_proj), per token and value head over d_v:
 *   y = norm_w * o / sqrt(mean(o^2) + eps) * silu(z)
 * in fp32, rounded once to the io dtype.
 *   num_tokens  rows of the token axis (B * L for a prefill output,
 *               B * T for a decode output), >= 0
 *   o, z, y     [num_tokens, H_v, d_v] io, 16-byte aligned; y may equal o
 *               or z exactly (in place), no other overlap
 *   norm_w      [d_v] io, 16-byte aligned
 *   eps         >= 0, finite (the models use 1e-6)
 * Supported: d_v in {32, 64, 128}, io GDN_F32 or GDN_BF16, num_tokens *
 * H_v <= 2^28 (else GDN_EUNSUPPORTED).  Only
 * cfg->num_v_heads, head_v_dim and io_dtype are used (the rest of cfg must
 * still be valid). */
gdn_status gdn_output_gate(const gdn_config* cfg, int64_t num_tokens, const void* o, const void* z,
                           const void* norm_w, float eps, void* y, void* stream);

/* Static description of a status code (never NULL). */
const char* gdn_status_string(gdn_status status);

/* Library version, major*10000 + minor*100 + patch.  gdn_config is passed
 * by pointer, so a caller compiled against a header of another minor
 * version must not call the library: compare gdn_version() with
 * GDN_VERSION first.  0.2.0 added gdn_config.precision and
 * gdn_prefill_chunked_noalloc. */
#define GDN_VERSION 200
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
