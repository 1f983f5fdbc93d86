// gdn_launch.h -- kernel parameter blocks and launchers (host side of libgdn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kMaxDecodeTokens = 8;   // tokens per multi-token decode call

struct DecodeParams {
    const void* qkv;        // [B, T, conv_dim] io
    const void* a;          // [B, T, H_v] io
    const void* b;          // [B, T, H_v] io
    const void* conv_w;     // [conv_dim, 4] io
    const float* A_log;     // [H_v]
    const float* dt_bias;   // [H_v]
    const void* conv_in;    // [B, conv_dim, 3] io or null (zeros)
    void* conv_out;         // [B, conv_dim, 3] io
    const float* rec_in;    // [B, H_v, d_k, d_v] or null (zeros)
    float* rec_out;         // [B, H_v, d_k, d_v]
    void* out;              // [B, T, H_v, d_v] io
    float* rec_snap;        // [T, B, H_v, d_k, d_v] state after each token, or null
    void* conv_snap;        // [T, B, conv_dim, 3] io conv tail after each token, or null
    const void* gate_z;     // [B, T, H_v, d_v] io gate input, with gate_y
    const void* gate_w;     // [d_v] io norm weight, with gate_y
    void* gate_y;           // [B, T, H_v, d_v] io gated output, or null (no gate)
    int64_t conv_dim;
    int32_t batch, num_k_heads, num_v_heads, head_k_dim, head_v_dim, io_dtype;
    int32_t num_tokens;     // T, 1 .. kMaxDecodeTokens
    float q_scale, l2_eps;
    float gate_eps;
};

struct PrefillParams {
    const void* qkv;        // [B, L, conv_dim] bf16
    const void* a;          // [B, L, H_v] bf16
    const void* b;          // [B, L, H_v] bf16
    const void* conv_w;     // [conv_dim, 4] bf16
    const float* A_log;     // [H_v]
    const float* dt_bias;   // [H_v]
    const void* conv_in;    // [B, conv_dim, 3] bf16 or null
    void* conv_out;         // [B, conv_dim, 3] bf16
    const float* rec_in;    // [B, H_v, 128, 128] or null
    float* rec_out;         // [B, H_v, 128, 128]
    void* out;              // [B, L, H_v, 128] bf16
    char* ckpt_buf;         // checkpoint slots or null
    uint64_t slot_bytes;    // bytes per slot
    uint64_t conv_slot_bytes;  // aligned bytes of the conv part of a slot
    int64_t ckpt_interval;  // 0 = none
    int64_t seq_len, start_pos, conv_dim;
    int32_t batch, num_k_heads, num_v_heads;
    float q_scale, l2_eps;
    int32_t diag_neumann;   // two-pass path: diagonal-block inverses by the Neumann product
    int32_t precise;        // bf16 hi + lo operands on the solve's and P Delta's products (GDN_PRECISION_HILO)
};

// Output gate: rows = tokens x H_v rows of d_v elements.
struct GateParams {
    const void* o;          // [rows, d_v] io
    const void* z;          // [rows, d_v] io
    const void* norm_w;     // [d_v] io
    void* y;                // [rows, d_v] io (may equal o or z exactly)
    int64_t rows;
    int32_t head_v_dim, io_dtype;
    float eps;
};

bool gate_supported(int head_v_dim, int io_dtype);
hipError_t launch_output_gate(const GateParams& p, hipStream_t stream);

bool decode_supported(int head_k_dim, int head_v_dim, int io_dtype);
hipError_t launch_decode_step(const DecodeParams& p, hipStream_t stream);

bool prefill_supported(int head_k_dim, int head_v_dim, int io_dtype, int conv_kernel, int chunk);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Two-pass path: workspace bytes per chunk of every sequence, whether the
// head grouping is supported, and the launcher (segments of
// ws_bytes / prefill_split_chunk_bytes chunks; at least one must fit).  A
// call in one segment with prefill_overlap_bytes more (ready flags and
// counters after the records) runs the tail of its prep concurrently with
// the state kernel on library-owned streams where allow_overlap is set and
// the shape, the chip and the stream (not capturing) qualify.
uint64_t prefill_split_chunk_bytes(int batch, int num_k_heads, int num_v_heads, bool precise);
uint64_t prefill_overlap_bytes(int batch, int num_k_heads, int64_t chunks);
bool prefill_split_supported(const PrefillParams& p);
hipError_t launch_prefill_split(const PrefillParams& p, void* ws, uint64_t ws_bytes, hipStream_t stream,
                                bool allow_overlap);

// Varlen two-pass path: p.batch sequences packed along the token axis
// (cu_seqlens[p.batch + 1], start_pos[p.batch], host arrays; p.seq_len and
// p.start_pos unused).  Sequences run in groups of prefill_varlen_group();
// the workspace must hold one chunk of records for a group
// (prefill_varlen_group_bytes) and is used in segments beyond that.
int prefill_varlen_group();
uint64_t prefill_varlen_group_bytes(int num_seqs, int num_k_heads, int num_v_heads, bool precise);
hipError_t launch_prefill_varlen(const PrefillParams& p, const int64_t* cu_seqlens, const int64_t* start_pos,
                                 void* ws, uint64_t ws_bytes, hipStream_t stream);

}  // namespace gdn
