// gdn_api.hip -- the C ABI of libgdn: validation, checkpoint plan, dispatch.
//
// Every entry point validates all arguments before it enqueues anything, so
// an error leaves every output untouched.  No allocation and no
// synchronisation.  The only global state is the device address of the
// static scratch array of gdn_prefill_chunked_noalloc, looked up once per
// device.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "gdn_launch.h"
#include "../../include/gdn.h"

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int io_size(int32_t io) { return io == GDN_BF16 ? 2 : 4; }

// The prefill kernels launch about 4 B H_v workgroups of 512 threads, and a
// launch's work-items along x must stay below 2^32: B H_v <= 2^20 keeps
// every prefill grid below 2^23 workgroups.
constexpr int64_t kMaxPrefillHeads = (int64_t)1 << 20;
// The output gate launches 256-thread workgroups of 4096 / d_v rows, 8 *
// rows work-items at d_v = 128: rows <= 2^28 keeps them below 2^31.
constexpr int64_t kMaxGateRows = (int64_t)1 << 28;

// Config checks shared by every entry point (shape sanity only; support for
// a particular shape is checked per path).
gdn_status check_config(const gdn_config* c) {
    if (!c) return GDN_EINVAL;
    if (c->batch < 0 || c->num_k_heads < 1 || c->num_v_heads < 1) return GDN_EINVAL;
    if (c->num_v_heads % c->num_k_heads != 0) return GDN_EINVAL;
    if (c->head_k_dim < 1 || c->head_v_dim < 1 || c->conv_kernel < 1 || c->chunk < 1)
        return GDN_EINVAL;
    if (c->io_dtype != GDN_F32 && c->io_dtype != GDN_BF16) return GDN_EINVAL;
    if (!std::isfinite(c->q_scale) || !std::isfinite(c->l2_eps) || c->l2_eps < 0.f) return GDN_EINVAL;
    if (c->precision != GDN_PRECISION_DEFAULT && c->precision != GDN_PRECISION_HILO) return GDN_EINVAL;
    return GDN_OK;
}

int64_t conv_dim_of(const gdn_config* c) {
    return 2 * (int64_t)c->num_k_heads * c->head_k_dim + (int64_t)c->num_v_heads * c->head_v_dim;
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned_to(p, 16); }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}

bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi && x.hi > x.lo && y.hi > y.lo; }

struct Plan {
    int64_t count = 0;
    int64_t first_slot = 0;
    uint64_t conv_bytes = 0;   // aligned conv part of a slot
    uint64_t slot_bytes = 0;
    uint64_t buffer_bytes = 0;
};

// The single source of checkpoint indices and offsets.
Plan checkpoint_plan(const gdn_config* c, int64_t start_pos, int64_t seq_len, int64_t interval) {
    Plan p;
    p.conv_bytes = align_up((uint64_t)c->batch * conv_dim_of(c) * (c->conv_kernel - 1) * io_size(c->io_dtype));
    const uint64_t rec_bytes = align_up((uint64_t)c->batch * c->num_v_heads * c->head_k_dim * c->head_v_dim * 4);
    p.slot_bytes = p.conv_bytes + rec_bytes;
    if (interval <= 0) return p;
    p.first_slot = start_pos / interval;
    const int64_t end_slot = (start_pos + seq_len) / interval;  // exclusive
    p.count = end_slot - p.first_slot;
    p.buffer_bytes = p.count > 0 ? (uint64_t)end_slot * p.slot_bytes : 0;
    return p;
}

}  // namespace

// Scratch of gdn_prefill_chunked_noalloc: the two-pass path's chunk records,
// in a device array that the code object brings (each device the library is
// loaded on holds its own copy until the process ends).  In host code the
// name `scratch` is only a stand-in; its device address comes from
// hipGetSymbolAddress, per device.
static constexpr uint64_t kNoAllocScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices];   // device address of `scratch`, per device

// Device address of the scratch array on the device of `stream` (the current
// device for the null stream), looked up on the first call on that device
// with the device current.
gdn_status scratch_of(void* stream, void** ptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GDN_EHIP;
    hipDevice_t dev = cur;
    if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return GDN_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GDN_EHIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return GDN_EHIP;
        if (e != hipSuccess || !p) return GDN_EHIP;
        scratch_addr[dev] = p;
    }
    *ptr = scratch_addr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_EINVAL: return "invalid argument";
        case GDN_EUNSUPPORTED: return "unsupported shape or dtype";
        case GDN_EALIAS: return "output overlaps an input";
        case GDN_ESPACE: return "buffer too small";
        case GDN_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int32_t gdn_version(void) { return GDN_VERSION; }

gdn_status gdn_state_checkpoint(const gdn_config* cfg, int64_t start_pos, int64_t seq_len,
                                int64_t interval, gdn_ckpt_entry* entries, int64_t capacity,
                                int64_t* count, uint64_t* buffer_bytes) {
    if (gdn_status s = check_config(cfg)) return s;
    if (!count || !buffer_bytes || start_pos < 0 || seq_len < 0 || interval < 0) return GDN_EINVAL;
    if (interval > 0 && interval % cfg->chunk != 0) return GDN_EINVAL;
    if (entries && capacity < 0) return GDN_EINVAL;
    const Plan p = checkpoint_plan(cfg, start_pos, seq_len, interval);
    *count = p.count;
    *buffer_bytes = p.buffer_bytes;
    if (!entries) return GDN_OK;
    const int64_t n = p.count < capacity ? p.count : capacity;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t slot = p.first_slot + i;
        entries[i].slot = slot;
        entries[i].position = (slot + 1) * interval;
        entries[i].conv_offset = (uint64_t)slot * p.slot_bytes;
        entries[i].rec_offset = entries[i].conv_offset + p.conv_bytes;
    }
    return capacity < p.count ? GDN_ESPACE : GDN_OK;
}

gdn_status gdn_prefill_workspace_bytes(const gdn_config* cfg, int64_t seq_len, uint64_t* bytes) {
    if (gdn_status s = check_config(cfg)) return s;
    if (!bytes || seq_len < 0) return GDN_EINVAL;
    // seq_len tokens starting anywhere inside a chunk span at most
    // floor((seq_len + chunk - 2) / chunk) + 1 chunks
    const int64_t chunks = seq_len == 0 ? 0 : (seq_len + cfg->chunk - 2) / cfg->chunk + 1;
    *bytes = (uint64_t)chunks * gdn::prefill_split_chunk_bytes(cfg->batch, cfg->num_k_heads, cfg->num_v_heads, cfg->precision == GDN_PRECISION_HILO);
    // and, from two chunks on, the ready flags of the overlapped prep
    if (chunks >= 2) *bytes += gdn::prefill_overlap_bytes(cfg->batch, cfg->num_k_heads, chunks);
    return GDN_OK;
}

static gdn_status prefill_chunked(const gdn_config* cfg, int64_t seq_len, int64_t start_pos,
                                  const void* qkv, const void* a, const void* b, const void* conv_w,
                                  const float* A_log, const float* dt_bias,
                                  const void* conv_state_in, void* conv_state_out,
                                  const float* rec_state_in, float* rec_state_out, void* out,
                                  void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval,
                                  void* workspace, uint64_t workspace_bytes, void* stream,
                                  bool allow_overlap) {
    if (gdn_status s = check_config(cfg)) return s;
    if (seq_len < 0 || start_pos < 0 || ckpt_interval < 0) return GDN_EINVAL;
    if (ckpt_interval > 0 && ckpt_interval % cfg->chunk != 0) return GDN_EINVAL;
    // qkv and out move in 16-byte vectors, ckpt_buf holds 256-byte aligned
    // slots; everything else needs its element alignment.  With no tokens,
    // qkv, a, b and out are never touched and may be NULL.
    const uintptr_t ea = cfg->io_dtype == GDN_BF16 ? 2 : 4;
    if (!conv_w || !aligned_to(conv_w, ea) || !conv_state_out || !aligned_to(conv_state_out, ea))
        return GDN_EINVAL;
    if (!A_log || !dt_bias || !rec_state_out || !aligned_to(A_log, 4) || !aligned_to(dt_bias, 4) ||
        !aligned_to(rec_state_out, 4))
        return GDN_EINVAL;
    if (seq_len > 0 && (!qkv || !a || !b || !out)) return GDN_EINVAL;
    if (!aligned16(qkv) || !aligned16(out) || !aligned_to(a, ea) || !aligned_to(b, ea)) return GDN_EINVAL;
    if (!aligned_to(conv_state_in, ea) || !aligned_to(rec_state_in, 4) || !aligned_to(ckpt_buf, 256) ||
        !aligned_to(workspace, 256))
        return GDN_EINVAL;
    if (!gdn::prefill_supported(cfg->head_k_dim, cfg->head_v_dim, cfg->io_dtype, cfg->conv_kernel,
                                cfg->chunk))
        return GDN_EUNSUPPORTED;
    if ((int64_t)cfg->batch * cfg->num_v_heads > kMaxPrefillHeads) return GDN_EUNSUPPORTED;

    const int64_t B = cfg->batch, L = seq_len, Hv = cfg->num_v_heads;
    const int64_t cd = conv_dim_of(cfg);
    const int ios = io_size(cfg->io_dtype);
    const uint64_t conv_state_bytes = (uint64_t)B * cd * (cfg->conv_kernel - 1) * ios;
    const uint64_t rec_bytes = (uint64_t)B * Hv * cfg->head_k_dim * cfg->head_v_dim * 4;
    const Range r_qkv = range_of(qkv, (uint64_t)B * L * cd * ios);
    const Range r_cin = range_of(conv_state_in, conv_state_in ? conv_state_bytes : 0);
    const Range r_cout = range_of(conv_state_out, conv_state_bytes);
    const Range r_rin = range_of(rec_state_in, rec_state_in ? rec_bytes : 0);
    const Range r_rout = range_of(rec_state_out, rec_bytes);
    const Range r_out = range_of(out, (uint64_t)B * L * Hv * cfg->head_v_dim * ios);
    if (overlap(r_cout, r_cin) || overlap(r_cout, r_qkv) || overlap(r_cout, r_out)) return GDN_EALIAS;
    if (rec_state_in && rec_state_in != rec_state_out && overlap(r_rin, r_rout)) return GDN_EALIAS;
    if (overlap(r_out, r_qkv) || overlap(r_out, r_rout) || overlap(r_out, r_cin) || overlap(r_out, r_rin))
        return GDN_EALIAS;
    if (overlap(r_rout, r_qkv) || overlap(r_rout, r_cout)) return GDN_EALIAS;

    const Plan plan = checkpoint_plan(cfg, start_pos, seq_len, ckpt_interval);
    if (plan.count > 0) {
        if (!ckpt_buf) return GDN_EINVAL;
        if (ckpt_buf_bytes < plan.buffer_bytes) return GDN_ESPACE;
        const Range r_ck = range_of(ckpt_buf, plan.buffer_bytes);
        if (overlap(r_ck, r_qkv) || overlap(r_ck, r_out) || overlap(r_ck, r_rout) || overlap(r_ck, r_cout) ||
            overlap(r_ck, r_cin) || overlap(r_ck, r_rin))
            return GDN_EALIAS;
    }

    // The two-pass path needs at least one chunk of records in the
    // workspace; GDN_PREFILL_PATH=split|fused overrides the choice.
    const uint64_t chunk_ws = gdn::prefill_split_chunk_bytes(cfg->batch, cfg->num_k_heads, cfg->num_v_heads, cfg->precision == GDN_PRECISION_HILO);
    const bool ws_ok = workspace && chunk_ws > 0 && workspace_bytes >= chunk_ws &&
                       cfg->num_v_heads / cfg->num_k_heads <= 8;
    const char* path_env = getenv("GDN_PREFILL_PATH");
    const bool force_fused = path_env && path_env[0] == 'f';
    const bool two_pass = ws_ok && !force_fused;
    if (two_pass) {
        // only the part a call can use is checked against the other buffers
        const int64_t k_first = start_pos / cfg->chunk;
        const int64_t chunks = L > 0 ? (start_pos + L - 1) / cfg->chunk + 1 - k_first : 0;
        const uint64_t need =
            (uint64_t)chunks * chunk_ws + (chunks >= 2 ? gdn::prefill_overlap_bytes(cfg->batch, cfg->num_k_heads, chunks) : 0);
        const Range r_ws = range_of(workspace, need < workspace_bytes ? need : workspace_bytes);
        const Range r_ck = range_of(ckpt_buf, plan.count > 0 ? plan.buffer_bytes : 0);
        if (overlap(r_ws, r_qkv) || overlap(r_ws, r_out) || overlap(r_ws, r_rout) || overlap(r_ws, r_cout) ||
            overlap(r_ws, r_cin) || overlap(r_ws, r_rin) || overlap(r_ws, r_ck))
            return GDN_EALIAS;
    }

    gdn::PrefillParams p{};
    p.qkv = qkv;
    p.a = a;
    p.b = b;
    p.conv_w = conv_w;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.conv_in = conv_state_in;
    p.conv_out = conv_state_out;
    p.rec_in = rec_state_in;
    p.rec_out = rec_state_out;
    p.out = out;
    p.ckpt_buf = plan.count > 0 ? static_cast<char*>(ckpt_buf) : nullptr;
    p.slot_bytes = plan.slot_bytes;
    p.conv_slot_bytes = plan.conv_bytes;
    p.ckpt_interval = plan.count > 0 ? ckpt_interval : 0;
    p.seq_len = L;
    p.start_pos = start_pos;
    p.conv_dim = cd;
    p.batch = cfg->batch;
    p.num_k_heads = cfg->num_k_heads;
    p.num_v_heads = cfg->num_v_heads;
    p.q_scale = cfg->q_scale;
    p.l2_eps = cfg->l2_eps;
    // GDN_DIAG_SOLVE=neumann: two-pass path, diagonal-block inverses by the
    // Neumann product instead of substitution
    const char* solve_env = getenv("GDN_DIAG_SOLVE");
    p.diag_neumann = solve_env && solve_env[0] == 'n';
    p.precise = cfg->precision == GDN_PRECISION_HILO;
    const hipError_t e = two_pass ? gdn::launch_prefill_split(p, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                                                              allow_overlap)
                                  : gdn::launch_prefill(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_prefill_chunked(const gdn_config* cfg, int64_t seq_len, int64_t start_pos,
                               const void* qkv, const void* a, const void* b, const void* conv_w,
                               const float* A_log, const float* dt_bias,
                               const void* conv_state_in, void* conv_state_out,
                               const float* rec_state_in, float* rec_state_out, void* out,
                               void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval,
                               void* workspace, uint64_t workspace_bytes, void* stream)  {
    return prefill_chunked(cfg, seq_len, start_pos, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, conv_state_out,
                           rec_state_in, rec_state_out, out, ckpt_buf, ckpt_buf_bytes, ckpt_interval, workspace,
                           workspace_bytes, stream, true);
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_config* cfg, int64_t seq_len, int64_t start_pos,
                                       const void* qkv, const void* a, const void* b, const void* conv_w,
                                       const float* A_log, const float* dt_bias, const void* conv_state_in,
                                       void* conv_state_out, const float* rec_state_in, float* rec_state_out,
                                       void* out, void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval,
                                       void* stream) {
    if (gdn_status s = check_config(cfg)) return s;
    // one chunk's records must fit the array; longer calls run in segments
    if (gdn::prefill_split_chunk_bytes(cfg->batch, cfg->num_k_heads, cfg->num_v_heads,
                                       cfg->precision == GDN_PRECISION_HILO) > kNoAllocScratchBytes)
        return GDN_ESPACE;
    void* ws = nullptr;
    if (gdn_status s = scratch_of(stream, &ws)) return s;
    // no overlapped prep: its streams would be created on first use
    return prefill_chunked(cfg, seq_len, start_pos, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, conv_state_out,
                           rec_state_in, rec_state_out, out, ckpt_buf, ckpt_buf_bytes, ckpt_interval, ws,
                           kNoAllocScratchBytes, stream, false);
}

// Output gate arguments of a decode call (y == NULL: no gate).
struct DecodeGate {
    const void* z = nullptr;
    const void* norm_w = nullptr;
    float eps = 0.f;
    void* y = nullptr;
};

// One or several tokens per sequence through the decode kernel (T = 1 is
// gdn_decode_step); snapshots and the output gate are optional.  With the
// gate, out may be NULL.
static gdn_status decode_tokens(const gdn_config* cfg, int32_t num_tokens, const void* qkv, const void* a,
                                const void* b, const void* conv_w, const float* A_log, const float* dt_bias,
                                const void* conv_state_in, void* conv_state_out, const float* rec_state_in,
                                float* rec_state_out, void* out, float* rec_snapshots, void* conv_snapshots,
                                const DecodeGate& gate, void* stream) {
    if (gdn_status s = check_config(cfg)) return s;
    if (num_tokens < 1 || num_tokens > gdn::kMaxDecodeTokens) return GDN_EINVAL;
    // the recurrent states move in 16-byte vectors; everything else needs its
    // element alignment
    const uintptr_t ea = cfg->io_dtype == GDN_BF16 ? 2 : 4;
    const bool gated = gate.y != nullptr;
    for (const void* p : {qkv, a, b, conv_w, (const void*)conv_state_out})
        if (!p || !aligned_to(p, ea)) return GDN_EINVAL;
    if ((!out && !gated) || !aligned_to(out, ea)) return GDN_EINVAL;
    if (gated) {
        for (const void* p : {gate.z, gate.norm_w, (const void*)gate.y})
            if (!p || !aligned_to(p, ea)) return GDN_EINVAL;
        if (!std::isfinite(gate.eps) || gate.eps < 0.f) return GDN_EINVAL;
    }
    if (!A_log || !dt_bias || !aligned_to(A_log, 4) || !aligned_to(dt_bias, 4)) return GDN_EINVAL;
    if (!rec_state_out || !aligned16(rec_state_out) || !aligned16(rec_state_in) ||
        !aligned_to(conv_state_in, ea) || !aligned16(rec_snapshots) || !aligned_to(conv_snapshots, ea))
        return GDN_EINVAL;
    if (cfg->conv_kernel != 4 || !gdn::decode_supported(cfg->head_k_dim, cfg->head_v_dim, cfg->io_dtype))
        return GDN_EUNSUPPORTED;
    // grid (d_v / columns, H_v, B): the y and z dimensions stay within 65535
    if (cfg->batch > 65535 || cfg->num_v_heads > 65535) return GDN_EUNSUPPORTED;

    const int64_t B = cfg->batch, Hv = cfg->num_v_heads, T = num_tokens;
    const int64_t cd = conv_dim_of(cfg);
    const int ios = io_size(cfg->io_dtype);
    const uint64_t conv_state_bytes = (uint64_t)B * cd * 3 * ios;
    const uint64_t rec_bytes = (uint64_t)B * Hv * cfg->head_k_dim * cfg->head_v_dim * 4;
    const Range r_qkv = range_of(qkv, (uint64_t)B * T * cd * ios);
    const Range r_a = range_of(a, (uint64_t)B * T * Hv * ios);
    const Range r_b = range_of(b, (uint64_t)B * T * Hv * ios);
    const Range r_cin = range_of(conv_state_in, conv_state_in ? conv_state_bytes : 0);
    const Range r_cout = range_of(conv_state_out, conv_state_bytes);
    const Range r_rin = range_of(rec_state_in, rec_state_in ? rec_bytes : 0);
    const Range r_rout = range_of(rec_state_out, rec_bytes);
    const uint64_t out_bytes = (uint64_t)B * T * Hv * cfg->head_v_dim * ios;
    const Range r_out = range_of(out, out ? out_bytes : 0);
    const Range r_y = range_of(gate.y, gated ? out_bytes : 0);
    const Range r_rs = range_of(rec_snapshots, rec_snapshots ? T * rec_bytes : 0);
    const Range r_cs = range_of(conv_snapshots, conv_snapshots ? T * conv_state_bytes : 0);
    if (overlap(r_cout, r_cin) || overlap(r_cout, r_qkv) || overlap(r_cout, r_out)) return GDN_EALIAS;
    if (rec_state_in && rec_state_in != rec_state_out && overlap(r_rin, r_rout)) return GDN_EALIAS;
    if (overlap(r_out, r_qkv) || overlap(r_out, r_rout) || overlap(r_out, r_cin) || overlap(r_out, r_rin))
        return GDN_EALIAS;
    if (overlap(r_rout, r_qkv) || overlap(r_rout, r_cout)) return GDN_EALIAS;
    // the snapshots are outputs of their own
    for (const Range& w : {r_rs, r_cs})
        for (const Range& o : {r_qkv, r_a, r_b, r_cin, r_cout, r_rin, r_rout, r_out})
            if (overlap(w, o)) return GDN_EALIAS;
    if (overlap(r_rs, r_cs)) return GDN_EALIAS;
    if (gated) {
        const Range r_z = range_of(gate.z, out_bytes);
        const Range r_w = range_of(gate.norm_w, (uint64_t)cfg->head_v_dim * ios);
        for (const Range& o : {r_qkv, r_a, r_b, r_cin, r_cout, r_rin, r_rout, r_out, r_rs, r_cs, r_z, r_w})
            if (overlap(r_y, o)) return GDN_EALIAS;
        for (const Range& w : {r_out, r_cout, r_rout, r_rs, r_cs})
            if (overlap(w, r_z) || overlap(w, r_w)) return GDN_EALIAS;
    }

    gdn::DecodeParams p{};
    p.qkv = qkv;
    p.a = a;
    p.b = b;
    p.conv_w = conv_w;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.conv_in = conv_state_in;
    p.conv_out = conv_state_out;
    p.rec_in = rec_state_in;
    p.rec_out = rec_state_out;
    p.out = out;
    p.rec_snap = rec_snapshots;
    p.conv_snap = conv_snapshots;
    p.gate_z = gate.z;
    p.gate_w = gate.norm_w;
    p.gate_y = gate.y;
    p.gate_eps = gate.eps;
    p.conv_dim = cd;
    p.batch = cfg->batch;
    p.num_k_heads = cfg->num_k_heads;
    p.num_v_heads = cfg->num_v_heads;
    p.head_k_dim = cfg->head_k_dim;
    p.head_v_dim = cfg->head_v_dim;
    p.io_dtype = cfg->io_dtype;
    p.num_tokens = num_tokens;
    p.q_scale = cfg->q_scale;
    p.l2_eps = cfg->l2_eps;
    const hipError_t e = gdn::launch_decode_step(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_decode_step(const gdn_config* cfg, const void* qkv, const void* a, const void* b,
                           const void* conv_w, const float* A_log, const float* dt_bias,
                           const void* conv_state_in, void* conv_state_out,
                           const float* rec_state_in, float* rec_state_out, void* out,
                           void* stream) {
    return decode_tokens(cfg, 1, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, conv_state_out, rec_state_in,
                         rec_state_out, out, nullptr, nullptr, DecodeGate{}, stream);
}

gdn_status gdn_decode_multi(const gdn_config* cfg, int32_t num_tokens, const void* qkv, const void* a,
                            const void* b, const void* conv_w, const float* A_log, const float* dt_bias,
                            const void* conv_state_in, void* conv_state_out, const float* rec_state_in,
                            float* rec_state_out, void* out, float* rec_snapshots, void* conv_snapshots,
                            void* stream) {
    return decode_tokens(cfg, num_tokens, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, conv_state_out,
                         rec_state_in, rec_state_out, out, rec_snapshots, conv_snapshots, DecodeGate{}, stream);
}

gdn_status gdn_decode_gated(const gdn_config* cfg, int32_t num_tokens, const void* qkv, const void* a,
                            const void* b, const void* conv_w, const float* A_log, const float* dt_bias,
                            const void* conv_state_in, void* conv_state_out, const float* rec_state_in,
                            float* rec_state_out, void* out, const void* z, const void* norm_w, float gate_eps,
                            void* y, float* rec_snapshots, void* conv_snapshots, void* stream) {
    if (!y) return GDN_EINVAL;
    if (gdn_status s = check_config(cfg)) return s;
    if (!gdn::gate_supported(cfg->head_v_dim, cfg->io_dtype)) return GDN_EUNSUPPORTED;
    DecodeGate gate;
    gate.z = z;
    gate.norm_w = norm_w;
    gate.eps = gate_eps;
    gate.y = y;
    return decode_tokens(cfg, num_tokens, qkv, a, b, conv_w, A_log, dt_bias, conv_state_in, conv_state_out,
                         rec_state_in, rec_state_out, out, rec_snapshots, conv_snapshots, gate, stream);
}

// Checks cu_seqlens / start_pos of a varlen call (host arrays) and returns
// the number of chunks the largest group of sequences spans per sequence
// and the workspace bytes with which every group runs in one segment.
static gdn_status varlen_shape(const gdn_config* cfg, const int64_t* cu_seqlens, const int64_t* start_pos,
                               uint64_t* ws_all) {
    if (!cu_seqlens || !start_pos || cu_seqlens[0] != 0) return GDN_EINVAL;
    const int G = gdn::prefill_varlen_group();
    uint64_t need = 0;
    for (int g0 = 0; g0 < cfg->batch; g0 += G) {
        const int n = cfg->batch - g0 < G ? cfg->batch - g0 : G;
        int64_t max_n = 0;
        for (int i = g0; i < g0 + n; ++i) {
            const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i], st = start_pos[i];
            if (len < 0 || st < 0 || st > ((int64_t)1 << 50) || len > ((int64_t)1 << 40)) return GDN_EINVAL;
            const int64_t chunks = len > 0 ? (st + len - 1) / cfg->chunk + 1 - st / cfg->chunk : 0;
            if (chunks > max_n) max_n = chunks;
        }
        const uint64_t g = (uint64_t)max_n * gdn::prefill_split_chunk_bytes(n, cfg->num_k_heads, cfg->num_v_heads, cfg->precision == GDN_PRECISION_HILO);
        if (g > need) need = g;
    }
    *ws_all = need;
    return GDN_OK;
}

gdn_status gdn_prefill_varlen_workspace_bytes(const gdn_config* cfg, const int64_t* cu_seqlens,
                                              const int64_t* start_pos, uint64_t* bytes) {
    if (gdn_status s = check_config(cfg)) return s;
    if (!bytes) return GDN_EINVAL;
    uint64_t all = 0;
    if (gdn_status s = varlen_shape(cfg, cu_seqlens, start_pos, &all)) return s;
    *bytes = all;
    return GDN_OK;
}

gdn_status gdn_prefill_varlen(const gdn_config* cfg, const int64_t* cu_seqlens, const int64_t* start_pos,
                              const void* qkv, const void* a, const void* b, const void* conv_w,
                              const float* A_log, const float* dt_bias, const void* conv_state_in,
                              void* conv_state_out, const float* rec_state_in, float* rec_state_out, void* out,
                              void* ckpt_buf, uint64_t ckpt_buf_bytes, int64_t ckpt_interval, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
    if (gdn_status s = check_config(cfg)) return s;
    if (ckpt_interval < 0 || (ckpt_interval > 0 && ckpt_interval % cfg->chunk != 0)) return GDN_EINVAL;
    uint64_t ws_all = 0;
    if (gdn_status s = varlen_shape(cfg, cu_seqlens, start_pos, &ws_all)) return s;
    const int64_t B = cfg->batch, T = cu_seqlens[B], Hv = cfg->num_v_heads;
    const uintptr_t ea = cfg->io_dtype == GDN_BF16 ? 2 : 4;
    if (!conv_w || !aligned_to(conv_w, ea) || !conv_state_out || !aligned_to(conv_state_out, ea))
        return GDN_EINVAL;
    if (!A_log || !dt_bias || !rec_state_out || !aligned_to(A_log, 4) || !aligned_to(dt_bias, 4) ||
        !aligned_to(rec_state_out, 4))
        return GDN_EINVAL;
    if (T > 0 && (!qkv || !a || !b || !out)) return GDN_EINVAL;
    if (!aligned16(qkv) || !aligned16(out) || !aligned_to(a, ea) || !aligned_to(b, ea)) return GDN_EINVAL;
    if (!aligned_to(conv_state_in, ea) || !aligned_to(rec_state_in, 4) || !aligned_to(ckpt_buf, 256) ||
        !workspace || !aligned_to(workspace, 256))
        return GDN_EINVAL;
    if (!gdn::prefill_supported(cfg->head_k_dim, cfg->head_v_dim, cfg->io_dtype, cfg->conv_kernel,
                                cfg->chunk))
        return GDN_EUNSUPPORTED;
    if (cfg->num_v_heads / cfg->num_k_heads > 8) return GDN_EUNSUPPORTED;
    if (B * Hv > kMaxPrefillHeads) return GDN_EUNSUPPORTED;
    if (B > 0 && workspace_bytes < gdn::prefill_varlen_group_bytes((int)B, cfg->num_k_heads, cfg->num_v_heads, cfg->precision == GDN_PRECISION_HILO))
        return GDN_ESPACE;

    const int64_t cd = conv_dim_of(cfg);
    const int ios = io_size(cfg->io_dtype);
    const uint64_t conv_state_bytes = (uint64_t)B * cd * (cfg->conv_kernel - 1) * ios;
    const uint64_t rec_bytes = (uint64_t)B * Hv * cfg->head_k_dim * cfg->head_v_dim * 4;
    const Range r_qkv = range_of(qkv, (uint64_t)T * cd * ios);
    const Range r_a = range_of(a, (uint64_t)T * Hv * ios), r_b = range_of(b, (uint64_t)T * Hv * ios);
    const Range r_cin = range_of(conv_state_in, conv_state_in ? conv_state_bytes : 0);
    const Range r_cout = range_of(conv_state_out, conv_state_bytes);
    const Range r_rin = range_of(rec_state_in, rec_state_in ? rec_bytes : 0);
    const Range r_rout = range_of(rec_state_out, rec_bytes);
    const Range r_out = range_of(out, (uint64_t)T * Hv * cfg->head_v_dim * ios);
    if (rec_state_in && rec_state_in != rec_state_out && overlap(r_rin, r_rout)) return GDN_EALIAS;
    for (const Range& w : {r_cout, r_out, r_rout})
        for (const Range& o : {r_qkv, r_a, r_b, r_cin})
            if (overlap(w, o)) return GDN_EALIAS;
    if (overlap(r_cout, r_out) || overlap(r_cout, r_rout) || overlap(r_out, r_rout) || overlap(r_out, r_rin) ||
        overlap(r_cout, r_rin))
        return GDN_EALIAS;

    // checkpoints: each sequence emits its own slots; the buffer spans the
    // furthest one
    uint64_t ck_need = 0;
    int64_t ck_count = 0;
    for (int64_t i = 0; i < B; ++i) {
        const Plan pl = checkpoint_plan(cfg, start_pos[i], cu_seqlens[i + 1] - cu_seqlens[i], ckpt_interval);
        ck_count += pl.count;
        if (pl.buffer_bytes > ck_need) ck_need = pl.buffer_bytes;
    }
    const Plan plan0 = checkpoint_plan(cfg, 0, 0, ckpt_interval);
    const Range r_ck = range_of(ckpt_buf, ck_count > 0 ? ck_need : 0);
    if (ck_count > 0) {
        if (!ckpt_buf) return GDN_EINVAL;
        if (ckpt_buf_bytes < ck_need) return GDN_ESPACE;
        for (const Range& o : {r_qkv, r_a, r_b, r_cin, r_cout, r_rin, r_rout, r_out})
            if (overlap(r_ck, o)) return GDN_EALIAS;
    }
    const Range r_ws = range_of(workspace, ws_all < workspace_bytes ? ws_all : workspace_bytes);
    for (const Range& o : {r_qkv, r_a, r_b, r_cin, r_cout, r_rin, r_rout, r_out, r_ck})
        if (overlap(r_ws, o)) return GDN_EALIAS;

    gdn::PrefillParams p{};
    p.qkv = qkv;
    p.a = a;
    p.b = b;
    p.conv_w = conv_w;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.conv_in = conv_state_in;
    p.conv_out = conv_state_out;
    p.rec_in = rec_state_in;
    p.rec_out = rec_state_out;
    p.out = out;
    p.ckpt_buf = ck_count > 0 ? static_cast<char*>(ckpt_buf) : nullptr;
    p.slot_bytes = plan0.slot_bytes;
    p.conv_slot_bytes = plan0.conv_bytes;
    p.ckpt_interval = ck_count > 0 ? ckpt_interval : 0;
    p.seq_len = 0;
    p.start_pos = 0;
    p.conv_dim = cd;
    p.batch = cfg->batch;
    p.num_k_heads = cfg->num_k_heads;
    p.num_v_heads = cfg->num_v_heads;
    p.q_scale = cfg->q_scale;
    p.l2_eps = cfg->l2_eps;
    const char* solve_env = getenv("GDN_DIAG_SOLVE");
    p.diag_neumann = solve_env && solve_env[0] == 'n';
    p.precise = cfg->precision == GDN_PRECISION_HILO;
    if (B == 0) return GDN_OK;
    const hipError_t e = gdn::launch_prefill_varlen(p, cu_seqlens, start_pos, workspace, workspace_bytes,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_ckpt_lookup(const gdn_config* cfg, int64_t interval, int64_t cached_tokens, int32_t seq_index,
                           gdn_ckpt_entry* entry) {
    if (gdn_status s = check_config(cfg)) return s;
    if (!entry || interval <= 0 || interval % cfg->chunk != 0 || cached_tokens < 0 || seq_index < 0 ||
        seq_index >= cfg->batch)
        return GDN_EINVAL;
    const Plan pl = checkpoint_plan(cfg, 0, 0, interval);
    const int64_t position = cached_tokens / interval * interval;
    entry->position = position;
    if (position == 0) {
        entry->slot = -1;
        entry->conv_offset = entry->rec_offset = 0;
        return GDN_OK;
    }
    entry->slot = position / interval - 1;
    const uint64_t base = (uint64_t)entry->slot * pl.slot_bytes;
    entry->conv_offset = base + (uint64_t)seq_index * conv_dim_of(cfg) * (cfg->conv_kernel - 1) * io_size(cfg->io_dtype);
    entry->rec_offset = base + pl.conv_bytes +
                        (uint64_t)seq_index * cfg->num_v_heads * cfg->head_k_dim * cfg->head_v_dim * 4;
    return GDN_OK;
}

gdn_status gdn_output_gate(const gdn_config* cfg, int64_t num_tokens, const void* o, const void* z,
                           const void* norm_w, float eps, void* y, void* stream) {
    if (gdn_status s = check_config(cfg)) return s;
    if (num_tokens < 0 || !std::isfinite(eps) || eps < 0.f) return GDN_EINVAL;
    if (!gdn::gate_supported(cfg->head_v_dim, cfg->io_dtype)) return GDN_EUNSUPPORTED;
    if (num_tokens > kMaxGateRows / cfg->num_v_heads) return GDN_EUNSUPPORTED;
    const int64_t rows = num_tokens * cfg->num_v_heads;
    if (!norm_w || !aligned16(norm_w)) return GDN_EINVAL;
    if (rows > 0 && (!o || !z || !y)) return GDN_EINVAL;
    if (!aligned16(o) || !aligned16(z) || !aligned16(y)) return GDN_EINVAL;
    const int ios = io_size(cfg->io_dtype);
    const uint64_t bytes = (uint64_t)rows * cfg->head_v_dim * ios;
    const Range r_o = range_of(o, bytes), r_z = range_of(z, bytes), r_y = range_of(y, bytes);
    const Range r_w = range_of(norm_w, (uint64_t)cfg->head_v_dim * ios);
    // in place over o or z is allowed (each element is read before it is written)
    if ((y != o && overlap(r_y, r_o)) || (y != z && overlap(r_y, r_z)) || overlap(r_y, r_w)) return GDN_EALIAS;

    gdn::GateParams p{};
    p.o = o;
    p.z = z;
    p.norm_w = norm_w;
    p.y = y;
    p.rows = rows;
    p.head_v_dim = cfg->head_v_dim;
    p.io_dtype = cfg->io_dtype;
    p.eps = eps;
    const hipError_t e = gdn::launch_output_gate(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // extern "C"
