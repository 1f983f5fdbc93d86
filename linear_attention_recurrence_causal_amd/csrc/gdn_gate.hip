// gdn_gate.hip -- the output gate of the Gated DeltaNet block (gfx950).
//
// The cortex commit page "feat(stage-8c): linear-attention layer (Qwen3-Next
// GatedDeltaNet)" ends the block ("Output") with RMSNormGated(core output,
// z) before out_proj.  Per token t and value head h, over the d_v channels:
//   y = w * o / sqrt(mean(o^2) + eps) * silu(z)
// computed in fp32 (SiLU with the hardware exp2 and reciprocal) and rounded
// once to the io dtype.
//
// HBM-bound: per element one read of o and z and one write of y (6 bytes in
// bf16), the d_v weights come from cache.  One row of d_v elements is spread
// over d_v / 8 lanes of 8 consecutive elements each (16-byte loads in bf16),
// so a wave covers 64 * 8 / d_v rows per pass and a 256-thread workgroup
// 2048 / d_v; the row's sum of squares is a fixed butterfly over its lanes.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kGateThreads = 256;
constexpr int kGateElems = 8;   // elements per lane

template <typename IO> struct vec8;

template <> struct vec8<bf16_t> {
    __device__ static __forceinline__ void load(const void* p, int64_t i, float x[8]) {
        const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
            x[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
        }
    }
    // round to nearest even with the packed hardware conversion
    __device__ static __forceinline__ void store(void* p, int64_t i, const float x[8]) {
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(p) + i) = __builtin_convertvector(v, bf16x8);
    }
};

template <> struct vec8<float> {
    __device__ static __forceinline__ void load(const void* p, int64_t i, float x[8]) {
        const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
        const float4 a = s[0], b = s[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    __device__ static __forceinline__ void store(void* p, int64_t i, const float x[8]) {
        float4* d = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
        d[0] = make_float4(x[0], x[1], x[2], x[3]);
        d[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
};

// GATE_ROWS rows per lane: every load of the workgroup is issued before the
// first row is finished, and the grid is GATE_ROWS times smaller.
template <typename IO, int DV, int GATE_ROWS>
__global__ __launch_bounds__(kGateThreads) void output_gate_kernel(GateParams p) {
    constexpr int LPR = DV / kGateElems;          // lanes per row
    constexpr int RPP = kGateThreads / LPR;       // rows per pass of the workgroup
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row lanes within one wave");
    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * RPP * GATE_ROWS + tid / LPR;
    const int j0 = (tid % LPR) * kGateElems;
    float w[8];
    vec8<IO>::load(p.norm_w, j0, w);
    float o[GATE_ROWS][8], z[GATE_ROWS][8];
#pragma unroll
    for (int r = 0; r < GATE_ROWS; ++r) {
        const int64_t row = row0 + (int64_t)r * RPP;
        if (row < p.rows) {
            vec8<IO>::load(p.o, row * DV + j0, o[r]);
            vec8<IO>::load(p.z, row * DV + j0, z[r]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) o[r][k] = z[r][k] = 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < GATE_ROWS; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fmaf(o[r][k], o[r][k], ss);
        // the row's lanes are LPR consecutive lanes of one wave
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + p.eps);
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = w[k] * (o[r][k] * inv) * silu_fast(z[r][k]);
        const int64_t row = row0 + (int64_t)r * RPP;
        if (row < p.rows) vec8<IO>::store(p.y, row * DV + j0, y);
    }
}

template <typename IO, int DV>
hipError_t launch_dv(const GateParams& p, hipStream_t stream) {
    constexpr int kRows = 2;
    const int64_t per_wg = (int64_t)(kGateThreads / (DV / kGateElems)) * kRows;
    const dim3 grid((unsigned)((p.rows + per_wg - 1) / per_wg));
    hipLaunchKernelGGL((output_gate_kernel<IO, DV, kRows>), grid, dim3(kGateThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const GateParams& p, hipStream_t stream) {
    switch (p.head_v_dim) {
        case 32: return launch_dv<IO, 32>(p, stream);
        case 64: return launch_dv<IO, 64>(p, stream);
        case 128: return launch_dv<IO, 128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool gate_supported(int head_v_dim, int io_dtype) {
    return (head_v_dim == 32 || head_v_dim == 64 || head_v_dim == 128) &&
           (io_dtype == GDN_F32 || io_dtype == GDN_BF16);
}

hipError_t launch_output_gate(const GateParams& p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    return p.io_dtype == GDN_BF16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace gdn
