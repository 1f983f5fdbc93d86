// A C-ABI caller with no Python: includes gdn.h, links libgdn.so, owns its
// device memory through the HIP runtime, and checks two bitwise identities
// the library documents:
//   * gdn_prefill_chunked gives the same bits on its fused path (no
//     workspace) and its two-pass path (with one);
//   * T calls of gdn_decode_step equal one gdn_decode_multi call of T tokens.
// Inputs are drawn by a fixed linear congruential generator.  Prints "OK" and
// exits 0 on success; any failed call or mismatch exits non-zero.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
float uniform() {   // [-1, 1)
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((g_state >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f;
}

uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        if ((x) != hipSuccess) {                                                  \
            std::fprintf(stderr, "HIP error %s at line %d\n", #x, __LINE__);      \
            return 2;                                                             \
        }                                                                         \
    } while (0)
#define CHECK_GDN(x)                                                                        \
    do {                                                                                    \
        gdn_status s_ = (x);                                                                \
        if (s_ != GDN_OK) {                                                                 \
            std::fprintf(stderr, "%s -> %s at line %d\n", #x, gdn_status_string(s_), __LINE__); \
            return 3;                                                                       \
        }                                                                                   \
    } while (0)

template <typename T>
T* upload(const std::vector<T>& h) {
    T* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T)) != hipSuccess) return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return d;
}

template <typename T>
std::vector<T> download(const T* d, size_t n) {
    std::vector<T> h(n);
    if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) h.clear();
    return h;
}

std::vector<uint16_t> bf16_vec(size_t n, float scale, float shift = 0.f) {
    std::vector<uint16_t> v(n);
    for (auto& x : v) x = to_bf16(scale * uniform() + shift);
    return v;
}

}  // namespace

int main() {
    if (gdn_version() != GDN_VERSION) {
        std::fprintf(stderr, "libgdn %d, header %d\n", gdn_version(), GDN_VERSION);
        return 2;
    }
    CHECK_HIP(hipSetDevice(0));
    gdn_config cfg{};
    cfg.batch = 2;
    cfg.num_k_heads = 2;
    cfg.num_v_heads = 4;
    cfg.head_k_dim = 128;
    cfg.head_v_dim = 128;
    cfg.conv_kernel = 4;
    cfg.chunk = 64;
    cfg.io_dtype = GDN_BF16;
    cfg.q_scale = 1.0f;
    cfg.l2_eps = 1e-6f;
    const int64_t B = cfg.batch, Hv = cfg.num_v_heads, L = 200, T = 3;
    const int64_t cd = 2 * cfg.num_k_heads * 128 + Hv * 128;

    // prefill inputs and two sets of outputs
    uint16_t* qkv = upload(bf16_vec(B * L * cd, 1.0f));
    uint16_t* a = upload(bf16_vec(B * L * Hv, 1.0f));
    uint16_t* b = upload(bf16_vec(B * L * Hv, 1.0f));
    uint16_t* conv_w = upload(bf16_vec(cd * 4, 0.5f));
    std::vector<float> alog(Hv), dtb(Hv);
    for (int64_t h = 0; h < Hv; ++h) {
        alog[h] = std::log(1.0f + 7.5f * (uniform() + 1.0f));
        dtb[h] = 0.1f * uniform();
    }
    float* A_log = upload(alog);
    float* dt_bias = upload(dtb);
    if (!qkv || !a || !b || !conv_w || !A_log || !dt_bias) return 2;
    const size_t out_n = B * L * Hv * 128, conv_n = B * cd * 3, rec_n = B * Hv * 128 * 128;
    uint16_t *out1, *out2, *conv1, *conv2;
    float *rec1, *rec2;
    CHECK_HIP(hipMalloc(&out1, out_n * 2));
    CHECK_HIP(hipMalloc(&out2, out_n * 2));
    CHECK_HIP(hipMalloc(&conv1, conv_n * 2));
    CHECK_HIP(hipMalloc(&conv2, conv_n * 2));
    CHECK_HIP(hipMalloc(&rec1, rec_n * 4));
    CHECK_HIP(hipMalloc(&rec2, rec_n * 4));
    uint64_t ws_bytes = 0;
    CHECK_GDN(gdn_prefill_workspace_bytes(&cfg, L, &ws_bytes));
    void* ws = nullptr;
    CHECK_HIP(hipMalloc(&ws, ws_bytes));

    // fused path (no workspace), then the two-pass path
    CHECK_GDN(gdn_prefill_chunked(&cfg, L, 0, qkv, a, b, conv_w, A_log, dt_bias, nullptr, conv1, nullptr, rec1,
                                  out1, nullptr, 0, 0, nullptr, 0, nullptr));
    CHECK_GDN(gdn_prefill_chunked(&cfg, L, 0, qkv, a, b, conv_w, A_log, dt_bias, nullptr, conv2, nullptr, rec2,
                                  out2, nullptr, 0, 0, ws, ws_bytes, nullptr));
    CHECK_HIP(hipDeviceSynchronize());
    auto o1 = download(out1, out_n), o2 = download(out2, out_n);
    auto s1 = download(rec1, rec_n), s2 = download(rec2, rec_n);
    auto c1 = download(conv1, conv_n), c2 = download(conv2, conv_n);
    if (o1.empty() || o1 != o2 || s1 != s2 || c1 != c2) {
        std::fprintf(stderr, "prefill paths differ\n");
        return 4;
    }
    for (uint16_t v : o1)
        if (!std::isfinite(from_bf16(v))) return 5;
    for (float v : s1)
        if (!std::isfinite(v)) return 5;
    // the two-pass path on the library's static scratch (no workspace)
    CHECK_GDN(gdn_prefill_chunked_noalloc(&cfg, L, 0, qkv, a, b, conv_w, A_log, dt_bias, nullptr, conv1, nullptr,
                                          rec1, out1, nullptr, 0, 0, nullptr));
    CHECK_HIP(hipDeviceSynchronize());
    if (download(out1, out_n) != o2 || download(rec1, rec_n) != s2 || download(conv1, conv_n) != c2) {
        std::fprintf(stderr, "static-scratch prefill differs\n");
        return 4;
    }

    // T decode steps from the prefill's states, one call each, then one
    // T-token call; the decode inputs are [T][B][...] for the single steps
    // and [B][T][...] for the multi-token call
    std::vector<uint16_t> dq = bf16_vec(T * B * cd, 1.0f), da = bf16_vec(T * B * Hv, 1.0f), db = bf16_vec(T * B * Hv, 1.0f);
    std::vector<uint16_t> mq(B * T * cd), ma(B * T * Hv), mb(B * T * Hv);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t s = 0; s < B; ++s) {
            std::memcpy(&mq[(s * T + t) * cd], &dq[(t * B + s) * cd], cd * 2);
            std::memcpy(&ma[(s * T + t) * Hv], &da[(t * B + s) * Hv], Hv * 2);
            std::memcpy(&mb[(s * T + t) * Hv], &db[(t * B + s) * Hv], Hv * 2);
        }
    uint16_t *dqd = upload(dq), *dad = upload(da), *dbd = upload(db), *mqd = upload(mq), *mad = upload(ma), *mbd = upload(mb);
    if (!dqd || !dad || !dbd || !mqd || !mad || !mbd) return 2;
    uint16_t *dout, *mout, *convA, *convB, *convM;
    CHECK_HIP(hipMalloc(&dout, T * B * Hv * 128 * 2));
    CHECK_HIP(hipMalloc(&mout, B * T * Hv * 128 * 2));
    CHECK_HIP(hipMalloc(&convA, conv_n * 2));
    CHECK_HIP(hipMalloc(&convB, conv_n * 2));
    CHECK_HIP(hipMalloc(&convM, conv_n * 2));
    CHECK_HIP(hipMemcpy(convA, conv1, conv_n * 2, hipMemcpyDeviceToDevice));
    // single steps: recurrent state in place in rec1, conv ping-pong
    for (int64_t t = 0; t < T; ++t) {
        uint16_t* cin = (t % 2 == 0) ? convA : convB;
        uint16_t* cout = (t % 2 == 0) ? convB : convA;
        CHECK_GDN(gdn_decode_step(&cfg, dqd + t * B * cd, dad + t * B * Hv, dbd + t * B * Hv, conv_w, A_log, dt_bias,
                                  cin, cout, rec1, rec1, dout + t * B * Hv * 128, nullptr));
    }
    // one T-token call from the same starting states (prefill's, kept in rec2 / conv2)
    CHECK_GDN(gdn_decode_multi(&cfg, (int32_t)T, mqd, mad, mbd, conv_w, A_log, dt_bias, conv2, convM, rec2, rec2, mout,
                               nullptr, nullptr, nullptr));
    CHECK_HIP(hipDeviceSynchronize());
    auto so = download(dout, T * B * Hv * 128), mo = download(mout, B * T * Hv * 128);
    auto sS = download(rec1, rec_n), mS = download(rec2, rec_n);
    auto sC = download((T % 2 == 0) ? convA : convB, conv_n), mC = download(convM, conv_n);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t s = 0; s < B; ++s)
            if (std::memcmp(&so[(t * B + s) * Hv * 128], &mo[(s * T + t) * Hv * 128], Hv * 128 * 2) != 0) {
                std::fprintf(stderr, "decode outputs differ at token %lld, sequence %lld\n", (long long)t, (long long)s);
                return 6;
            }
    if (sS != mS || sC != mC) {
        std::fprintf(stderr, "decode states differ\n");
        return 6;
    }
    // an invalid call is refused without touching anything
    if (gdn_decode_multi(&cfg, 0, mqd, mad, mbd, conv_w, A_log, dt_bias, conv2, convM, rec2, rec2, mout, nullptr,
                         nullptr, nullptr) != GDN_EINVAL)
        return 7;
    std::printf("OK (library %d)\n", gdn_version());
    return 0;
}
