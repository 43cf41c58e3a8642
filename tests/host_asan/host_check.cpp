// Host-side checks of libekv's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; the device code is not built,
// and nothing here launches a kernel or touches a GPU).  It drives every
// entry point through its argument validation and the workspace planner
// (decode: fused, streamed and softmax plans; selection: every selector)
// over a grid of shapes, including the limits, and checks the statuses.
// Device pointers are dummy addresses: the host code must never dereference
// them.  Exit status 0 and "host checks passed" when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ekv.h"

static int g_fail = 0, g_pass = 0;

#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (cond) {                                              \
            ++g_pass;                                            \
        } else {                                                 \
            ++g_fail;                                            \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                   \
            std::fprintf(stderr, " [%s]\n", ekv_last_error());   \
        }                                                        \
    } while (0)

static void* dev(uintptr_t k) { return reinterpret_cast<void*>(0x100000u + 0x1000u * k); }

static ekv_shape shape(int B, int HQ, int G, int D, int MP, int NP, int kv, int st) {
    ekv_shape s;
    s.batch = B;
    s.num_q_heads = HQ;
    s.num_kv_groups = G;
    s.head_dim = D;
    s.page_size = 16;
    s.max_pages_per_seq = MP;
    s.num_phys_pages = NP;
    s.kv_dtype = kv;
    s.stat_dtype = st;
    return s;
}

static ekv_status decode_query(const ekv_shape& s, bool sparse, int stride, float alpha, size_t* bytes) {
    return ekv_entmax_decode(&s, dev(1), dev(2), dev(3), (const int32_t*)dev(4), (const int32_t*)dev(5),
                             sparse ? (const int32_t*)dev(6) : nullptr, sparse ? (const int32_t*)dev(7) : nullptr,
                             stride, alpha, nullptr, nullptr, (float*)dev(8), (float*)dev(9), nullptr, nullptr,
                             nullptr, nullptr, bytes, nullptr);
}

static ekv_status select_query(const ekv_shape& s, int sel, int budget, float alpha, size_t* bytes) {
    return ekv_select(&s, sel, (const int32_t*)dev(5), alpha, budget, 3.0f, (const float*)dev(10),
                      (const float*)dev(11), (const float*)dev(12), (int32_t*)dev(13), (int32_t*)dev(14),
                      (float*)dev(15), nullptr, bytes, nullptr);
}

int main() {
    CHECK(ekv_abi_version() == EKV_ABI_VERSION, "abi version %d", ekv_abi_version());
    CHECK(std::strcmp(ekv_last_error(), "") == 0 || std::strlen(ekv_last_error()) < 4096, "last error readable");

    // shape validation (query path)
    struct Bad { int B, HQ, G, D, P, kv, st; ekv_status want; };
    const Bad bad[] = {
        {2, 30, 8, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_INVALID_ARG},   // HQ not a multiple of G
        {2, 24, 8, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_UNSUPPORTED},   // r = 3
        {2, 32, 8, 96, 16, EKV_BF16, EKV_F32, EKV_ERR_UNSUPPORTED},    // D = 96
        {2, 32, 8, 128, 8, EKV_BF16, EKV_F32, EKV_ERR_UNSUPPORTED},    // P = 8
        {0, 32, 8, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_INVALID_ARG},   // B = 0
        {2, 32, 32, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_UNSUPPORTED},  // G > 16
        {2, 32, 8, 128, 16, 7, EKV_F32, EKV_ERR_UNSUPPORTED},          // bad kv dtype
        {2, 32, 8, 128, 16, EKV_BF16, 9, EKV_ERR_UNSUPPORTED},         // bad stat dtype
        {-3, 32, 8, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_INVALID_ARG},
        {2, 0, 8, 128, 16, EKV_BF16, EKV_F32, EKV_ERR_INVALID_ARG},
    };
    for (const Bad& b : bad) {
        ekv_shape s = shape(b.B, b.HQ, b.G, b.D, 64, 128, b.kv, b.st);
        s.page_size = b.P;
        size_t n = 0;
        const ekv_status st = decode_query(s, false, 0, 1.5f, &n);
        CHECK(st == b.want, "shape B=%d HQ=%d G=%d D=%d P=%d: status %d, want %d", b.B, b.HQ, b.G, b.D, b.P, st,
              b.want);
        CHECK(std::strlen(ekv_last_error()) > 0, "an error message after a rejected shape");
    }
    {
        size_t n = 0;
        CHECK(ekv_entmax_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1.5f,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &n,
                                nullptr) == EKV_ERR_INVALID_ARG, "null shape");
        const ekv_shape s = shape(2, 32, 8, 128, 64, 128, EKV_BF16, EKV_F32);
        CHECK(decode_query(s, false, 0, 1.5f, nullptr) == EKV_ERR_INVALID_ARG, "null workspace_bytes");
        CHECK(decode_query(s, false, 0, 0.5f, &n) != EKV_OK, "alpha < 1 rejected");
        CHECK(decode_query(s, true, 0, 1.5f, &n) != EKV_OK, "sparse with stride 0 rejected");
    }

    // decode workspace plans over a grid of shapes
    const int kvs[] = {EKV_BF16, EKV_F32};
    const int dims[] = {64, 128};
    const int hg[][2] = {{32, 8}, {8, 8}, {64, 8}, {8, 1}, {16, 16}, {12, 6}};
    const int batches[] = {1, 16, 64};
    const int mps[] = {1, 100, 8192, 65536, 1 << 20};
    const int strides[] = {0, 1, 256, 300, 4096, 65536};
    const float alphas[] = {1.0f, 4.0f / 3.0f, 1.5f, 2.0f, 3.0f};
    int plans = 0;
    for (int kv : kvs)
        for (int D : dims)
            for (const auto& h : hg)
                for (int B : batches)
                    for (int MP : mps)
                        for (int stride : strides)
                            for (float a : alphas) {
                                if (stride > MP) continue;
                                const ekv_shape s = shape(B, h[0], h[1], D, MP, MP, kv, EKV_F32);
                                size_t n1 = 0, n2 = 0;
                                const bool sparse = stride > 0;
                                const ekv_status s1 = decode_query(s, sparse, stride, a, &n1);
                                const ekv_status s2 = decode_query(s, sparse, stride, a, &n2);
                                CHECK(s1 == s2 && n1 == n2, "repeat query differs");
                                CHECK(s1 == EKV_OK || s1 == EKV_ERR_UNSUPPORTED, "decode plan status %d", s1);
                                if (s1 == EKV_OK) {
                                    CHECK(n1 > 0, "decode plan of 0 bytes");
                                    // one byte short: refused before anything is enqueued
                                    size_t m = n1 - 1;
                                    const ekv_status s3 = ekv_entmax_decode(
                                        &s, dev(1), dev(2), dev(3), (const int32_t*)dev(4), (const int32_t*)dev(5),
                                        sparse ? (const int32_t*)dev(6) : nullptr,
                                        sparse ? (const int32_t*)dev(7) : nullptr, stride, a, nullptr, nullptr,
                                        (float*)dev(8), (float*)dev(9), nullptr, nullptr, nullptr, dev(20), &m,
                                        nullptr);
                                    CHECK(s3 == EKV_ERR_WORKSPACE, "short workspace: status %d", s3);
                                    ++plans;
                                }
                            }
    CHECK(plans > 1000, "decode plans exercised: %d", plans);
    {
        // past what the streamed path builds (16M tokens per row): unsupported, not a wrong plan
        const ekv_shape s = shape(1, 32, 8, 128, 1 << 21, 1 << 21, EKV_BF16, EKV_F32);
        size_t n = 0;
        CHECK(decode_query(s, false, 0, 1.5f, &n) == EKV_ERR_UNSUPPORTED, "2M-page full-cache row");
        CHECK(decode_query(s, false, 0, 1.0f, &n) == EKV_ERR_UNSUPPORTED, "2M-page full-cache softmax row");
        const ekv_shape sf = shape(1, 32, 8, 128, 1 << 21, 1 << 21, EKV_F32, EKV_F32);
        CHECK(decode_query(sf, false, 0, 1.0f, &n) == EKV_ERR_UNSUPPORTED, "2M-page fp32 softmax row");
        CHECK(decode_query(sf, false, 0, 1.5f, &n) == EKV_ERR_UNSUPPORTED, "2M-page fp32 entmax row");
        // the longest supported row, in a ragged batch (the cache holds far fewer pages than B rows of it)
        const ekv_shape r = shape(4, 32, 8, 128, 1 << 20, 1 << 18, EKV_BF16, EKV_F32);
        CHECK(decode_query(r, false, 0, 1.5f, &n) == EKV_OK && n > 0, "1M-page row in a ragged batch");
        CHECK(decode_query(r, false, 0, 1.0f, &n) == EKV_OK && n > 0, "1M-page softmax row in a ragged batch");
    }

    // selection workspace plans
    const int sels[] = {EKV_SEL_TOPK, EKV_SEL_GAUSS, EKV_SEL_SUPERSET};
    const int budgets[] = {1, 128, 256, 4096, 65536};
    int splans = 0;
    for (int sel : sels)
        for (const auto& h : hg)
            for (int B : batches)
                for (int MP : mps)
                    for (int budget : budgets)
                        for (float a : alphas) {
                            const ekv_shape s = shape(B, h[0], h[1], 128, MP, MP, EKV_BF16, EKV_F32);
                            size_t n1 = 0, n2 = 0;
                            const ekv_status s1 = select_query(s, sel, budget, a, &n1);
                            const ekv_status s2 = select_query(s, sel, budget, a, &n2);
                            CHECK(s1 == s2 && n1 == n2, "repeat select query differs");
                            CHECK(s1 == EKV_OK || s1 == EKV_ERR_UNSUPPORTED || s1 == EKV_ERR_INVALID_ARG,
                                  "select status %d", s1);
                            if (s1 == EKV_OK) ++splans;
                        }
    CHECK(splans > 500, "selection plans exercised: %d", splans);
    {
        const ekv_shape s = shape(2, 32, 8, 128, 64, 128, EKV_BF16, EKV_F32);
        size_t n = 0;
        CHECK(select_query(s, 7, 16, 1.5f, &n) != EKV_OK, "unknown selector");
        CHECK(select_query(s, EKV_SEL_TOPK, 0, 1.5f, &n) != EKV_OK, "budget 0");
        CHECK(select_query(s, EKV_SEL_TOPK, 16, 1.5f, nullptr) == EKV_ERR_INVALID_ARG, "null workspace_bytes");
    }

    // required pointers of the compute calls
    {
        const ekv_shape s = shape(2, 32, 8, 128, 64, 128, EKV_BF16, EKV_F32);
        CHECK(ekv_build_page_stats(&s, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                                   nullptr) == EKV_ERR_INVALID_ARG, "page stats without inputs");
        CHECK(ekv_build_page_stats(&s, dev(2), (const int32_t*)dev(4), (const int32_t*)dev(5), nullptr, 0,
                                   nullptr, nullptr, nullptr, nullptr, nullptr) == EKV_ERR_INVALID_ARG,
              "page stats with no output");
        CHECK(ekv_append_kv(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr) == EKV_ERR_INVALID_ARG, "append without inputs");
        CHECK(ekv_score_pages(&s, EKV_SEL_TOPK, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, nullptr) == EKV_ERR_INVALID_ARG,
              "scores without inputs");
        CHECK(ekv_score_pages(&s, EKV_SEL_GAUSS, dev(1), (const int32_t*)dev(4), (const int32_t*)dev(5), nullptr,
                              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
                  EKV_ERR_INVALID_ARG,
              "Gaussian scores without statistics");
        CHECK(ekv_score_pages(&s, EKV_SEL_GAUSS, dev(1), (const int32_t*)dev(4), (const int32_t*)dev(5), nullptr,
                              nullptr, dev(6), dev(7), nullptr, (float*)dev(9), (float*)dev(10), (float*)dev(11),
                              nullptr) == EKV_ERR_INVALID_ARG,
              "per-head box scores asked of Gaussian scoring");
        CHECK(ekv_score_pages(&s, 5, dev(1), (const int32_t*)dev(4), (const int32_t*)dev(5), dev(2), dev(3),
                              dev(6), dev(7), (float*)dev(8), (float*)dev(9), (float*)dev(10), nullptr, nullptr) !=
                  EKV_OK,
              "unknown selector in scoring");
        size_t n = size_t(1) << 34;   // past any plan: the pointer checks are what answers
        CHECK(ekv_entmax_decode(&s, nullptr, dev(2), dev(3), (const int32_t*)dev(4), (const int32_t*)dev(5),
                                nullptr, nullptr, 0, 1.5f, nullptr, nullptr, (float*)dev(8), (float*)dev(9), nullptr,
                                nullptr, nullptr, dev(20), &n, nullptr) == EKV_ERR_INVALID_ARG, "decode without q");
        CHECK(ekv_entmax_decode(&s, dev(1), dev(2), dev(3), (const int32_t*)dev(4), (const int32_t*)dev(5),
                                nullptr, nullptr, 0, 1.5f, nullptr, nullptr, (float*)dev(8), (float*)dev(9), nullptr,
                                (float*)dev(10), nullptr, dev(20), &n, nullptr) == EKV_ERR_INVALID_ARG,
              "delta without tau_ref");
    }

    // the streaming-read probe's arguments
    {
        CHECK(ekv_probe_read(nullptr, 8192, nullptr, 4, 16, (uint32_t*)dev(1), nullptr) == EKV_ERR_INVALID_ARG,
              "probe without buffer");
        CHECK(ekv_probe_read(dev(1), 4097, nullptr, 4, 16, (uint32_t*)dev(2), nullptr) == EKV_ERR_INVALID_ARG,
              "probe size not a multiple of 4096");
        CHECK(ekv_probe_read(dev(1), 8192, nullptr, 3, 16, (uint32_t*)dev(2), nullptr) == EKV_ERR_UNSUPPORTED,
              "probe unroll 3");
        CHECK(ekv_probe_read(dev(1), 8192, nullptr, 4, 0, (uint32_t*)dev(2), nullptr) == EKV_ERR_INVALID_ARG,
              "probe with no blocks");
        CHECK(ekv_probe_read(dev(1), 8192, nullptr, 4, 16, nullptr, nullptr) == EKV_ERR_INVALID_ARG,
              "probe without sink");
    }

    std::printf("host checks: %d passed, %d failed\n", g_pass, g_fail);
    if (g_fail == 0) std::printf("host checks passed\n");
    return g_fail == 0 ? 0 : 1;
}
