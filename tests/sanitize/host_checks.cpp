// Host-side checks of libwoq's CPU functions, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py (no GPU code is
// compiled: the host translation units only).  Every call runs on ragged and
// degenerate shapes with exact-size buffers, so any read or write past a
// buffer, any use of freed memory and any undefined arithmetic aborts the
// program; the results themselves are checked by round trips and invariants.
// Exit status 0 and the line "host checks ok" mean every check passed.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include <unistd.h>

#include "woq.h"

static int failures = 0;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

static uint16_t f32_to_f16_bits(float f) {
    // round to nearest even via the hardware-independent bit route (normal range only)
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    int32_t e = (int32_t)((x >> 23) & 0xFF) - 127 + 15;
    uint32_t m = x & 0x7FFFFFu;
    if (e <= 0) return (uint16_t)sign;                       // tiny values flush to zero here
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);
    uint32_t h = sign | ((uint32_t)e << 10) | (m >> 13);
    const uint32_t rest = m & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) ++h;
    return (uint16_t)h;
}

static void check_int8(std::mt19937& rng) {
    std::normal_distribution<float> nd(0.f, 0.02f);
    const int64_t shapes[][2] = {{1, 1}, {3, 7}, {17, 65}, {5, 130}, {64, 64}};
    for (auto& sh : shapes) {
        const int64_t N = sh[0], K = sh[1];
        std::vector<float> W((size_t)(N * K));
        for (auto& v : W) v = nd(rng);
        std::vector<int8_t> q((size_t)(N * K));
        float s = -1.f;
        CHECK(woq_quantize_int8(W.data(), N, K, q.data(), &s) == WOQ_OK);
        CHECK(s > 0.f);
        for (size_t i = 0; i < W.size(); ++i) CHECK(std::fabs(W[i] - q[i] * s) <= 0.5f * s * 1.0001f);
        std::vector<uint8_t> dev((size_t)woq_int8_dev_bytes(N, K));
        CHECK(woq_layout_int8(q.data(), N, K, dev.data()) == WOQ_OK);
        std::vector<int8_t> back((size_t)(N * K));
        CHECK(woq_layout_int8_inverse(dev.data(), N, K, back.data()) == WOQ_OK);
        CHECK(back == q);
    }
    std::vector<float> Z(12, 0.f);
    std::vector<int8_t> qz(12, 5);
    float sz = -1.f;
    CHECK(woq_quantize_int8(Z.data(), 3, 4, qz.data(), &sz) == WOQ_OK && sz == 0.f && qz[11] == 0);
    Z[5] = NAN;
    CHECK(woq_quantize_int8(Z.data(), 3, 4, qz.data(), &sz) == WOQ_ERANGE);
    CHECK(woq_quantize_int8(nullptr, 3, 4, qz.data(), &sz) == WOQ_EINVAL);
}

static void check_int4o(std::mt19937& rng) {
    std::normal_distribution<float> nd(0.f, 0.02f);
    const int64_t shapes[][3] = {{1, 2, -1}, {3, 130, -1}, {17, 257, -1}, {4, 257, 0}, {2, 16, 16}, {9, 1000, 3}};
    for (auto& sh : shapes) {
        const int64_t N = sh[0], K = sh[1];
        woq_int4o_geom g;
        CHECK(woq_int4o_geometry(K, sh[2], &g) == WOQ_OK);
        std::vector<float> W((size_t)(N * K));
        for (auto& v : W) v = nd(rng);
        // selection over two "linears" (the same weight twice) and its sums form
        std::vector<uint16_t> xprof((size_t)(3 * K));
        for (auto& v : xprof) v = f32_to_f16_bits(std::fabs(nd(rng)) * 50.f + 0.01f);
        std::vector<int32_t> perm((size_t)K), perm2((size_t)K);
        const float* Ws[2] = {W.data(), W.data()};
        const int64_t Ns[2] = {N, N};
        CHECK(woq_outlier_perm(Ws, Ns, 2, K, xprof.data(), 3, g.n_out, perm.data()) == WOQ_OK);
        std::vector<double> cs1((size_t)K, 0.0), cs2((size_t)K, 0.0);
        CHECK(woq_colabs_accumulate(W.data(), N, K, cs1.data()) == WOQ_OK);
        CHECK(woq_colabs_accumulate(W.data(), N, K, cs2.data()) == WOQ_OK);
        const double* parts[2] = {cs1.data(), cs2.data()};
        CHECK(woq_outlier_perm_sums(parts, 2, K, xprof.data(), 3, g.n_out, perm2.data()) == WOQ_OK);
        CHECK(perm == perm2);
        std::vector<char> seen((size_t)K, 0);
        for (int32_t v : perm) {
            CHECK(v >= 0 && v < K);
            if (v >= 0 && v < K) seen[(size_t)v]++;
        }
        for (char c : seen) CHECK(c == 1);
        // encoding, unpacking, device layout and its inverse
        std::vector<uint8_t> packed((size_t)(N * g.K_pad / 2));
        std::vector<uint16_t> scales((size_t)(N * g.G)), wout((size_t)(N * g.n_out));
        CHECK(woq_quantize_int4o(W.data(), N, K, perm.data(), g.n_out, packed.data(), scales.data(), wout.data()) ==
              WOQ_OK);
        std::vector<int8_t> codes((size_t)(N * g.K_pad));
        CHECK(woq_unpack_int4(packed.data(), N, g.K_pad, codes.data()) == WOQ_OK);
        for (int8_t c : codes) CHECK(c >= -7 && c <= 7);
        int64_t cb = 0, sb = 0, wb = 0;
        CHECK(woq_int4o_dev_sizes(N, &g, &cb, &sb, &wb) == WOQ_OK);
        std::vector<uint8_t> dc((size_t)cb);
        std::vector<uint16_t> ds((size_t)(sb / 2)), dw((size_t)(wb / 2));
        CHECK(woq_layout_int4o(packed.data(), scales.data(), wout.data(), N, &g, dc.data(), ds.data(), dw.data()) ==
              WOQ_OK);
        std::vector<uint8_t> p2(packed.size());
        std::vector<uint16_t> s2(scales.size()), w2(wout.size());
        CHECK(woq_layout_int4o_inverse(dc.data(), ds.data(), dw.data(), N, &g, p2.data(), s2.data(), w2.data()) ==
              WOQ_OK);
        CHECK(p2 == packed && s2 == scales && w2 == wout);
        if (g.xp_len <= 65535) {
            std::vector<uint16_t> pos((size_t)((K + 7) / 8 * 8));
            CHECK(woq_perm_positions(perm.data(), &g, pos.data()) == WOQ_OK);
            for (int64_t j = 0; j < K; ++j) CHECK(pos[(size_t)j] < g.xp_len);
        }
    }
    // a non-permutation is refused before anything is written
    std::vector<float> W(8 * 4, 0.01f);
    std::vector<int32_t> bad = {0, 1, 1, 3};
    std::vector<uint8_t> packed(8 * 128 / 2, 0xAB);
    std::vector<uint16_t> scales(8, 0), wout(8, 0);
    CHECK(woq_quantize_int4o(W.data(), 8, 4, bad.data(), 1, packed.data(), scales.data(), wout.data()) == WOQ_EINVAL);
}

static void check_pool(const std::string& dir) {
    const std::string path = dir + "/host_checks.woqpool";
    std::vector<uint8_t> a(5000), b(1), c(1 << 20);
    for (size_t i = 0; i < a.size(); ++i) a[i] = (uint8_t)(i * 7);
    b[0] = 42;
    for (size_t i = 0; i < c.size(); ++i) c[i] = (uint8_t)(i >> 3);
    const void* blocks[3] = {a.data(), b.data(), c.data()};
    const int64_t sizes[3] = {(int64_t)a.size(), 1, (int64_t)c.size()};
    const char meta[] = "meta";
    CHECK(woq_pool_save(path.c_str(), meta, 4, blocks, sizes, 3) == WOQ_OK);
    int32_t n = 0;
    int64_t mb = 0, bs[3] = {0, 0, 0};
    char mbuf[4] = {0, 0, 0, 0};
    CHECK(woq_pool_info(path.c_str(), &n, &mb, bs, 3, mbuf, 4) == WOQ_OK);
    CHECK(n == 3 && mb == 4 && bs[0] == 5000 && bs[1] == 1 && bs[2] == (1 << 20) && std::memcmp(mbuf, "meta", 4) == 0);
    std::vector<uint8_t> back(c.size());
    CHECK(woq_pool_read_block(path.c_str(), 2, back.data(), (int64_t)back.size()) == WOQ_OK && back == c);
    std::vector<uint8_t> small(1);
    CHECK(woq_pool_read_block(path.c_str(), 1, small.data(), 1) == WOQ_OK && small[0] == 42);
    CHECK(woq_pool_read_block(path.c_str(), 2, small.data(), 1) != WOQ_OK);        // destination too small
    CHECK(woq_pool_read_block(path.c_str(), 7, back.data(), (int64_t)back.size()) != WOQ_OK);
    // flip one byte of the last block: its checksum must fail
    FILE* f = std::fopen(path.c_str(), "r+b");
    CHECK(f != nullptr);
    if (f) {
        std::fseek(f, -100, SEEK_END);
        int ch = std::fgetc(f);
        std::fseek(f, -100, SEEK_END);
        std::fputc(ch ^ 0x5A, f);
        std::fclose(f);
    }
    CHECK(woq_pool_read_block(path.c_str(), 2, back.data(), (int64_t)back.size()) == WOQ_EFORMAT);
    // a truncated file
    f = std::fopen(path.c_str(), "r+b");
    if (f) {
        std::fclose(f);
        CHECK(truncate(path.c_str(), 3000) == 0);
    }
    CHECK(woq_pool_read_block(path.c_str(), 2, back.data(), (int64_t)back.size()) != WOQ_OK);
    std::remove(path.c_str());
    CHECK(woq_pool_info((dir + "/missing.woqpool").c_str(), &n, &mb, nullptr, 0, nullptr, 0) != WOQ_OK);
}

int main(int argc, char** argv) {
    std::mt19937 rng(1234);
    check_int8(rng);
    check_int4o(rng);
    check_pool(argc > 1 ? argv[1] : "/tmp");
    for (int s = -9; s <= 0; ++s) CHECK(woq_strerror(s) != nullptr);
    if (failures) {
        std::printf("%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
