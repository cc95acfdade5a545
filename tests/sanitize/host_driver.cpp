// Host-only exercise of libpingala's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitize.py): the reference
// encoder on several shapes and thread counts, the tables, every argument
// check of the device calls (which must refuse before launching), and the
// per-thread error messages.  Exit 0 when every check holds; any sanitizer
// report aborts the run.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "../../include/pingala.h"

static int failures = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                               \
        }                                                             \
    } while (0)

static void encode_case(int64_t n, int64_t k, int threads, unsigned seed) {
    std::mt19937 rng(seed);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    std::vector<float> w((size_t)(n * k));
    for (auto& v : w) v = nd(rng);
    if (n > 1) std::fill(w.begin() + k, w.begin() + 2 * k, 0.0f);     // a zero row: zero scales, zero codes
    std::vector<uint8_t> signs((size_t)(k / 8));
    for (auto& s : signs) s = (uint8_t)(rng() & 0xff);
    std::vector<uint8_t> c1((size_t)(n * k / 4)), c2((size_t)(n * k / 4));
    std::vector<uint16_t> s1((size_t)(n * k / 128)), s2((size_t)(n * k / 128));
    CHECK(pg_encode_ref(w.data(), n, k, signs.data(), c1.data(), s1.data(), 1) == PG_OK);
    CHECK(pg_encode_ref(w.data(), n, k, signs.data(), c2.data(), s2.data(), threads) == PG_OK);
    CHECK(c1 == c2 && s1 == s2);                                        // thread count does not change the output
    if (n > 1) {
        for (int64_t i = 0; i < k / 4; ++i) CHECK(c1[(size_t)(k / 4 + i)] == 0);
        for (int64_t b = 0; b < k / 128; ++b) CHECK(s1[(size_t)(k / 128 + b)] == 0);
    }
}

int main() {
    CHECK(pg_version() == ((PG_FORMAT_VERSION << 16) | PG_LIB_VERSION));
    CHECK(pg_footprint_bytes(512, 2048) == 278528);
    CHECK(pg_footprint_bytes(0, 2048) == 0 && pg_footprint_bytes(4, 100) == 0);
    CHECK(pg_q16_row_bytes(2560) % 64 == 0 && pg_q16_row_bytes(100) == 0);
    std::vector<int8_t> tab(8 * 256 * 4);
    CHECK(pg_codebook_table(tab.data()) == PG_OK);
    for (int8_t v : tab) CHECK(v >= -7 && v <= 7 && (v & 1));
    CHECK(pg_codebook_table(nullptr) == PG_ERR_INVALID_ARG);

    encode_case(3, 128, 2, 1);
    encode_case(17, 384, 4, 2);
    encode_case(64, 2048, 0, 3);
    encode_case(1, 256, 8, 4);

    // argument checks: every device call refuses before launching
    alignas(64) static uint8_t buf[1 << 16];
    uint8_t* p = buf;
    const pg_stream_t st = nullptr;
    CHECK(pg_encode_ref(nullptr, 1, 128, p, p, (uint16_t*)p, 1) == PG_ERR_INVALID_ARG);
    CHECK(pg_encode_ref((float*)p, 1, 100, p, p, (uint16_t*)p, 1) == PG_ERR_INVALID_ARG);
    CHECK(pg_decode(p, (uint16_t*)p, 0, 256, (float*)p, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_decode(p + 4, (uint16_t*)p, 4, 256, (float*)p, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_decode_ex(p, (uint16_t*)p, 4, 256, 64, (float*)p, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_fwht_rotate(p, PG_F32, p, PG_F32, p, 1, 256, 0, st) == PG_ERR_INVALID_ARG);     // overlap
    CHECK(pg_fwht_rotate(p, 9, p + 4096, PG_F32, p, 1, 256, 0, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_fwht_rotate_ex(p, PG_F32, 100, p + 4096, PG_F32, p, 2, 256, 0, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_qgemv(p, (uint16_t*)p, 8, 256, p, PG_F32, 0, (float*)p, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_qgemv_ex(p, (uint16_t*)p, 8, 256, p, PG_Q16, 2, PG_FLAG_KERNEL_VDOT | PG_FLAG_KERNEL_MMA, (float*)p, st) ==
          PG_ERR_INVALID_ARG);
    CHECK(pg_rot_qgemv(p, (uint16_t*)p, 8, 256, p, PG_F16, 256, p, 64, 1, (float*)(p + 8192), st) == PG_ERR_INVALID_ARG);
    CHECK(pg_rot_qgemv(p, (uint16_t*)p, 8, 256, p, PG_F16, 200, p, 0, 1, (float*)(p + 8192), st) == PG_ERR_INVALID_ARG);
    CHECK(pg_qgemm(p, (uint16_t*)p, 8, 256, (uint16_t*)p, 0, (float*)p, st) == PG_ERR_INVALID_ARG);
    CHECK(pg_qgemm_ex(p, (uint16_t*)p, 8, 256, (uint16_t*)(p + 16384), 4, (float*)(p + 32768), p + 256, 64, st) ==
          PG_ERR_INVALID_ARG);                                                                  // overlaps codes
    CHECK(pg_qgemm_tune(p, (uint16_t*)p, 8, 256, (uint16_t*)p, 4, (float*)p, nullptr, 0, 9, 0, 0, st) ==
          PG_ERR_INVALID_ARG);
    CHECK(pg_hbm_read(p, 100, (uint32_t*)(p + 4096), st) == PG_ERR_INVALID_ARG);
    CHECK(pg_hbm_read(p, 4096, (uint32_t*)(p + 64), st) == PG_ERR_INVALID_ARG);             // out inside the range
    const int8_t* tb = (const int8_t*)(p + 8192);
    CHECK(pg_decode_table(p, (uint16_t*)p, 4, 256, tb, PG_FLAG_RMSNORM, (float*)(p + 16384), st) == PG_ERR_INVALID_ARG);
    CHECK(pg_decode_table(p, (uint16_t*)p, 4, 256, tb + 4, 0, (float*)(p + 16384), st) == PG_ERR_INVALID_ARG);
    CHECK(pg_rot_qgemv_table(p, (uint16_t*)p, 8, 256, p, PG_BF16, p, tb, 0, (float*)(p + 16384), st) ==
          PG_ERR_INVALID_ARG);
    CHECK(pg_rot_qgemv_table(p, (uint16_t*)p, 8, 256, p, PG_F16, p, tb, PG_FLAG_KERNEL_MMA, (float*)(p + 16384), st) ==
          PG_ERR_INVALID_ARG);
    CHECK(pg_rot_qgemv_table(p, (uint16_t*)p, 8, 256, p + 16384, PG_F16, p, tb, 0, (float*)(p + 16384), st) ==
          PG_ERR_INVALID_ARG);                                                                  // x, y overlap
    CHECK(std::strlen(pg_last_error()) > 0);
    // a valid request reaches the (stubbed) launcher
    CHECK(pg_decode(p, (uint16_t*)p, 4, 256, (float*)(p + 16384), st) == PG_ERR_UNSUPPORTED);
    CHECK(pg_decode_table(p, (uint16_t*)p, 4, 256, tb, PG_FLAG_CARRY_STATE, (float*)(p + 16384), st) ==
          PG_ERR_UNSUPPORTED);
    CHECK(pg_rot_qgemv_table(p, (uint16_t*)p, 8, 256, p + 4096, PG_F16, p, tb, PG_FLAG_RMSNORM, (float*)(p + 16384),
                             st) == PG_ERR_UNSUPPORTED);

    // messages are per thread
    std::string other;
    std::thread t([&] {
        CHECK(pg_decode(p, (uint16_t*)p, 0, 256, (float*)p, st) == PG_ERR_INVALID_ARG);
        other = pg_last_error();
    });
    t.join();
    CHECK(pg_codebook_table(tab.data()) == PG_OK);
    CHECK(std::strlen(pg_last_error()) == 0);
    CHECK(other.find("n must be") != std::string::npos);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
