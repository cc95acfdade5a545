// Host-side parts of libpingala: status/error plumbing, the decode table and
// the CPU reference encoder pg_encode_ref.  Plain C++17, no HIP calls.
//
// The trellis and rotation rules are those of format P8F v1, stated in
// include/pingala.h; their source is the "Pingala-8" landing page, section
// "How it works" (8-state Ungerboeck trellis over groups of 4 weights, the
// carried state choosing the next group's value set, random Hadamard
// rotation before coding).
#include <algorithm>
#include <cstdarg>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "pg_internal.h"

namespace pg {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

// level_j of byte c read in state s (format P8F v1)
void group_levels(int s, int c, int out[4]) {
    const int u = c & 1;
    const int z0 = (s >> 1) & 1;
    const int z1 = u ^ (s & 1) ^ ((s >> 2) & 1);
    int b[4] = {(c >> 1) & 1, (c >> 2) & 1, (c >> 3) & 1, 0};
    b[3] = z1 ^ b[0] ^ b[1] ^ b[2];
    for (int j = 0; j < 4; ++j) {
        const int e = (c >> (4 + j)) & 1;
        out[j] = 4 * (2 * e + b[j]) + 2 * z0 - 7;
    }
}

// level_j of byte c read in state s, rate-2/3 trellis (include/pingala.h):
// z0 = bit 0 of s, z1 = u0 ^ bit 1 of s, z2 = u1 ^ bit 2 of s; b0, b2 from
// bits 2, 3, b1 = b0 ^ z2, b3 = b2 ^ z1 ^ z2; e from bits 4..7
void group_levels_r23(int s, int c, int out[4]) {
    const int z0 = s & 1, z1 = (c & 1) ^ ((s >> 1) & 1), z2 = ((c >> 1) & 1) ^ ((s >> 2) & 1);
    const int b0 = (c >> 2) & 1, b2 = (c >> 3) & 1;
    const int b[4] = {b0, b0 ^ z2, b2, b2 ^ z1 ^ z2};
    for (int j = 0; j < 4; ++j) out[j] = 4 * (2 * ((c >> (4 + j)) & 1) + b[j]) + 2 * z0 - 7;
}

void build_codebook_r23(int8_t* out /* [8][256][4] */) {
    for (int s = 0; s < 8; ++s)
        for (int c = 0; c < 256; ++c) {
            int lv[4];
            group_levels_r23(s, c, lv);
            for (int j = 0; j < 4; ++j) out[(s * 256 + c) * 4 + j] = (int8_t)lv[j];
        }
}

void build_codebook(int8_t* out /* [8][256][4] */) {
    for (int s = 0; s < 8; ++s)
        for (int c = 0; c < 256; ++c) {
            int lv[4];
            group_levels(s, c, lv);
            for (int j = 0; j < 4; ++j) out[(s * 256 + c) * 4 + j] = (int8_t)lv[j];
        }
}

// IEEE binary16 bits of a double, round to nearest even (direct, no detour
// through float, so there is a single rounding).
uint16_t double_to_half_rne(double v) {
    const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (std::isnan(v)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;             // rounds to infinity
    if (a < 6.103515625e-05) {                          // below 2^-14: subnormal grid 2^-24
        double m = std::nearbyint(a * 16777216.0);      // exact scaling, RNE
        return sign | (uint16_t)m;                      // m == 1024 gives the smallest normal
    }
    int e;
    double f = std::frexp(a, &e);                       // a = f * 2^e, f in [0.5, 1)
    double m = std::nearbyint(std::ldexp(f, 11));       // 1024..2048
    if (m == 2048.0) { m = 1024.0; e += 1; }
    const int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)m - 1024);
}

double half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int exp = (h >> 10) & 0x1f;
    const int man = h & 0x3ff;
    double v;
    if (exp == 0) v = std::ldexp((double)man, -24);
    else if (exp == 31) v = man ? NAN : INFINITY;
    else v = std::ldexp((double)(man | 0x400), exp - 25);
    return sign ? -v : v;
}

namespace {

constexpr double kScaleC = 0.29;

struct CosetPoints {
    // [z0][z1][i][j]: level_j of the i-th point (byte bits 1..7 = i)
    double lv[2][2][128][4];
    CosetPoints() {
        for (int z0 = 0; z0 < 2; ++z0)
            for (int z1 = 0; z1 < 2; ++z1)
                for (int i = 0; i < 128; ++i) {
                    // a state with bit1 = z0 and bit0 = bit2 = 0 read with u = z1
                    int l[4];
                    group_levels(z0 << 1, (i << 1) | z1, l);
                    for (int j = 0; j < 4; ++j) lv[z0][z1][i][j] = (double)l[j];
                }
    }
};

// In-place orthonormal random-sign Hadamard transform of one 128-block (fp64):
// v <- 2^-3.5 * H * diag(sigma) * v.
void rotate_block(double* v, const uint8_t* sign_bits, int64_t k0) {
    for (int i = 0; i < 128; ++i) {
        const int64_t kk = k0 + i;
        if ((sign_bits[kk >> 3] >> (kk & 7)) & 1) v[i] = -v[i];
    }
    for (int h = 1; h < 128; h <<= 1)
        for (int i = 0; i < 128; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                const double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
    const double c = std::ldexp(std::sqrt(2.0), -4);   // 2^-3.5
    for (int i = 0; i < 128; ++i) v[i] *= c;
}

void encode_block(const double* w, uint16_t scale_bits, const CosetPoints& P, uint8_t* out) {
    const double s = half_to_double(scale_bits);
    double bm[32][2][2];
    int barg[32][2][2];
    for (int t = 0; t < 32; ++t)
        for (int z0 = 0; z0 < 2; ++z0)
            for (int z1 = 0; z1 < 2; ++z1) {
                double best = INFINITY;
                int arg = 0;
                for (int i = 0; i < 128; ++i) {
                    const double* p = P.lv[z0][z1][i];
                    const double d0 = w[4 * t + 0] - s * p[0];
                    const double d1 = w[4 * t + 1] - s * p[1];
                    const double d2 = w[4 * t + 2] - s * p[2];
                    const double d3 = w[4 * t + 3] - s * p[3];
                    const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
                    if (m < best) { best = m; arg = i; }
                }
                bm[t][z0][z1] = best;
                barg[t][z0][z1] = arg;
            }
    double metric[8], next[8];
    int8_t prev[32][8];
    uint8_t byte[32][8];
    for (int st = 0; st < 8; ++st) metric[st] = INFINITY;
    metric[0] = 0.0;
    for (int t = 0; t < 32; ++t) {
        for (int sn = 0; sn < 8; ++sn) {
            const int u = sn & 1;
            next[sn] = INFINITY;
            prev[t][sn] = 0;
            byte[t][sn] = 0;
            const int cand[2] = {sn >> 1, (sn >> 1) | 4};
            for (int c = 0; c < 2; ++c) {
                const int cs = cand[c];
                const int z0 = (cs >> 1) & 1;
                const int z1 = u ^ (cs & 1) ^ ((cs >> 2) & 1);
                const double tot = metric[cs] + bm[t][z0][z1];
                if (tot < next[sn]) {
                    next[sn] = tot;
                    prev[t][sn] = (int8_t)cs;
                    byte[t][sn] = (uint8_t)((barg[t][z0][z1] << 1) | u);
                }
            }
        }
        std::memcpy(metric, next, sizeof(metric));
    }
    int st = 0;
    for (int q = 1; q < 8; ++q)
        if (metric[q] < metric[st]) st = q;
    for (int t = 31; t >= 0; --t) {
        out[t] = byte[t][st];
        st = prev[t][st];
    }
    if (s == 0.0) std::memset(out, 0, 32);
}

// level_j of every weight of one block from its 32 code bytes (state 0 at the start)
void decode_block_levels(const uint8_t* c, double* lv) {
    int st = 0;
    for (int t = 0; t < 32; ++t) {
        int l[4];
        group_levels(st, c[t], l);
        for (int j = 0; j < 4; ++j) lv[4 * t + j] = (double)l[j];
        st = ((st << 1) | (c[t] & 1)) & 7;
    }
}

// run f(r) for r in [0, count) on up to n_threads threads
template <class F>
void parallel_rows(int64_t count, int n_threads, F f) {
    if (n_threads <= 0) n_threads = (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
    n_threads = (int)std::max<int64_t>(1, std::min<int64_t>(n_threads, count));
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (;;) {
            const int64_t r = next.fetch_add(1);
            if (r >= count) break;
            f(r);
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker);
    worker();
    for (auto& th : pool) th.join();
}

}  // namespace

// Viterbi through a codebook table (P8F v1's trellis, or the rate-2/3 one):
// for every group, state p and byte c the distortion ((d0^2 + d1^2) + d2^2)
// + d3^2 with d_j = w_j - s * T[p][c][j]; per state and branch u (the byte's
// branch bits) the first byte of least distortion; add-compare-select from
// state 0 with each next state's predecessors in increasing order, strict
// improvement, the first best end state; a zero scale codes byte 0.
void encode_block_table(const double* w, uint16_t scale_bits, const int8_t* table, bool r23, uint8_t* out) {
    const double s = half_to_double(scale_bits);
    if (s == 0.0) {
        std::memset(out, 0, 32);
        return;
    }
    const int nbr = r23 ? 4 : 2, um = nbr - 1;
    static thread_local double bd[32][8][4];
    static thread_local uint8_t bc[32][8][4];
    for (int t = 0; t < 32; ++t)
        for (int p = 0; p < 8; ++p) {
            for (int u = 0; u < nbr; ++u) bd[t][p][u] = INFINITY;
            for (int c = 0; c < 256; ++c) {
                const int8_t* L = table + (p * 256 + c) * 4;
                const double d0 = w[4 * t + 0] - s * (double)L[0];
                const double d1 = w[4 * t + 1] - s * (double)L[1];
                const double d2 = w[4 * t + 2] - s * (double)L[2];
                const double d3 = w[4 * t + 3] - s * (double)L[3];
                const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
                const int u = c & um;
                if (m < bd[t][p][u]) {
                    bd[t][p][u] = m;
                    bc[t][p][u] = (uint8_t)c;
                }
            }
        }
    double metric[8], next[8];
    int8_t prev[32][8];
    uint8_t byte[32][8];
    for (int st = 0; st < 8; ++st) metric[st] = INFINITY;
    metric[0] = 0.0;
    for (int t = 0; t < 32; ++t) {
        for (int sn = 0; sn < 8; ++sn) next[sn] = INFINITY;
        for (int p = 0; p < 8; ++p)
            for (int u = 0; u < nbr; ++u) {
                const int sn = r23 ? ((p << 2) | u) & 7 : ((p << 1) | u) & 7;
                const double tot = metric[p] + bd[t][p][u];
                if (tot < next[sn]) {
                    next[sn] = tot;
                    prev[t][sn] = (int8_t)p;
                    byte[t][sn] = bc[t][p][u];
                }
            }
        std::memcpy(metric, next, sizeof(metric));
    }
    int st = 0;
    for (int q = 1; q < 8; ++q)
        if (metric[q] < metric[st]) st = q;
    for (int t = 31; t >= 0; --t) {
        out[t] = byte[t][st];
        st = prev[t][st];
    }
}

int encode_ref_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                     bool r23, uint8_t* codes, uint16_t* scales, int n_threads) {
    const int64_t nb = k / 128;
    parallel_rows(n, n_threads, [&](int64_t r) {
        std::vector<double> v(128);
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 128; ++i) v[i] = (double)w[r * k + b * 128 + i];
            rotate_block(v.data(), sign_bits, b * 128);
            double acc = 0.0;
            for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
            const double rms = std::sqrt(acc / 128.0);
            const double val = std::min(kScaleC * rms, 65504.0);
            const uint16_t sb = double_to_half_rne(val);
            scales[r * nb + b] = sb;
            encode_block_table(v.data(), sb, table, r23, codes + r * (k / 4) + b * 32);
        }
    });
    return PG_OK;
}

// LDLQ feedback (landing page, "How it works": LDLQ rounding).  H~ = R H R^T
// (the block rotation on both sides), then H~ = U D U^T with U unit upper
// block-triangular and D block-diagonal (blocks of 128), eliminating blocks
// from the last one up: U[<j, j] = H[<j, j] D_j^-1 through a Cholesky of D_j,
// then H[<j, <j] -= U[<j, j] H[<j, j]^T.  fb receives U - I (k x k,
// row-major; only blocks above the diagonal are non-zero).
int ldlq_feedback(const double* hessian, int64_t k, const uint8_t* sign_bits, int n_threads, double* fb) {
    const int64_t nb = k / 128;
    for (int64_t i = 0; i < k * k; ++i)
        if (!std::isfinite(hessian[i])) return fail(PG_ERR_INVALID_ARG, "hessian holds a non-finite value");
    double amax = 0.0;
    for (int64_t i = 0; i < k * k; ++i) amax = std::max(amax, std::fabs(hessian[i]));
    for (int64_t r = 0; r < k; ++r)
        for (int64_t c = r + 1; c < k; ++c)
            if (std::fabs(hessian[r * k + c] - hessian[c * k + r]) > 1e-12 * amax)
                return fail(PG_ERR_INVALID_ARG, "hessian is not symmetric (entries %lld, %lld)", (long long)r,
                            (long long)c);
    std::vector<double> a((size_t)(k * k)), tmp((size_t)(k * k));
    // H R^T: every row's blocks rotated; then the same on the transpose
    parallel_rows(k, n_threads, [&](int64_t r) {
        std::memcpy(&tmp[(size_t)(r * k)], hessian + r * k, sizeof(double) * (size_t)k);
        for (int64_t b = 0; b < nb; ++b) rotate_block(&tmp[(size_t)(r * k + b * 128)], sign_bits, b * 128);
    });
    parallel_rows(k, n_threads, [&](int64_t r) {
        for (int64_t c = 0; c < k; ++c) a[(size_t)(r * k + c)] = tmp[(size_t)(c * k + r)];
        for (int64_t b = 0; b < nb; ++b) rotate_block(&a[(size_t)(r * k + b * 128)], sign_bits, b * 128);
    });
    std::fill(fb, fb + k * k, 0.0);
    std::vector<double> chol(128 * 128);
    for (int64_t j = nb - 1; j >= 1; --j) {
        const int64_t j0 = j * 128;
        // Cholesky of D_j = a[j0.., j0..]: chol lower triangular
        for (int p = 0; p < 128; ++p) {
            for (int q = 0; q <= p; ++q) {
                double v = a[(size_t)((j0 + p) * k + j0 + q)];
                for (int t = 0; t < q; ++t) v -= chol[p * 128 + t] * chol[q * 128 + t];
                if (p == q) {
                    if (!(v > 0.0)) return fail(PG_ERR_INVALID_ARG, "hessian is not positive definite");
                    chol[p * 128 + p] = std::sqrt(v);
                } else {
                    chol[p * 128 + q] = v / chol[q * 128 + q];
                }
            }
        }
        // rows above: D_j x = a[r, block j]^T, x = U[r, block j]
        parallel_rows(j0, n_threads, [&](int64_t r) {
            double y[128];
            const double* h = &a[(size_t)(r * k + j0)];
            for (int p = 0; p < 128; ++p) {
                double v = h[p];
                for (int t = 0; t < p; ++t) v -= chol[p * 128 + t] * y[t];
                y[p] = v / chol[p * 128 + p];
            }
            double* x = fb + r * k + j0;
            for (int p = 127; p >= 0; --p) {
                double v = y[p];
                for (int t = p + 1; t < 128; ++t) v -= chol[t * 128 + p] * x[t];
                x[p] = v / chol[p * 128 + p];
            }
        });
        // Schur complement of the rows and columns above block j
        parallel_rows(j0, n_threads, [&](int64_t r) {
            const double* x = fb + r * k + j0;
            for (int64_t c = 0; c <= r; ++c) {
                const double* h = &a[(size_t)(c * k + j0)];
                double v = 0.0;
                for (int q = 0; q < 128; ++q) v += x[q] * h[q];
                a[(size_t)(r * k + c)] -= v;
            }
        });
        parallel_rows(j0, n_threads, [&](int64_t r) {
            for (int64_t c = r + 1; c < j0; ++c) a[(size_t)(r * k + c)] = a[(size_t)(c * k + r)];
        });
    }
    // the first block's D must be positive definite too
    for (int p = 0; p < 128; ++p)
        for (int q = 0; q <= p; ++q) {
            double v = a[(size_t)(p * k + q)];
            for (int t = 0; t < q; ++t) v -= chol[p * 128 + t] * chol[q * 128 + t];
            if (p == q) {
                if (!(v > 0.0)) return fail(PG_ERR_INVALID_ARG, "hessian is not positive definite");
                chol[p * 128 + p] = std::sqrt(v);
            } else {
                chol[p * 128 + q] = v / chol[q * 128 + q];
            }
        }
    return PG_OK;
}

// Reference LDLQ encoder: per row, blocks in order; block b's target is
// t_c = v_c + sum_{c' < 128 b} e_c' * fb[c'][128 b + c] (increasing c', one
// rounding per product and per sum), v the rotated weights and e = v - What
// of the blocks already coded; scale rule and Viterbi as encode_ref.
int encode_ref_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* fb,
                    uint8_t* codes, uint16_t* scales, int n_threads) {
    static const CosetPoints P;
    const int64_t nb = k / 128;
    parallel_rows(n, n_threads, [&](int64_t r) {
        std::vector<double> e((size_t)k), v(128), t(128), lv(128);
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 128; ++i) v[i] = (double)w[r * k + b * 128 + i];
            rotate_block(v.data(), sign_bits, b * 128);
            for (int i = 0; i < 128; ++i) {
                double acc = 0.0;
                for (int64_t cp = 0; cp < b * 128; ++cp) acc = acc + e[(size_t)cp] * fb[cp * k + b * 128 + i];
                t[i] = v[i] + acc;
            }
            double acc = 0.0;
            for (int i = 0; i < 128; ++i) acc = acc + t[i] * t[i];
            const double rms = std::sqrt(acc / 128.0);
            const double val = std::min(kScaleC * rms, 65504.0);
            const uint16_t sb = double_to_half_rne(val);
            scales[r * nb + b] = sb;
            uint8_t* cb = codes + r * (k / 4) + b * 32;
            encode_block(t.data(), sb, P, cb);
            decode_block_levels(cb, lv.data());
            const double s = half_to_double(sb);
            for (int i = 0; i < 128; ++i) e[(size_t)(b * 128 + i)] = v[i] - s * lv[i];
        }
    });
    return PG_OK;
}

int encode_ref(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
               uint16_t* scales, int n_threads) {
    static const CosetPoints P;
    const int64_t nb = k / 128;
    if (n_threads <= 0) n_threads = (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
    n_threads = (int)std::min<int64_t>(n_threads, n);
    std::atomic<int64_t> next_row{0};
    auto worker = [&]() {
        std::vector<double> v(128);
        for (;;) {
            const int64_t r = next_row.fetch_add(1);
            if (r >= n) break;
            for (int64_t b = 0; b < nb; ++b) {
                for (int i = 0; i < 128; ++i) v[i] = (double)w[r * k + b * 128 + i];
                rotate_block(v.data(), sign_bits, b * 128);
                double acc = 0.0;
                for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
                const double rms = std::sqrt(acc / 128.0);
                const double val = std::min(kScaleC * rms, 65504.0);
                const uint16_t sb = double_to_half_rne(val);
                scales[r * nb + b] = sb;
                encode_block(v.data(), sb, P, codes + r * (k / 4) + b * 32);
            }
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker);
    worker();
    for (auto& th : pool) th.join();
    return PG_OK;
}

}  // namespace pg
