// libpingala: the trellis encoder on the GPU (pg_encode).
//
// Pingala-8 landing page, "How it works": weights are rotated by a random
// Hadamard transform, then coded group by group (4 weights per group) along an
// 8-state trellis whose state, carried from group to group, picks the value
// set the next group may use; the rounding is LDLQ, here with an identity
// Hessian, i.e. plain minimum squared error found by a Viterbi search.  Format
// P8F v1 as stated in include/pingala.h.
//
// One workgroup of 128 threads codes one 128-block of one row and reproduces
// the host reference encoder (pg_encode_ref) bit for bit: every step runs in
// fp64 in the reference's operation order, with no fused multiply-add:
//   1. thread i loads weight i, applies the site's sign, and the block is
//      rotated in LDS by seven butterfly stages (each output depends only on
//      the previous stage, so the parallel order gives the same values), then
//      multiplied by 2^-3.5;
//   2. thread 0 sums the squares in index order, and the scale is
//      fp16_RNE(min(0.29 * rms, 65504));
//   3. thread 4 t + c scores the 128 points of coset c = (z0, z1) against group
//      t (distortion ((d0^2 + d1^2) + d2^2) + d3^2, first minimum kept);
//   4. threads 0..7 run the add-compare-select of the 32 trellis steps, one
//      next state each (ties keep the predecessor s' >> 1); thread 0 picks the
//      first best end state and traces the path back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "pg_internal.h"

namespace pg {
namespace {

// fp16 bits of a double, round to nearest even (one rounding), as the host
// reference does it
__device__ uint16_t enc_half_rne(double v) {
#pragma clang fp contract(off)
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (isnan(v)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;
    if (a < 6.103515625e-05) return sign | (uint16_t)rint(a * 16777216.0);
    int e;
    const double f = frexp(a, &e);
    double m = rint(ldexp(f, 11));
    if (m == 2048.0) { m = 1024.0; e += 1; }
    const int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)m - 1024);
}

__device__ double enc_half_to_double(uint16_t h) {
    const int exp = (h >> 10) & 0x1f, man = h & 0x3ff;
    double v;
    if (exp == 0) v = ldexp((double)man, -24);
    else if (exp == 31) v = man ? __builtin_nan("") : __builtin_inf();
    else v = ldexp((double)(man | 0x400), exp - 25);
    return (h >> 15) ? -v : v;
}

__global__ __launch_bounds__(128) void k_encode(const float* __restrict__ w, int n, int k,
                                                const uint8_t* __restrict__ sign_bits,
                                                uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
#pragma clang fp contract(off)
    __shared__ double v[128];
    __shared__ double bm[32][4];          // best distortion of group t in coset 2 z0 + z1
    __shared__ int barg[32][4];           // its point: byte bits 1..7
    __shared__ double metric[8];
    __shared__ int8_t prv[32][8];
    __shared__ uint8_t byt[32][8];
    __shared__ uint32_t sbits;
    const int tid = threadIdx.x;
    const int nb = k >> 7;
    const int row = blockIdx.x / nb, b = blockIdx.x - row * nb;
    const int64_t kk = (int64_t)b * 128 + tid;

    // ---- 1. signed input, seven butterfly stages, 2^-3.5
    double x = (double)w[(int64_t)row * k + kk];
    if ((sign_bits[kk >> 3] >> (kk & 7)) & 1) x = -x;
    v[tid] = x;
    __syncthreads();
    for (int h = 1; h < 128; h <<= 1) {
        const int j = (tid / h) * 2 * h + (tid % h);    // pair (j, j + h) of thread tid < 64
        double a = 0.0, c = 0.0;
        if (tid < 64) { a = v[j]; c = v[j + h]; }
        __syncthreads();
        if (tid < 64) { v[j] = a + c; v[j + h] = a - c; }
        __syncthreads();
    }
    v[tid] = v[tid] * 0x1.6a09e667f3bcdp-4;              // 2^-3.5 = sqrt(2) / 16, rounded once
    __syncthreads();

    // ---- 2. scale from the RMS of the rotated block
    if (tid == 0) {
        double acc = 0.0;
        for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
        const double rms = sqrt(acc / 128.0);
        const double sc = 0.29 * rms;
        const double val = 65504.0 < sc ? 65504.0 : sc;  // std::min's order (a NaN passes through)
        sbits = enc_half_rne(val);
        scales[(int64_t)row * nb + b] = (uint16_t)sbits;
    }
    __syncthreads();
    const double s = enc_half_to_double((uint16_t)sbits);

    // ---- 3. branch metrics: nearest point of coset (z0, z1) to group t.
    // Point i is byte (i << 1) | z1 read in a state with bit 1 = z0 and
    // bits 0, 2 clear: b0..b2 = bits 0..2 of i, b3 = z1 ^ b0 ^ b1 ^ b2,
    // e_j = bit 3 + j of i, level_j = 4 (2 e_j + b_j) + 2 z0 - 7.
    {
        const int t = tid >> 2, cs = tid & 3, z0 = cs >> 1, z1 = cs & 1;
        const double w0 = v[4 * t], w1 = v[4 * t + 1], w2 = v[4 * t + 2], w3 = v[4 * t + 3];
        double best = __builtin_inf();
        int arg = 0;
        for (int i = 0; i < 128; ++i) {
            const int b0 = i & 1, b1 = (i >> 1) & 1, b2 = (i >> 2) & 1, b3 = z1 ^ b0 ^ b1 ^ b2;
            const double p0 = (double)(4 * (2 * ((i >> 3) & 1) + b0) + 2 * z0 - 7);
            const double p1 = (double)(4 * (2 * ((i >> 4) & 1) + b1) + 2 * z0 - 7);
            const double p2 = (double)(4 * (2 * ((i >> 5) & 1) + b2) + 2 * z0 - 7);
            const double p3 = (double)(4 * (2 * ((i >> 6) & 1) + b3) + 2 * z0 - 7);
            const double d0 = w0 - s * p0, d1 = w1 - s * p1, d2 = w2 - s * p2, d3 = w3 - s * p3;
            const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
            if (m < best) { best = m; arg = i; }
        }
        bm[t][cs] = best;
        barg[t][cs] = arg;
    }
    if (tid < 8) metric[tid] = tid == 0 ? 0.0 : __builtin_inf();
    __syncthreads();

    // ---- 4. add-compare-select from state 0, free end state
    for (int t = 0; t < 32; ++t) {
        double nxt = __builtin_inf();
        if (tid < 8) {
            const int sn = tid, u = sn & 1;
            int pv = 0, by = 0;
            for (int c = 0; c < 2; ++c) {
                const int ps = c == 0 ? sn >> 1 : (sn >> 1) | 4;
                const int z0 = (ps >> 1) & 1, z1 = u ^ (ps & 1) ^ ((ps >> 2) & 1);
                const double tot = metric[ps] + bm[t][2 * z0 + z1];
                if (tot < nxt) { nxt = tot; pv = ps; by = (barg[t][2 * z0 + z1] << 1) | u; }
            }
            prv[t][sn] = (int8_t)pv;
            byt[t][sn] = (uint8_t)by;
        }
        __syncthreads();
        if (tid < 8) metric[tid] = nxt;
        __syncthreads();
    }
    if (tid == 0) {
        int st = 0;
        for (int q = 1; q < 8; ++q)
            if (metric[q] < metric[st]) st = q;
        uint8_t out[32];
        for (int t = 31; t >= 0; --t) {
            out[t] = byt[t][st];
            st = prv[t][st];
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (int64_t)row * (k >> 2) + 32 * b);
        for (int i = 0; i < 8; ++i) {
            const uint32_t wv = (uint32_t)out[4 * i] | ((uint32_t)out[4 * i + 1] << 8) |
                                ((uint32_t)out[4 * i + 2] << 16) | ((uint32_t)out[4 * i + 3] << 24);
            dst[i] = s == 0.0 ? 0u : wv;                    // a zero scale codes every group as byte 0
        }
    }
}

// LDLQ variant (landing page, "How it works": LDLQ rounding): one launch per
// 128-block b, one workgroup per row.  Thread i rotates weight i of the
// block as above (v_i), adds the feedback of the blocks already coded,
//   t_i = v_i + sum_{c < 128 b} err[row][c] * fb[c][128 b + i]
// (increasing c, one rounding per product and per sum, as the host
// reference), and the block is coded against t by the steps above; then
// thread i decodes its own weight from the chosen bytes and stores
// err[row][128 b + i] = v_i - s * level_i for the next blocks.
__global__ __launch_bounds__(128) void k_encode_ldlq(const float* __restrict__ w, int n, int k,
                                                     const uint8_t* __restrict__ sign_bits,
                                                     const double* __restrict__ fb, double* __restrict__ err,
                                                     uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                     int b) {
#pragma clang fp contract(off)
    __shared__ double v[128];
    __shared__ double bm[32][4];
    __shared__ int barg[32][4];
    __shared__ double metric[8];
    __shared__ int8_t prv[32][8];
    __shared__ uint8_t byt[32][8];
    __shared__ uint8_t out[32];
    __shared__ uint32_t sbits;
    const int tid = threadIdx.x;
    const int nb = k >> 7;
    const int row = blockIdx.x;
    const int64_t kk = (int64_t)b * 128 + tid;

    // ---- 1. rotation (as k_encode)
    double x = (double)w[(int64_t)row * k + kk];
    if ((sign_bits[kk >> 3] >> (kk & 7)) & 1) x = -x;
    v[tid] = x;
    __syncthreads();
    for (int h = 1; h < 128; h <<= 1) {
        const int j = (tid / h) * 2 * h + (tid % h);
        double a = 0.0, c = 0.0;
        if (tid < 64) { a = v[j]; c = v[j + h]; }
        __syncthreads();
        if (tid < 64) { v[j] = a + c; v[j + h] = a - c; }
        __syncthreads();
    }
    const double vr = v[tid] * 0x1.6a09e667f3bcdp-4;

    // ---- LDLQ feedback of the coded blocks: the loads run ahead, the sum in order
    {
        const double* e = err + (int64_t)row * k;
        const double* f = fb + kk;
        double acc = 0.0;
        const int m = 128 * b;
        int c = 0;
        for (; c + 8 <= m; c += 8) {
            double p[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) p[q] = e[c + q] * f[(int64_t)(c + q) * k];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = acc + p[q];
        }
        for (; c < m; ++c) acc = acc + e[c] * f[(int64_t)c * k];
        __syncthreads();
        v[tid] = vr + acc;
    }
    __syncthreads();

    // ---- 2. scale from the RMS of the target
    if (tid == 0) {
        double acc = 0.0;
        for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
        const double rms = sqrt(acc / 128.0);
        const double sc = 0.29 * rms;
        const double val = 65504.0 < sc ? 65504.0 : sc;
        sbits = enc_half_rne(val);
        scales[(int64_t)row * nb + b] = (uint16_t)sbits;
    }
    __syncthreads();
    const double s = enc_half_to_double((uint16_t)sbits);

    // ---- 3. branch metrics (as k_encode)
    {
        const int t = tid >> 2, cs = tid & 3, z0 = cs >> 1, z1 = cs & 1;
        const double w0 = v[4 * t], w1 = v[4 * t + 1], w2 = v[4 * t + 2], w3 = v[4 * t + 3];
        double best = __builtin_inf();
        int arg = 0;
        for (int i = 0; i < 128; ++i) {
            const int b0 = i & 1, b1 = (i >> 1) & 1, b2 = (i >> 2) & 1, b3 = z1 ^ b0 ^ b1 ^ b2;
            const double p0 = (double)(4 * (2 * ((i >> 3) & 1) + b0) + 2 * z0 - 7);
            const double p1 = (double)(4 * (2 * ((i >> 4) & 1) + b1) + 2 * z0 - 7);
            const double p2 = (double)(4 * (2 * ((i >> 5) & 1) + b2) + 2 * z0 - 7);
            const double p3 = (double)(4 * (2 * ((i >> 6) & 1) + b3) + 2 * z0 - 7);
            const double d0 = w0 - s * p0, d1 = w1 - s * p1, d2 = w2 - s * p2, d3 = w3 - s * p3;
            const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
            if (m < best) { best = m; arg = i; }
        }
        bm[t][cs] = best;
        barg[t][cs] = arg;
    }
    if (tid < 8) metric[tid] = tid == 0 ? 0.0 : __builtin_inf();
    __syncthreads();

    // ---- 4. add-compare-select and traceback (as k_encode)
    for (int t = 0; t < 32; ++t) {
        double nxt = __builtin_inf();
        if (tid < 8) {
            const int sn = tid, u = sn & 1;
            int pv = 0, by = 0;
            for (int c = 0; c < 2; ++c) {
                const int ps = c == 0 ? sn >> 1 : (sn >> 1) | 4;
                const int z0 = (ps >> 1) & 1, z1 = u ^ (ps & 1) ^ ((ps >> 2) & 1);
                const double tot = metric[ps] + bm[t][2 * z0 + z1];
                if (tot < nxt) { nxt = tot; pv = ps; by = (barg[t][2 * z0 + z1] << 1) | u; }
            }
            prv[t][sn] = (int8_t)pv;
            byt[t][sn] = (uint8_t)by;
        }
        __syncthreads();
        if (tid < 8) metric[tid] = nxt;
        __syncthreads();
    }
    if (tid == 0) {
        int st = 0;
        for (int q = 1; q < 8; ++q)
            if (metric[q] < metric[st]) st = q;
        for (int t = 31; t >= 0; --t) {
            out[t] = s == 0.0 ? 0 : byt[t][st];             // a zero scale codes every group as byte 0
            st = prv[t][st];
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (int64_t)row * (k >> 2) + 32 * b);
        for (int i = 0; i < 8; ++i)
            dst[i] = (uint32_t)out[4 * i] | ((uint32_t)out[4 * i + 1] << 8) | ((uint32_t)out[4 * i + 2] << 16) |
                     ((uint32_t)out[4 * i + 3] << 24);
    }
    __syncthreads();

    // ---- 5. the error of this weight: state from the three bytes before its group
    {
        const int t = tid >> 2, j = tid & 3;
        int st = 0;
        for (int q = t - 3; q < t; ++q)
            if (q >= 0) st = ((st << 1) | (out[q] & 1)) & 7;
        const int c = out[t], u = c & 1, z0 = (st >> 1) & 1, z1 = u ^ (st & 1) ^ ((st >> 2) & 1);
        const int bb0 = (c >> 1) & 1, bb1 = (c >> 2) & 1, bb2 = (c >> 3) & 1;
        const int bj = j == 0 ? bb0 : j == 1 ? bb1 : j == 2 ? bb2 : (z1 ^ bb0 ^ bb1 ^ bb2);
        const int lvl = 4 * (2 * ((c >> (4 + j)) & 1) + bj) + 2 * z0 - 7;
        err[(int64_t)row * k + kk] = vr - s * (double)lvl;
    }
}

// Through a codebook table (P8F v1's trellis or the rate-2/3 one), the
// host reference's encode_block_table step for step: one 128-thread
// workgroup per 128-block copies the 8 KB table to LDS, rotates and scales
// the block as k_encode does; thread i scores every byte of state p = i % 8
// against groups i / 8 and 16 + i / 8 (first byte of least distortion per
// branch); threads 0..7 run the add-compare-select (predecessors in
// increasing order), thread 0 traces back.
__global__ __launch_bounds__(128) void k_encode_table(const float* __restrict__ w, int n, int k,
                                                      const uint8_t* __restrict__ sign_bits,
                                                      const uint4* __restrict__ table, int r23,
                                                      uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
#pragma clang fp contract(off)
    __shared__ uint4 tab[512];
    __shared__ double v[128];
    __shared__ double bd[32][8][4];
    __shared__ uint8_t bc[32][8][4];
    __shared__ double metric[8];
    __shared__ int8_t prv[32][8];
    __shared__ uint8_t byt[32][8];
    __shared__ uint32_t sbits;
    const int tid = threadIdx.x;
    const int nb = k >> 7;
    const int row = blockIdx.x / nb, b = blockIdx.x - row * nb;
    const int64_t kk = (int64_t)b * 128 + tid;
#pragma unroll
    for (int i = 0; i < 4; ++i) tab[tid + 128 * i] = table[tid + 128 * i];

    double x = (double)w[(int64_t)row * k + kk];
    if ((sign_bits[kk >> 3] >> (kk & 7)) & 1) x = -x;
    v[tid] = x;
    __syncthreads();
    for (int h = 1; h < 128; h <<= 1) {
        const int j = (tid / h) * 2 * h + (tid % h);
        double a = 0.0, c = 0.0;
        if (tid < 64) { a = v[j]; c = v[j + h]; }
        __syncthreads();
        if (tid < 64) { v[j] = a + c; v[j + h] = a - c; }
        __syncthreads();
    }
    v[tid] = v[tid] * 0x1.6a09e667f3bcdp-4;
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0;
        for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
        const double rms = sqrt(acc / 128.0);
        const double sc = 0.29 * rms;
        const double val = 65504.0 < sc ? 65504.0 : sc;
        sbits = enc_half_rne(val);
        scales[(int64_t)row * nb + b] = (uint16_t)sbits;
    }
    __syncthreads();
    const double s = enc_half_to_double((uint16_t)sbits);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (int64_t)row * (k >> 2) + 32 * b);
    if (s == 0.0) {                                  // a zero scale codes every group as byte 0
        if (tid < 8) dst[tid] = 0u;
        return;
    }
    const int nbr = r23 ? 4 : 2, um = nbr - 1;
    const int8_t* T = reinterpret_cast<const int8_t*>(tab);
    for (int h = 0; h < 2; ++h) {
        const int t = (tid >> 3) + 16 * h, p = tid & 7;
        const double w0 = v[4 * t], w1 = v[4 * t + 1], w2 = v[4 * t + 2], w3 = v[4 * t + 3];
        double best[4] = {__builtin_inf(), __builtin_inf(), __builtin_inf(), __builtin_inf()};
        int arg[4] = {0, 0, 0, 0};
        for (int c = 0; c < 256; ++c) {
            const int8_t* L = T + (p * 256 + c) * 4;
            const double d0 = w0 - s * (double)L[0], d1 = w1 - s * (double)L[1];
            const double d2 = w2 - s * (double)L[2], d3 = w3 - s * (double)L[3];
            const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
            const int u = c & um;
            if (m < best[u]) { best[u] = m; arg[u] = c; }
        }
        for (int u = 0; u < nbr; ++u) {
            bd[t][p][u] = best[u];
            bc[t][p][u] = (uint8_t)arg[u];
        }
    }
    if (tid < 8) metric[tid] = tid == 0 ? 0.0 : __builtin_inf();
    __syncthreads();
    for (int t = 0; t < 32; ++t) {
        double nxt = __builtin_inf();
        if (tid < 8) {
            const int sn = tid;
            int pv = 0, by = 0;
            for (int p = 0; p < 8; ++p) {
                // the branch from p into sn, if there is one
                int u;
                if (r23) {
                    if ((p & 1) != (sn >> 2)) continue;
                    u = sn & 3;
                } else {
                    if ((p & 3) != (sn >> 1)) continue;
                    u = sn & 1;
                }
                const double tot = metric[p] + bd[t][p][u];
                if (tot < nxt) { nxt = tot; pv = p; by = bc[t][p][u]; }
            }
            prv[t][sn] = (int8_t)pv;
            byt[t][sn] = (uint8_t)by;
        }
        __syncthreads();
        if (tid < 8) metric[tid] = nxt;
        __syncthreads();
    }
    if (tid == 0) {
        int st = 0;
        for (int q = 1; q < 8; ++q)
            if (metric[q] < metric[st]) st = q;
        uint8_t out[32];
        for (int t = 31; t >= 0; --t) {
            out[t] = byt[t][st];
            st = prv[t][st];
        }
        for (int i = 0; i < 8; ++i)
            dst[i] = (uint32_t)out[4 * i] | ((uint32_t)out[4 * i + 1] << 8) | ((uint32_t)out[4 * i + 2] << 16) |
                     ((uint32_t)out[4 * i + 3] << 24);
    }
}

// Carried-state variant: one workgroup per row walks its blocks in order,
// each block rotated, scaled and scored as above, the path metrics carried
// from block to block; the survivors of all 32 nb steps stay in LDS (2 bytes
// per step and state) for one traceback at the end of the row.  In a
// zero-scale block the only branch is byte 0 (u = 0) at no cost.
__global__ __launch_bounds__(128) void k_encode_carry(const float* __restrict__ w, int n, int k,
                                                      const uint8_t* __restrict__ sign_bits,
                                                      uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    __shared__ double v[128];
    __shared__ double bm[32][4];
    __shared__ int barg[32][4];
    __shared__ double metric[8];
    __shared__ uint32_t sbits;
    const int tid = threadIdx.x;
    const int nb = k >> 7, row = blockIdx.x;
    int8_t* prv = reinterpret_cast<int8_t*>(lds_dyn);              // [32 nb][8]
    uint8_t* byt = lds_dyn + (size_t)32 * nb * 8;                   // [32 nb][8]
    if (tid < 8) metric[tid] = tid == 0 ? 0.0 : __builtin_inf();
    for (int b = 0; b < nb; ++b) {
        const int64_t kk = (int64_t)b * 128 + tid;
        double x = (double)w[(int64_t)row * k + kk];
        if ((sign_bits[kk >> 3] >> (kk & 7)) & 1) x = -x;
        v[tid] = x;
        __syncthreads();
        for (int h = 1; h < 128; h <<= 1) {
            const int j = (tid / h) * 2 * h + (tid % h);
            double a = 0.0, c = 0.0;
            if (tid < 64) { a = v[j]; c = v[j + h]; }
            __syncthreads();
            if (tid < 64) { v[j] = a + c; v[j + h] = a - c; }
            __syncthreads();
        }
        v[tid] = v[tid] * 0x1.6a09e667f3bcdp-4;
        __syncthreads();
        if (tid == 0) {
            double acc = 0.0;
            for (int i = 0; i < 128; ++i) acc = acc + v[i] * v[i];
            const double rms = sqrt(acc / 128.0);
            const double sc = 0.29 * rms;
            const double val = 65504.0 < sc ? 65504.0 : sc;
            sbits = enc_half_rne(val);
            scales[(int64_t)row * nb + b] = (uint16_t)sbits;
        }
        __syncthreads();
        const double s = enc_half_to_double((uint16_t)sbits);
        {
            const int t = tid >> 2, cs = tid & 3, z0 = cs >> 1, z1 = cs & 1;
            const double w0 = v[4 * t], w1 = v[4 * t + 1], w2 = v[4 * t + 2], w3 = v[4 * t + 3];
            double best = __builtin_inf();
            int arg = 0;
            for (int i = 0; i < 128; ++i) {
                const int b0 = i & 1, b1 = (i >> 1) & 1, b2 = (i >> 2) & 1, b3 = z1 ^ b0 ^ b1 ^ b2;
                const double p0 = (double)(4 * (2 * ((i >> 3) & 1) + b0) + 2 * z0 - 7);
                const double p1 = (double)(4 * (2 * ((i >> 4) & 1) + b1) + 2 * z0 - 7);
                const double p2 = (double)(4 * (2 * ((i >> 5) & 1) + b2) + 2 * z0 - 7);
                const double p3 = (double)(4 * (2 * ((i >> 6) & 1) + b3) + 2 * z0 - 7);
                const double d0 = w0 - s * p0, d1 = w1 - s * p1, d2 = w2 - s * p2, d3 = w3 - s * p3;
                const double m = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
                if (m < best) { best = m; arg = i; }
            }
            bm[t][cs] = best;
            barg[t][cs] = arg;
        }
        __syncthreads();
        for (int t = 0; t < 32; ++t) {
            double nxt = __builtin_inf();
            if (tid < 8) {
                const int sn = tid, u = sn & 1;
                int pv = 0, by = 0;
                for (int c = 0; c < 2; ++c) {
                    const int ps = c == 0 ? sn >> 1 : (sn >> 1) | 4;
                    double tot;
                    int byte;
                    if (s == 0.0) {
                        if (u != 0) continue;
                        tot = metric[ps] + 0.0;
                        byte = 0;
                    } else {
                        const int z0 = (ps >> 1) & 1, z1 = u ^ (ps & 1) ^ ((ps >> 2) & 1);
                        tot = metric[ps] + bm[t][2 * z0 + z1];
                        byte = (barg[t][2 * z0 + z1] << 1) | u;
                    }
                    if (tot < nxt) { nxt = tot; pv = ps; by = byte; }
                }
                prv[(32 * b + t) * 8 + sn] = (int8_t)pv;
                byt[(32 * b + t) * 8 + sn] = (uint8_t)by;
            }
            __syncthreads();
            if (tid < 8) metric[tid] = nxt;
            __syncthreads();
        }
    }
    if (tid == 0) {
        int st = 0;
        for (int q = 1; q < 8; ++q)
            if (metric[q] < metric[st]) st = q;
        uint8_t* dst = codes + (int64_t)row * (k >> 2);
        for (int i = 32 * nb - 1; i >= 0; --i) {
            dst[i] = byt[i * 8 + st];
            st = prv[i * 8 + st];
        }
    }
}

}  // namespace

int launch_encode_carry(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
                        uint16_t* scales, pg_stream_t s) {
    const size_t lds = (size_t)(k / 128) * 32 * 16;        // survivors: 2 bytes per step and state
    hipLaunchKernelGGL(k_encode_carry, dim3((unsigned)n), dim3(128), lds, (hipStream_t)s, w, (int)n, (int)k, sign_bits,
                       codes, scales);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_encode_ex launch: %s", hipGetErrorString(e));
    return PG_OK;
}

int launch_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* fb,
                       double* err, uint8_t* codes, uint16_t* scales, pg_stream_t s) {
    if (n > 0x7fffffff) return fail(PG_ERR_UNSUPPORTED, "pg_encode_ldlq: too many rows");
    for (int64_t b = 0; b < k / 128; ++b) {
        hipLaunchKernelGGL(k_encode_ldlq, dim3((unsigned)n), dim3(128), 0, (hipStream_t)s, w, (int)n, (int)k,
                           sign_bits, fb, err, codes, scales, (int)b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_encode_ldlq launch: %s", hipGetErrorString(e));
    }
    return PG_OK;
}

// pg_encode_ldlq: sign bits to the host, the feedback matrix factored there
// (ldlq_feedback, shared with pg_encode_ref_ldlq), copied up with an error
// buffer, one launch per block, then everything freed; returns when done.
int run_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                    uint8_t* codes, uint16_t* scales, pg_stream_t s) {
    hipStream_t st = (hipStream_t)s;
    std::vector<uint8_t> sb((size_t)(k / 8));
    hipError_t e = hipMemcpyAsync(sb.data(), sign_bits, sb.size(), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_encode_ldlq: reading sign_bits: %s", hipGetErrorString(e));
    std::vector<double> fb((size_t)(k * k));
    int rc = ldlq_feedback(hessian, k, sb.data(), 0, fb.data());
    if (rc != PG_OK) return rc;
    double* fb_d = nullptr;
    double* err_d = nullptr;
    e = hipMalloc((void**)&fb_d, sizeof(double) * (size_t)(k * k));
    if (e == hipSuccess) e = hipMalloc((void**)&err_d, sizeof(double) * (size_t)(n * k));
    if (e == hipSuccess) e = hipMemcpyAsync(fb_d, fb.data(), sizeof(double) * fb.size(), hipMemcpyHostToDevice, st);
    if (e != hipSuccess) {
        rc = fail(PG_ERR_HIP, "pg_encode_ldlq: %s", hipGetErrorString(e));
    } else {
        rc = launch_encode_ldlq(w, n, k, sign_bits, fb_d, err_d, codes, scales, s);
        e = hipStreamSynchronize(st);
        if (rc == PG_OK && e != hipSuccess) rc = fail(PG_ERR_HIP, "pg_encode_ldlq: %s", hipGetErrorString(e));
    }
    if (fb_d) (void)hipFree(fb_d);
    if (err_d) (void)hipFree(err_d);
    return rc;
}

int launch_encode_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                        bool r23, uint8_t* codes, uint16_t* scales, pg_stream_t s) {
    const int64_t blocks = n * (k / 128);
    if (blocks > 0x7fffffff) return fail(PG_ERR_UNSUPPORTED, "pg_encode_table: too many blocks (%lld)", (long long)blocks);
    hipLaunchKernelGGL(k_encode_table, dim3((unsigned)blocks), dim3(128), 0, (hipStream_t)s, w, (int)n, (int)k,
                       sign_bits, reinterpret_cast<const uint4*>(table), r23 ? 1 : 0, codes, scales);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_encode_table launch: %s", hipGetErrorString(e));
    return PG_OK;
}

int launch_encode(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
                  uint16_t* scales, pg_stream_t s) {
    const int64_t blocks = n * (k / 128);
    if (blocks > 0x7fffffff) return fail(PG_ERR_UNSUPPORTED, "pg_encode: too many blocks (%lld)", (long long)blocks);
    hipLaunchKernelGGL(k_encode, dim3((unsigned)blocks), dim3(128), 0, (hipStream_t)s, w, (int)n, (int)k, sign_bits,
                       codes, scales);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_encode launch: %s", hipGetErrorString(e));
    return PG_OK;
}

}  // namespace pg
