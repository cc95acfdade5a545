/* Plain-C twin of the oracle's Viterbi encoder (format P8F v1).
 *
 * TEST INFRASTRUCTURE ONLY: built as oracle/liboracle_p8f.so and called from
 * oracle/p8f.py to encode large synthetic matrices in reasonable time.  It is
 * the same brute-force search as p8f.viterbi_encode, evaluated in the same
 * floating-point order, and the tests require the two to agree bit for bit.
 * Nothing in the product library links or calls it.
 *
 * Source: "Pingala-8" landing page, section "How it works" (an 8-state
 * Ungerboeck trellis over groups of 4 weights; the carried state picks the
 * value set of the next group).  The bit layout is format P8F v1:
 *   state s = last 3 branch bits, s' = ((s << 1) | u) & 7, u = byte bit 0;
 *   z0 = (s >> 1) & 1, z1 = u ^ (s & 1) ^ ((s >> 2) & 1);
 *   b0..b2 = byte bits 1..3, b3 = z1 ^ b0 ^ b1 ^ b2, e_j = byte bit 4+j;
 *   level_j = 4 * (2 e_j + b_j) + 2 z0 - 7.
 * Build with -ffp-contract=off so that no multiply-add is fused. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* subnormal or zero */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), exp - 25);
    return sign ? -v : v;
}

/* levels of `byte` read with value set z0 and parity coset z1 */
static void levels_of(int byte, int z0, int z1, double out[4]) {
    int b[4];
    b[0] = (byte >> 1) & 1;
    b[1] = (byte >> 2) & 1;
    b[2] = (byte >> 3) & 1;
    b[3] = z1 ^ b[0] ^ b[1] ^ b[2];
    for (int j = 0; j < 4; ++j) {
        int e = (byte >> (4 + j)) & 1;
        out[j] = (double)(4 * (2 * e + b[j]) + 2 * z0 - 7);
    }
}

/* w_rot [nb][4*G] fp64, scale_bits [nb] fp16 bits, codes [nb][G] out.
 * Start state 0, free end state; ties: predecessor s'>>1 over (s'>>1)|4,
 * smaller byte among equally near points, smaller end state; zero scale
 * gives all-zero bytes.  Returns 0, or -1 if G is out of range. */
int p8f_oracle_viterbi(const double* w_rot, const uint16_t* scale_bits, int64_t nb,
                       int G, uint8_t* codes) {
    if (G < 1 || G > 4096) return -1;
    double pts[2][2][128][4];           /* [z0][z1][point in ascending byte order] */
    for (int z0 = 0; z0 < 2; ++z0)
        for (int z1 = 0; z1 < 2; ++z1)
            for (int i = 0; i < 128; ++i)
                levels_of(i << 1, z0, z1, pts[z0][z1][i]);   /* byte bits 1..7 = i */

    /* per-block work arrays (G is small: 32 for real blocks) */
    double bm[4096][2][2];
    int barg[4096][2][2];
    int8_t bprev[4096][8];
    int16_t bbyte[4096][8];

    for (int64_t blk = 0; blk < nb; ++blk) {
        const double* w = w_rot + blk * (int64_t)4 * G;
        uint8_t* out = codes + blk * (int64_t)G;
        double s = half_to_double(scale_bits[blk]);
        for (int t = 0; t < G; ++t) {
            for (int z0 = 0; z0 < 2; ++z0)
                for (int z1 = 0; z1 < 2; ++z1) {
                    double best = INFINITY;
                    int arg = 0;
                    for (int i = 0; i < 128; ++i) {
                        const double* p = pts[z0][z1][i];
                        double d0 = w[4 * t + 0] - s * p[0];
                        double d1 = w[4 * t + 1] - s * p[1];
                        double d2 = w[4 * t + 2] - s * p[2];
                        double d3 = w[4 * t + 3] - s * p[3];
                        double q0 = d0 * d0, q1 = d1 * d1, q2 = d2 * d2, q3 = d3 * d3;
                        double m = ((q0 + q1) + q2) + q3;
                        if (m < best) { best = m; arg = i; }
                    }
                    bm[t][z0][z1] = best;
                    barg[t][z0][z1] = arg;
                }
        }
        double metric[8], next[8];
        for (int st = 0; st < 8; ++st) metric[st] = INFINITY;
        metric[0] = 0.0;
        for (int t = 0; t < G; ++t) {
            for (int sn = 0; sn < 8; ++sn) {
                int u = sn & 1;
                next[sn] = INFINITY;
                bprev[t][sn] = 0;
                bbyte[t][sn] = 0;
                int cands[2] = {sn >> 1, (sn >> 1) | 4};
                for (int c = 0; c < 2; ++c) {
                    int cs = cands[c];
                    int z0 = (cs >> 1) & 1;
                    int z1 = u ^ (cs & 1) ^ ((cs >> 2) & 1);
                    double tot = metric[cs] + bm[t][z0][z1];
                    if (tot < next[sn]) {
                        next[sn] = tot;
                        bprev[t][sn] = (int8_t)cs;
                        bbyte[t][sn] = (int16_t)((barg[t][z0][z1] << 1) | u);
                    }
                }
            }
            memcpy(metric, next, sizeof(metric));
        }
        int st = 0;
        for (int k = 1; k < 8; ++k)
            if (metric[k] < metric[st]) st = k;
        for (int t = G - 1; t >= 0; --t) {
            out[t] = (uint8_t)bbyte[t][st];
            st = bprev[t][st];
        }
        if (s == 0.0)
            for (int t = 0; t < G; ++t) out[t] = 0;
    }
    return 0;
}
