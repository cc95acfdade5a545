// Batch-1 fused stage of a stack for gfx950 (MI355X, wave64):
// y = W~ . R . n(x) in one launch, with the activation rotation computed in
// registers (butterflies inside the lane and across lanes) instead of
// staging fp16 blocks in LDS for the matrix cores.  Two decodes share it:
// P8F v1's closed-form bit planes, and the table-driven codebook (the 8 x 256
// points of four int8 levels staged in LDS, one lookup per group).
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode
// and random Hadamard rotation); the table variant is the codebook half of
// the small-state coset trellis of section "Paper".  Bit layout:
// include/pingala.h.
#pragma once
#include "pg_fused.h"

namespace pg {

// Launch shape of the batch-1 stage: W waves; R rows per workgroup with
// all k columns; column groups CG = ceil(k / 512) of 8 chunks; RP = 8W / CG
// row phases; RS rows per lane; U rounds of the rotation (four 128-blocks
// per wave and round).
struct Fused1Shape {
    int W, R, CG, RP, RS, U;
};

// R, CG, RP and U in one argument dword (11, 7, 7 and 7 bits; fused1_shape
// keeps them in range).  With the arguments in 14 dwords, the hardware
// preloads all of them into scalar registers (the build asks for preloading;
// the argument-segment pointer takes 2 of the 16 user registers), so no wave
// waits for a scalar load of its arguments before its first requests.
__host__ inline uint32_t fused1_shape_word(const Fused1Shape& S) {
    return (uint32_t)S.R | ((uint32_t)S.CG << 11) | ((uint32_t)S.RP << 18) | ((uint32_t)S.U << 25);
}

// PG_ERR_UNSUPPORTED (message set) when the shape does not fit the kernel
// with at most umax rotation rounds (and the codebook table in LDS if asked)
int fused1_shape(int64_t n, int64_t k, int umax, bool table, Fused1Shape* out);

// the rate-2/3 table instances (pg_fused1_r23.hip, compiled on their own)
int launch_table_r23(const Fused1Shape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                     const void* x, int x_dt, const uint8_t* sign_bits, const uint32_t* table, uint32_t flags,
                     float* y, hipStream_t st);

namespace {

constexpr int F1_UMAX = 1;       // rotation rounds per wave of the closed-form stage: k <= 4096 with 8 waves
constexpr int F1T_UMAX = 4;      // and of the table stage: k <= 16384
constexpr int F1T_TABLE_BYTES = 8 * 256 * 4;

// LDS of one launch: [the codebook table,] the digits row of the rotated
// activations (per 32-value quarter its scale and its sum of q after the
// digits), the team sums and the per-wave sums of squares
__host__ inline size_t fused1_lds_bytes(int k, const Fused1Shape& S, bool table) {
    return (table ? (size_t)F1T_TABLE_BYTES : 0) + (size_t)fused_row_bytes(k) + (size_t)S.R * S.CG * 4 +
           (size_t)S.W * 4;
}

// 4 x 4 byte transpose across the lanes of a quad: lane j holds byte g of row
// j on entry and byte j of row g on return (two DPP exchanges, two permutes)
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t o, int lane) {
    uint32_t p = (uint32_t)xor_lane_i<1>((int)o, lane);
    o = __builtin_amdgcn_perm(p, o, (lane & 1) ? 0x03070105u : 0x06020400u);
    p = (uint32_t)xor_lane_i<2>((int)o, lane);
    return __builtin_amdgcn_perm(p, o, (lane & 2) ? 0x03020706u : 0x05040100u);
}

// The rotation's lane roles.  Four 128-blocks per wave and round: lane
// l = j + 4 bb + 16 mh works on block bb of the round and holds the eight
// positions 16 (m0 + 2 mh) + 4 g + j (m0 in 0..1, g in 0..3) of it, value
// index 4 m0 + g.  Position bits 2, 3 (g) and 4 (m0) are inside the lane,
// bits 0, 1 (j) cross lanes l ^ 1, l ^ 2 (DPP quad permutes), bits 5, 6 (mh)
// cross lanes l ^ 16, l ^ 32 (gfx950 permlane swaps), so a block's 16 lanes
// exchange only among themselves.  A lane's four values of one m0 are the
// four groups g of one digit dword (plane j of code dword m = m0 + 2 mh of
// the block): its digits leave in two dword stores.  The 32 values of a
// quarter (mh fixed) sit in one quad, whose maximum and sum of q take two
// DPP steps.
//
// TAB = 1, the table-driven codebook (TAB = 2: the same on the rate-2/3
// trellis, whose state is the previous byte's two branch bits and bit 0 of
// the byte before): the digits are balanced (q = 256 hi +
// lo with both signed bytes, hi = (q + 128) >> 8) and stored group-major
// (one dword holds the four weights of one group, as a table point does),
// after a 4 x 4 byte transpose across the quad.  A group read in state s as
// byte c takes the point T[s][c] from the LDS copy of the table; its dot
// products with the digits are two v_dot4_i32_i8.  The state of each byte of
// a code dword comes from the branch bits of the three bytes before it
// (funnel shifts of the dword and its predecessor); flags PG_FLAG_CARRY_STATE
// continues the state from the previous 64-value chunk of the row, whose
// last code dword every lane loads itself.
//
// Arguments: the first 14 dwords arrive preloaded in scalar registers (see
// fused1_shape_word), so the requests need no scalar load; only the table
// pointer, used by TAB > 0 alone, comes after them.
template <int XDT, int RS, int TAB, int UMAX>
__global__ __launch_bounds__(512) void k_rot_qgemv1(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     const void* __restrict__ x,
                                                     const uint8_t* __restrict__ sign_bits,
                                                     float* __restrict__ y, int n, int k, uint32_t flags,
                                                     uint32_t shape, const uint32_t* __restrict__ table) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_all[];
    const int R = (int)(shape & 0x7ffu), CG = (int)((shape >> 11) & 0x7fu), RP = (int)((shape >> 18) & 0x7fu),
              U = (int)(shape >> 25);
    uint8_t* lds = lds_all + (TAB ? F1T_TABLE_BYTES : 0);                    // the table, if any, sits first
    constexpr int W = 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int T = wave * 8 + (lane >> 3), tl = lane & 7;
    const int kg = k >> 2, nchunk = k >> 6, nbk = k >> 7;
    const int row0 = blockIdx.x * R;
    uint8_t* dig = lds;                                                       // [nchunk][FS_PITCH] digits
    float* sxq = reinterpret_cast<float*>(dig + nchunk * FS_PITCH);           // [k/32] quarter scales
    int* sqq = reinterpret_cast<int*>(dig + nchunk * FS_PITCH + (k / 32) * 4);   // [k/32] quarter sums of q
    float* part = reinterpret_cast<float*>(dig + fused_row_bytes(k));          // [R][CG] team sums
    float* wsum = part + R * CG;                                               // [W] sums of squares
    const bool norm = (flags & PG_FLAG_RMSNORM) != 0;
    const bool carry = TAB && (flags & PG_FLAG_CARRY_STATE) != 0;
    float rk = 1.0f / (float)k;
    asm volatile("" : "+v"(rk));                      // computed here, before any wait (the
                                                      // compiler would sink it past the barrier)

    // ---- 1. requests: the lane's x values and sign words of every round,
    // then its code chunks and scales (memory operations of a wave complete
    // in order, so waiting until only the code requests are outstanding
    // means x has arrived)
    const int rj = lane & 3, rbb = (lane >> 2) & 3, rmh = lane >> 4;
    uint32_t xr[UMAX][8];
    uint32_t sw[UMAX];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
        if (u < U && 4 * (wave + W * u) < nbk) {               // uniform: a round with blocks for this wave
            const int blk = 4 * (wave + W * u) + rbb;
            const int bc = blk < nbk ? blk : nbk - 1;          // clamped: every lane issues the same loads
            const int p0 = bc * 128 + 32 * rmh + rj;             // position of (m0, g) = (0, 0)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = p0 + 16 * (i >> 2) + 4 * (i & 3);
                xr[u][i] = XDT == PG_F32 ? reinterpret_cast<const uint32_t*>(x)[p]
                                         : (uint32_t)reinterpret_cast<const uint16_t*>(x)[p];
            }
            sw[u] = reinterpret_cast<const uint32_t*>(sign_bits)[bc * 4 + rmh];
        }
    }
    // this lane's column of chunks and its rows in the dot products
    const int cg = T % CG, rp = T / CG;
    const int c = 8 * cg + tl;
    const bool col_ok = rp < RP && c < nchunk;
    const int cc = c < nchunk ? c : nchunk - 1;
    int rowj[RS];
    bool rok[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
        const int r = rp + j * RP;
        rok[j] = col_ok && r < R && row0 + r < n;
        rowj[j] = rok[j] ? row0 + r : (row0 < n ? row0 : n - 1);
    }
    // the table (16 bytes per thread) and, for carried state, the code dword
    // before each of the lane's chunks: requested before the codes, so the
    // wait below covers them
    uint4 tv = {0u, 0u, 0u, 0u};
    uint32_t pq[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) pq[j] = 0u;
    if constexpr (TAB) {
        tv = reinterpret_cast<const uint4*>(table)[tid];
        if (carry && cc > 0) {
#pragma unroll
            for (int j = 0; j < RS; ++j)
                pq[j] = *reinterpret_cast<const uint32_t*>(codes + (int64_t)rowj[j] * kg + 16 * cc - 4);
        }
    }
    asm volatile("" ::: "memory");
    uint4 q[RS];
    uint32_t wsr[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
        const int row = rowj[j];
        q[j] = *reinterpret_cast<const uint4*>(codes + (int64_t)row * kg + 16 * cc);
        wsr[j] = scales[(int64_t)row * nbk + (cc >> 1)];
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * RS));      // x, sign words (and table, carried dwords) have arrived
    if constexpr (TAB) reinterpret_cast<uint4*>(lds_all)[tid] = tv;   // read after the barriers below

    // ---- 2. the RMS factor: sum of squares over the lane's valid blocks,
    // wave sums, the waves' sums added in wave order by every thread
    float inv = 1.0f;
    if (norm) {
        float ss = 0.0f;
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
            if (u < U && 4 * (wave + W * u) + rbb < nbk) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float f = XDT == PG_F32 ? __builtin_bit_cast(float, xr[u][i]) : h2f((uint16_t)xr[u][i]);
                    ss += f * f;
                }
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) wsum[wave] = ss;
        lds_barrier();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += wsum[w];
        inv = rms_inv(tot, rk);
    }

    // ---- 3. rotation rounds: n(x) rounded to fp16 and sign-flipped, the
    // butterflies, quantisation per 32 values, digits to LDS
    const float sg1 = (lane & 1) ? -1.0f : 1.0f, sg2 = (lane & 2) ? -1.0f : 1.0f;
    const float sg16 = (lane & 16) ? -1.0f : 1.0f, sg32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
        if (u >= U || 4 * (wave + W * u) >= nbk) break;   // wave-uniform: no block left for this wave
        const int blk = 4 * (wave + W * u) + rbb;
        const bool ok = blk < nbk;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float f = XDT == PG_F32 ? __builtin_bit_cast(float, xr[u][i]) : h2f((uint16_t)xr[u][i]);
            uint32_t h = f2h(norm ? f * inv : f);
            h ^= ((sw[u] >> (16 * (i >> 2) + 4 * (i & 3) + rj)) & 1u) << 15;
            v[i] = h2f((uint16_t)h);
        }
        // position bits 2, 3 (g) and 4 (m0): value index bits 0, 1, 2
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (!(i & h)) {
                    const float a = v[i], b = v[i | h];
                    v[i] = a + b;
                    v[i | h] = a - b;
                }
        // position bits 0, 1 (j) and 5, 6 (mh): across lanes; the lane with the
        // bit set takes partner - own, the other own + partner
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(sg1, v[i], xor_lane<1>(v[i], lane));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(sg2, v[i], xor_lane<2>(v[i], lane));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(sg16, v[i], xor_lane16(v[i], lane));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(sg32, v[i], xor_lane32(v[i], lane));
        // quarter mh of the block: its maximum over the quad, q = rint(v * 32512 / max)
        // as the low 16 bits of fma(v, s, 1.5 * 2^23) (of q + 128 with 128
        // added to the constant, for the balanced digits: rounding to an
        // integer commutes with adding an even integer)
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
        mx = fmaxf(mx, xor_lane<1>(mx, lane));
        mx = fmaxf(mx, xor_lane<2>(mx, lane));
        const float s = mx > 0.0f ? (float)Q16_MAXQ * __builtin_amdgcn_rcpf(mx) : 0.0f;   // hardware reciprocal
        uint32_t bits[8];
        int qs = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bits[i] = __builtin_bit_cast(uint32_t, fmaf(v[i], s, TAB ? 12583040.0f : 12582912.0f));
            if constexpr (!TAB) qs += (int)(int16_t)(bits[i] & 0xffffu);
        }
        if constexpr (!TAB) {
            qs += xor_lane_i<1>(qs, lane);
            qs += xor_lane_i<2>(qs, lane);
        }
        if (ok) {
            // chunk 2 blk + mh / 2; code dword m0 + 2 (mh % 2) of it; plane j
            uint8_t* d = dig + (2 * blk + (rmh >> 1)) * FS_PITCH + 64 * (rmh & 1) + 4 * rj;
#pragma unroll
            for (int m0 = 0; m0 < 2; ++m0) {
                const uint32_t t01 = __builtin_amdgcn_perm(bits[4 * m0 + 1], bits[4 * m0], 0x05040100u);
                const uint32_t t23 = __builtin_amdgcn_perm(bits[4 * m0 + 3], bits[4 * m0 + 2], 0x05040100u);
                uint32_t dh = __builtin_amdgcn_perm(t23, t01, 0x07050301u);   // floor(q / 256); balanced: (q + 128) >> 8
                uint32_t dl = __builtin_amdgcn_perm(t23, t01, 0x06040200u);   // q mod 256; balanced: its signed byte
                if constexpr (TAB) {
                    dl ^= 0x80808080u;
                    dh = quad_transpose_bytes(dh, lane);
                    dl = quad_transpose_bytes(dl, lane);
                }
                *reinterpret_cast<uint32_t*>(d + 32 * m0) = dh;
                *reinterpret_cast<uint32_t*>(d + 32 * m0 + 16) = dl;
            }
            if (rj == 0) {
                sxq[4 * blk + rmh] = mx * (0.08838834764831845f / (float)Q16_MAXQ);   // 2^-3.5 max / 32512
                if constexpr (!TAB) sqq[4 * blk + rmh] = qs;
            }
        }
    }
    lds_barrier();

    // ---- 4. decode and dot products (as k_rot_qgemv at batch 1)
    {
        uint4 qb[RS];
        uint32_t wb[RS];
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            qb[j] = q[j];
            wb[j] = wsr[j];
            asm volatile("" : "+v"(qb[j].x), "+v"(qb[j].y), "+v"(qb[j].z), "+v"(qb[j].w), "+v"(wb[j]));
        }
        const uint32_t left_mask = (c & 1) ? ~0u : 0u;   // odd chunks continue the left lane's block
        const float sx0 = sxq[2 * cc], sx1 = sxq[2 * cc + 1];
        float tq[RS];
        int hi[RS], lo[RS];
        if constexpr (TAB) {
            const uint32_t* tab = reinterpret_cast<const uint32_t*>(lds_all);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m == 0 || m == 2)
#pragma unroll
                    for (int j = 0; j < RS; ++j) { hi[j] = 0; lo[j] = 0; }
                const uint8_t* dg = dig + cc * FS_PITCH + 32 * m;
                const uint4 xh4 = *reinterpret_cast<const uint4*>(dg);
                const uint4 xl4 = *reinterpret_cast<const uint4*>(dg + 16);
                const uint32_t xh[4] = {xh4.x, xh4.y, xh4.z, xh4.w}, xl[4] = {xl4.x, xl4.y, xl4.z, xl4.w};
#pragma unroll
                for (int j = 0; j < RS; ++j) {
                    const uint32_t w4[4] = {qb[j].x, qb[j].y, qb[j].z, qb[j].w};
                    uint32_t prev;
                    if (m > 0)
                        prev = w4[m - 1];
                    else if (carry)
                        prev = pq[j];
                    else
                        prev = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb[j].w, 0x111, 0xf, 0xf, true) & left_mask;
                    const uint32_t w = w4[m];
                    uint32_t st;
                    if constexpr (TAB == 1) {
                        // state of byte b: branch bits of bytes b-1, b-2, b-3 at its bits 0, 1, 2;
                        // with only the branch bits kept, the three shifted copies
                        // land on disjoint bits and need no masks
                        const uint32_t uw = w & 0x01010101u, up = prev & 0x01010101u;
                        st = __builtin_amdgcn_alignbit(uw, up, 24) | __builtin_amdgcn_alignbit(uw, up, 15) |
                             __builtin_amdgcn_alignbit(uw, up, 6);
                    } else {
                        // rate 2/3: byte b-1's two branch bits at bits 0, 1, bit 0 of byte b-2 at bit 2
                        const uint32_t w2 = w & 0x03030303u, p2 = prev & 0x03030303u;
                        const uint32_t w1 = w & 0x01010101u, p1 = prev & 0x01010101u;
                        st = __builtin_amdgcn_alignbit(w2, p2, 24) | __builtin_amdgcn_alignbit(w1, p1, 14);
                    }
                    int h = hi[j], l = lo[j];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        // table index s * 256 + byte: the byte, then its state, as bytes 0 and 1
                        const uint32_t idx = __builtin_amdgcn_perm(st, w, 0x0c0c0400u + 0x0101u * g);
                        const uint32_t pt = tab[idx];
                        h = __builtin_amdgcn_sdot4((int)pt, (int)xh[g], h, false);
                        l = __builtin_amdgcn_sdot4((int)pt, (int)xl[g], l, false);
                    }
                    hi[j] = h;
                    lo[j] = l;
                }
                // quarter done: sum level * q = 256 hi + lo
                if (m == 1)
#pragma unroll
                    for (int j = 0; j < RS; ++j) tq[j] = sx0 * (float)(hi[j] * 256 + lo[j]);
                if (m == 3)
#pragma unroll
                    for (int j = 0; j < RS; ++j) tq[j] += sx1 * (float)(hi[j] * 256 + lo[j]);
            }
        } else {
        const int sq0 = sqq[2 * cc], sq1 = sqq[2 * cc + 1];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m == 0 || m == 2)
#pragma unroll
                for (int j = 0; j < RS; ++j) { hi[j] = 0; lo[j] = 0; }
            const uint8_t* dg = dig + cc * FS_PITCH + 32 * m;
            const uint4 xh4 = *reinterpret_cast<const uint4*>(dg);
            const uint4 xl4 = *reinterpret_cast<const uint4*>(dg + 16);
#pragma unroll
            for (int j = 0; j < RS; ++j) {
                const uint32_t w4[4] = {qb[j].x, qb[j].y, qb[j].z, qb[j].w};
                const uint32_t prev =
                    m == 0 ? ((uint32_t)__builtin_amdgcn_mov_dpp((int)qb[j].w, 0x111, 0xf, 0xf, true) & left_mask)
                           : w4[m - 1];
                uint32_t P[4];
                planes_of(w4[m], prev, P);
                int h = hi[j];
                uint32_t l = (uint32_t)lo[j];
                h = __builtin_amdgcn_sdot4((int)P[0], (int)xh4.x, h, false);
                l = __builtin_amdgcn_udot4(P[0], xl4.x, l, false);
                h = __builtin_amdgcn_sdot4((int)P[1], (int)xh4.y, h, false);
                l = __builtin_amdgcn_udot4(P[1], xl4.y, l, false);
                h = __builtin_amdgcn_sdot4((int)P[2], (int)xh4.z, h, false);
                l = __builtin_amdgcn_udot4(P[2], xl4.z, l, false);
                h = __builtin_amdgcn_sdot4((int)P[3], (int)xh4.w, h, false);
                l = __builtin_amdgcn_udot4(P[3], xl4.w, l, false);
                hi[j] = h;
                lo[j] = (int)l;
            }
            // quarter done: sum level * q = 2 (256 hi + lo) - 7 sum q
            if (m == 1)
#pragma unroll
                for (int j = 0; j < RS; ++j) tq[j] = sx0 * (float)(2 * (hi[j] * 256 + lo[j]) - 7 * sq0);
            if (m == 3)
#pragma unroll
                for (int j = 0; j < RS; ++j) tq[j] += sx1 * (float)(2 * (hi[j] * 256 + lo[j]) - 7 * sq1);
        }
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            float v = rok[j] ? h2f((uint16_t)wb[j]) * tq[j] : 0.0f;
            v += xor_lane<4>(v, lane);
            v += xor_lane<2>(v, lane);
            v += xor_lane<1>(v, lane);
            if (tl == 0 && rp < RP && rp + j * RP < R) part[(rp + j * RP) * CG + cg] = v;
        }
    }
    __syncthreads();
    // ---- 5. team sums added in column-group order
    for (int r = tid; r < R; r += 64 * W) {
        if (row0 + r >= n) continue;
        const float* pr = part + r * CG;
        float v = 0.0f;
        for (int g = 0; g < CG; ++g) v += pr[g];
        y[row0 + r] = v;
    }
}

template <int XDT, int RS, int TAB, int UMAX>
int launch_fused1_t(const Fused1Shape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                    const void* x, const uint8_t* sign_bits, const uint32_t* table, uint32_t flags, float* y,
                    hipStream_t st) {
    const dim3 grid((unsigned)((n + S.R - 1) / S.R));
    hipLaunchKernelGGL((k_rot_qgemv1<XDT, RS, TAB, UMAX>), grid, dim3(64 * S.W), fused1_lds_bytes((int)k, S, TAB != 0),
                       st, codes, scales, x, sign_bits, y, (int)n, (int)k, flags, fused1_shape_word(S), table);
    return hip_check(hipGetLastError(), TAB ? "pg_rot_qgemv_table launch" : "pg_rot_qgemv launch");
}

// rows per lane as exact as possible: every row slot costs a full decode
template <int XDT, int TAB, int UMAX>
int launch_fused1_rs(const Fused1Shape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                     const void* x, const uint8_t* sign_bits, const uint32_t* table, uint32_t flags, float* y,
                     hipStream_t st) {
#define PG_F1(RS_) \
    return launch_fused1_t<XDT, RS_, TAB, UMAX>(S, codes, scales, n, k, x, sign_bits, table, flags, y, st)
    if (S.RS <= 1) PG_F1(1);
    if (S.RS <= 2) PG_F1(2);
    if (S.RS <= 3) PG_F1(3);
    if (S.RS <= 4) PG_F1(4);
    if (S.RS <= 5) PG_F1(5);
    if (S.RS <= 6) PG_F1(6);
    if (S.RS <= 7) PG_F1(7);
    if (S.RS <= 8) PG_F1(8);
    if (S.RS <= 10) PG_F1(10);
    if (S.RS <= 12) PG_F1(12);
    if (S.RS <= 14) PG_F1(14);
    PG_F1(16);
#undef PG_F1
}

}  // namespace
}  // namespace pg
