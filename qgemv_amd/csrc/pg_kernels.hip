// HIP kernels of libpingala for gfx950 (MI355X, wave64): trellis decode,
// the run-time Hadamard rotation, the batch-1..8 product (qgemv) and the
// prompt product on the matrix cores (qgemm).
//
// Method: "Pingala-8" landing page, section "How it works" -- an 8-state
// Ungerboeck trellis over groups of 4 weights, the state carried from group
// to group choosing the value set of the next group, plus a random Hadamard
// rotation.  Bit layout: format P8F v1 as stated in include/pingala.h.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "pg_internal.h"

namespace pg {
namespace {

typedef _Float16 half_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(half_t, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (half_t)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
    // round to nearest even (finite inputs; NaN kept quiet)
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_elem(const void* p, int dt, int64_t i) {
    if (dt == PG_F32) return ((const float*)p)[i];
    if (dt == PG_F16) return h2f(((const uint16_t*)p)[i]);
    return bf2f(((const uint16_t*)p)[i]);
}

__device__ __forceinline__ void store_elem(void* p, int dt, int64_t i, float v) {
    if (dt == PG_F32) ((float*)p)[i] = v;
    else if (dt == PG_F16) ((uint16_t*)p)[i] = f2h(v);
    else ((uint16_t*)p)[i] = f2bf(v);
}

// Levels of byte c read in state s (P8F v1): 4 * (2 e_j + b_j) + 2 z0 - 7.
__device__ __forceinline__ void levels_of(uint32_t s, uint32_t c, int lv[4]) {
    const uint32_t u = c & 1u;
    const int z0 = (int)((s >> 1) & 1u);
    const uint32_t z1 = u ^ (s & 1u) ^ ((s >> 2) & 1u);
    const uint32_t b0 = (c >> 1) & 1u, b1 = (c >> 2) & 1u, b2 = (c >> 3) & 1u;
    const uint32_t b3 = z1 ^ b0 ^ b1 ^ b2;
    const int base = 2 * z0 - 7;
    lv[0] = 4 * (int)(2 * ((c >> 4) & 1u) + b0) + base;
    lv[1] = 4 * (int)(2 * ((c >> 5) & 1u) + b1) + base;
    lv[2] = 4 * (int)(2 * ((c >> 6) & 1u) + b2) + base;
    lv[3] = 4 * (int)(2 * ((c >> 7) & 1u) + b3) + base;
}

// ------------------------------------------------------------------ decode
// One thread per code byte; the state comes from the bit 0 of the previous
// (at most three) bytes of the same 128-block.  w = fp32(scale) * level is
// exact, so the output is bit-identical to any exact decoder.
__global__ void k_decode(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                         int64_t total_groups, int kg, float* __restrict__ w) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total_groups) return;
    const int64_t row = g / kg;
    const int t = (int)(g - row * kg);
    const int tb = t & 31;
    const uint8_t* rp = codes + row * kg;
    const uint32_t c = rp[t];
    const uint32_t u1 = tb >= 1 ? (rp[t - 1] & 1u) : 0u;
    const uint32_t u2 = tb >= 2 ? (rp[t - 2] & 1u) : 0u;
    const uint32_t u3 = tb >= 3 ? (rp[t - 3] & 1u) : 0u;
    int lv[4];
    levels_of(u1 | (u2 << 1) | (u3 << 2), c, lv);
    const float s = h2f(scales[row * (kg / 32) + (t >> 5)]);
    float4 o;
    o.x = s * (float)lv[0];
    o.y = s * (float)lv[1];
    o.z = s * (float)lv[2];
    o.w = s * (float)lv[3];
    reinterpret_cast<float4*>(w)[g] = o;
}

// ---------------------------------------------------------------- rotation
// Grid (ceil(nblocks/4), rows): each of the 4 waves of a workgroup transforms
// one 128-block; lane l holds elements l and l+64, the first butterfly stage
// (distance 64) is inside the lane, the other six exchange across lanes.
// With PG_FLAG_RMSNORM every workgroup first sums the squares of its whole
// row (fixed order: strided per thread, then waves 0..3) and rounds the
// normalised values to fp16.  PG_Q16 output writes the 16-bit fixed-point
// activation format that pg_qgemv reads (layout in include/pingala.h).
// Value of lane (lane ^ H) for H < 16, with DPP row shifts (no LDS trip).
template <int H>
__device__ __forceinline__ float xor_lane(float v, int lane) {
    const int iv = __builtin_bit_cast(int, v);
    if (H == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    if (H == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    const int up = __builtin_amdgcn_mov_dpp(iv, 0x100 + H, 0xf, 0xf, false);   // row_shl:H -> lane + H
    const int dn = __builtin_amdgcn_mov_dpp(iv, 0x110 + H, 0xf, 0xf, false);   // row_shr:H -> lane - H
    return __builtin_bit_cast(float, (lane & H) ? dn : up);
}
template <int H>
__device__ __forceinline__ int xor_lane_i(int v, int lane) {
    return __builtin_bit_cast(int, xor_lane<H>(__builtin_bit_cast(float, v), lane));
}

// Value of lane (lane ^ 16) / (lane ^ 32): gfx950's v_permlane16_swap /
// v_permlane32_swap exchange rows of 16 / halves of 32 lanes in registers.
__device__ __forceinline__ float xor_lane16(float v, int lane) {
    const int iv = __builtin_bit_cast(int, v);
    const auto r = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
    return __builtin_bit_cast(float, (lane & 16) ? (int)r[0] : (int)r[1]);
}
__device__ __forceinline__ float xor_lane32(float v, int lane) {
    const int iv = __builtin_bit_cast(int, v);
    const auto r = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
    return __builtin_bit_cast(float, (lane & 32) ? (int)r[0] : (int)r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
    const int lane = threadIdx.x & 63;
    v += xor_lane<1>(v, lane);
    v += xor_lane<2>(v, lane);
    v += xor_lane<4>(v, lane);
    v += xor_lane<8>(v, lane);
    v += xor_lane16(v, lane);
    v += xor_lane32(v, lane);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
    const int lane = threadIdx.x & 63;
    v += xor_lane_i<1>(v, lane);
    v += xor_lane_i<2>(v, lane);
    v += xor_lane_i<4>(v, lane);
    v += xor_lane_i<8>(v, lane);
    v += __builtin_bit_cast(int, xor_lane16(__builtin_bit_cast(float, v), lane));
    v += __builtin_bit_cast(int, xor_lane32(__builtin_bit_cast(float, v), lane));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    const int lane = threadIdx.x & 63;
    v = fmaxf(v, xor_lane<1>(v, lane));
    v = fmaxf(v, xor_lane<2>(v, lane));
    v = fmaxf(v, xor_lane<4>(v, lane));
    v = fmaxf(v, xor_lane<8>(v, lane));
    v = fmaxf(v, xor_lane16(v, lane));
    v = fmaxf(v, xor_lane32(v, lane));
    return v;
}

constexpr int Q16_MAXQ = 32512;

__device__ __forceinline__ void q16_store(uint8_t* row, int k, int blk, int i, int q) {
    // element i of block blk: chunk c' = i/16, group g = (i/4)%4, position j = i%4
    const int hi = (q + 128) >> 8;
    const int lo = q - (hi << 8);
    const int off = (blk * 8 + (i >> 4)) * 32 + 4 * (i & 3) + ((i >> 2) & 3);
    row[off] = (uint8_t)(int8_t)hi;
    row[off + 16] = (uint8_t)(int8_t)lo;
}

__global__ __launch_bounds__(256) void k_fwht(const void* __restrict__ x, int in_dt, void* __restrict__ y,
                                              int out_dt, const uint8_t* __restrict__ sign_bits, int k,
                                              uint32_t flags, int64_t q16_stride) {
    const int64_t row = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nblk = k >> 7;
    const int blk = blockIdx.x * 4 + wave;
    const int64_t base = row * (int64_t)k;
    __shared__ float red[4];
    // this wave's block first (its loads overlap the normalisation pass)
    const bool active = blk < nblk;
    const int i0 = (active ? blk : 0) * 128 + lane, i1 = i0 + 64;
    float a = load_elem(x, in_dt, base + i0);
    float c = load_elem(x, in_dt, base + i1);
    const uint32_t sg0 = sign_bits[i0 >> 3], sg1 = sign_bits[i1 >> 3];
    float inv = 1.0f;
    if (flags & PG_FLAG_RMSNORM) {
        // the whole row's squares: up to 64 loads per thread in flight at once
        float ss = 0.0f;
        for (int i0r = threadIdx.x; i0r < k; i0r += 256 * 64) {
            float v[64];
#pragma unroll
            for (int u = 0; u < 64; ++u) {
                const int i = i0r + 256 * u;
                v[u] = i < k ? load_elem(x, in_dt, base + i) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 64; ++u) ss += v[u] * v[u];
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        inv = 1.0f / sqrtf(tot / (float)k + 1e-6f);
    }
    if (!active) return;
    const float cnorm = 0.08838834764831845f;   // 2^-3.5
    if (flags & PG_FLAG_RMSNORM) {
        a = h2f(f2h(a * inv));
        c = h2f(f2h(c * inv));
    }
    if ((sg0 >> (i0 & 7)) & 1) a = -a;
    if ((sg1 >> (i1 & 7)) & 1) c = -c;
    {
        const float t0 = a + c, t1 = a - c;
        a = t0;
        c = t1;
    }
    // butterflies at distance 32 and 16 cross DPP rows (lane exchange); 8..1
    // stay inside a row of 16 lanes (DPP shifts)
    {
        float pa = xor_lane32(a, lane), pc = xor_lane32(c, lane);
        bool upper = (lane & 32) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
        pa = xor_lane16(a, lane); pc = xor_lane16(c, lane); upper = (lane & 16) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
        pa = xor_lane<8>(a, lane); pc = xor_lane<8>(c, lane); upper = (lane & 8) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
        pa = xor_lane<4>(a, lane); pc = xor_lane<4>(c, lane); upper = (lane & 4) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
        pa = xor_lane<2>(a, lane); pc = xor_lane<2>(c, lane); upper = (lane & 2) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
        pa = xor_lane<1>(a, lane); pc = xor_lane<1>(c, lane); upper = (lane & 1) != 0;
        a = upper ? pa - a : a + pa;
        c = upper ? pc - c : c + pc;
    }
    a *= cnorm;
    c *= cnorm;
    if (out_dt != PG_Q16) {
        store_elem(y, out_dt, base + i0, a);
        store_elem(y, out_dt, base + i1, c);
        return;
    }
    uint8_t* rowp = (uint8_t*)y + row * q16_stride;
    const float mx = wave_max(fmaxf(fabsf(a), fabsf(c)));
    const float inv_sx = mx > 0.0f ? (float)Q16_MAXQ / mx : 0.0f;
    const int qa = (int)rintf(a * inv_sx);
    const int qc = (int)rintf(c * inv_sx);
    q16_store(rowp, k, blk, lane, qa);
    q16_store(rowp, k, blk, lane + 64, qc);
    const int sa = wave_sum_i(qa), sc = wave_sum_i(qc);
    if (lane == 0) {
        float* sxp = (float*)(rowp + 2 * (int64_t)k);
        int* sump = (int*)(rowp + 2 * (int64_t)k + k / 32);
        sxp[blk] = mx / (float)Q16_MAXQ;
        sump[2 * blk] = sa;
        sump[2 * blk + 1] = sc;
    }
}

// ------------------------------------------------------------------- qgemv
// Batch 1..8 product.  A wave holds 8 teams of 8 lanes; a team owns one row
// and its lanes take 16-byte chunks (16 groups = half a 128-block) of the row
// in turn, so each team reads one full 128-byte line per step and the
// workgroup's 32 rows are streamed once.  The rotated activations of a tile
// of batch rows sit in LDS (fp32).  A chunk's starting state is 0 on even
// chunks (block start) and comes from the last three bytes of the left
// neighbour lane's chunk on odd chunks.  Per chunk: levels times x in fp32,
// then one multiply by the block scale; the 8 lane partials of a row are
// summed with lane exchanges in a fixed order.
template <int BT>
__global__ __launch_bounds__(256) void k_qgemv_v1(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const void* __restrict__ x, int x_dt, int batch,
                                                  float* __restrict__ y) {
    extern __shared__ float xs[];   // [BT][k]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = lane >> 3, tl = lane & 7;
    const int row = blockIdx.x * 32 + wave * 8 + team;
    const int rowc = row < n ? row : n - 1;
    const int kg = k >> 2;                 // code bytes per row
    const int nchunk = k >> 6;             // 16-byte chunks per row
    const uint8_t* rp = codes + (int64_t)rowc * kg;
    const uint16_t* sp = scales + (int64_t)rowc * (k >> 7);
    for (int b0 = 0; b0 < batch; b0 += BT) {
        const int bt = batch - b0 < BT ? batch - b0 : BT;
        __syncthreads();
        for (int i = threadIdx.x; i < bt * k; i += 256) xs[i] = load_elem(x, x_dt, (int64_t)b0 * k + i);
        __syncthreads();
        float acc[BT];
#pragma unroll
        for (int q = 0; q < BT; ++q) acc[q] = 0.0f;
        for (int c0 = 0; c0 < nchunk; c0 += 8) {
            const int c = c0 + tl;
            uint4 q4 = make_uint4(0, 0, 0, 0);
            float sc = 0.0f;
            if (c < nchunk) {
                q4 = *reinterpret_cast<const uint4*>(rp + 16 * c);
                sc = h2f(sp[c >> 1]);
            }
            const uint32_t prev_w = __shfl(q4.w, (lane + 63) & 63);   // left neighbour's last dword
            uint32_t s = 0;
            if (c & 1) s = ((prev_w >> 24) & 1u) | (((prev_w >> 16) & 1u) << 1) | (((prev_w >> 8) & 1u) << 2);
            float cacc[BT];
#pragma unroll
            for (int q = 0; q < BT; ++q) cacc[q] = 0.0f;
            const uint32_t words[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const uint32_t byte = (words[g >> 2] >> (8 * (g & 3))) & 0xffu;
                int lv[4];
                levels_of(s, byte, lv);
                s = ((s << 1) | (byte & 1u)) & 7u;
                const int kk = 64 * c + 4 * g;
#pragma unroll
                for (int q = 0; q < BT; ++q) {
                    if (q < bt && c < nchunk) {
                        const float* xr = xs + q * k + kk;
                        cacc[q] += (float)lv[0] * xr[0] + (float)lv[1] * xr[1] + (float)lv[2] * xr[2] +
                                   (float)lv[3] * xr[3];
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < BT; ++q) acc[q] += sc * cacc[q];
        }
#pragma unroll
        for (int q = 0; q < BT; ++q) {
            float v = acc[q];
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 1);
            if (tl == 0 && row < n && q < bt) y[(int64_t)(b0 + q) * n + row] = v;
        }
    }
}

// ------------------------------------------------------- qgemv, fast path
// Batch 1..8 product on PG_Q16 activations.  Same team layout as above
// (8 lanes x 16-byte chunks per row step, each team reading whole 128-byte
// lines), R rows per team, the workgroup's activations staged once in LDS
// with direct global->LDS copies.  Decode never materialises a level: for a
// code dword (4 groups) and position j, the bytes of plane P_j hold
// (level + 7) / 2 = 4 e_j + 2 b_j + z0 of the four groups, built with a
// handful of shifts and masks (z0 and the parity bit b3 come from bit 0 of
// the three preceding bytes, obtained with byte-aligns against the previous
// dword); v_dot4_i32_i8 then multiplies the plane by the four groups'
// activation digits.  Per half-block:
//   sum level * q = 2 * (256 * hi + lo) - 7 * sum q
// exactly in int32, then one fp32 multiply by (weight scale * activation
// block scale).
// (a & m) | c and a ^ b ^ c, one gfx950 three-input bit operation each
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
__device__ __forceinline__ void planes_of(uint32_t d, uint32_t dp, uint32_t P[4]) {
    const uint32_t M1 = 0x01010101u, M2 = 0x02020202u, M4 = 0x04040404u;
    const uint32_t z = __builtin_amdgcn_alignbyte(d, dp, 2) & M1;    // z0 = u_{t-2}: bit 0 of byte g-2
    const uint32_t d1 = d >> 1, d2 = d >> 2, d3 = d >> 3, d4 = d >> 4, d5 = d >> 5;
    P[0] = and_or(d2, M4, and_or(d, M2, z));
    P[1] = and_or(d3, M4, and_or(d1, M2, z));
    P[2] = and_or(d4, M4, and_or(d2, M2, z));
    // b3 = z1 ^ b0 ^ b1 ^ b2 with z1 = u_t ^ u_{t-1} ^ u_{t-3} (bit 0 of bytes
    // g, g-1, g-3), formed directly at bit 1 of each byte: the funnel shifts
    // move those bit-0s there
    const uint32_t x1 = xor3(__builtin_amdgcn_alignbit(d, dp, 31), d, d1);
    const uint32_t x2 = xor3(d2, __builtin_amdgcn_alignbit(d, dp, 23), __builtin_amdgcn_alignbit(d, dp, 7));
    P[3] = and_or(d5, M4, and_or(x1 ^ x2, M2, z));
}

// The workgroup's W waves share 8*R rows and split each row's chunks between
// them (wave w, team lane tl takes chunks w*8 + tl + 8W*i), so a small matrix
// still spreads over many waves.  Each wave copies only the activation digits
// of its own chunks (1 KiB per round i, one direct global->LDS copy) plus the
// block scales and half-block sums into its own LDS region, so no
// workgroup-wide barrier precedes the dot products; the per-wave partial sums
// meet in LDS at the end and are added in wave order.
struct Q16Layout {
    int rounds;      // chunk rounds per wave: ceil(nchunk / (8W))
    int sxs_bytes;   // staged scale + sum bytes per batch row (multiple of 16)
    int wave_bytes;  // LDS bytes per wave
};

__host__ __device__ inline Q16Layout q16_layout(int k, int W, int BS) {
    Q16Layout L;
    const int nchunk = k / 64;
    L.rounds = (nchunk + 8 * W - 1) / (8 * W);
    L.sxs_bytes = ((3 * k / 32) + 15) & ~15;
    L.wave_bytes = BS * (L.rounds * 1024 + ((L.sxs_bytes + 1023) & ~1023));
    return L;
}

template <int BS, int R>
__global__ __launch_bounds__(512) void k_qgemv_q16(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int n, int k,
                                                   const uint8_t* __restrict__ xq, int xq_stride, int batch,
                                                   float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int W = nthr >> 6;
    const int lane = tid & 63, wave = tid >> 6;
    const int team = lane >> 3, tl = lane & 7;
    const int rbase = blockIdx.x * 8 * R + team * R;
    const int kg = k >> 2, nchunk = k >> 6, nbk = k >> 7;
    const int cstep = 8 * W;
    const Q16Layout L = q16_layout(k, W, BS);
    const int bregion = L.wave_bytes / BS;                      // per batch row inside a wave's region
    uint8_t* wlds = lds + wave * L.wave_bytes;
    float* red = reinterpret_cast<float*>(lds + W * L.wave_bytes);   // [W][8][R][BS]
    const uint8_t* rp[R];
    const uint16_t* sp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = rbase + r < n ? rbase + r : n - 1;
        rp[r] = codes + (int64_t)row * kg;
        sp[r] = scales + (int64_t)row * nbk;
    }
    const int cfirst = wave * 8 + tl;
    for (int b0 = 0; b0 < batch; b0 += BS) {
        const int bs = batch - b0 < BS ? batch - b0 : BS;
        if (b0 > 0) __syncthreads();                            // previous round's reduction done
        // first code chunk in flight before the activations are staged
        uint4 q[R];
        float ws[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            q[r] = cfirst < nchunk ? *reinterpret_cast<const uint4*>(rp[r] + 16 * cfirst) : make_uint4(0, 0, 0, 0);
            ws[r] = cfirst < nchunk ? h2f(sp[r][cfirst >> 1]) : 0.0f;
        }
        // this wave's activation digits, block scales and half-block sums
        for (int b = 0; b < bs; ++b) {
            const uint8_t* xrow = xq + (int64_t)(b0 + b) * xq_stride;
            uint8_t* dst = wlds + b * bregion;
            for (int i = 0; i < L.rounds; ++i) {
                const int c0 = wave * 8 + cstep * i;                 // first chunk of the round
                if (c0 < nchunk && 128 * c0 + 16 * lane < 2 * k)
                    __builtin_amdgcn_global_load_lds(xrow + 128 * c0 + 16 * lane, dst + 1024 * i, 16, 0, 0);
            }
            uint8_t* sdst = dst + 1024 * L.rounds;
            for (int o = 0; o < L.sxs_bytes; o += 1024)
                if (o + 16 * lane < L.sxs_bytes)
                    __builtin_amdgcn_global_load_lds(xrow + 2 * k + o + 16 * lane, sdst + o, 16, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        float acc[R][BS];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < BS; ++b) acc[r][b] = 0.0f;
        // Up to U chunks per lane are requested together before any is used,
        // so a lane that owns only a few chunks (small matrices) waits for one
        // memory latency, not one per chunk.  The loop bound is wave-uniform:
        // every lane steps through the same iterations (lanes past the end
        // compute on clamped data and discard it).
        constexpr int U = 4;
        for (int c0 = wave * 8; c0 < nchunk; c0 += U * cstep) {
            uint4 qu[U][R];
            float wsu[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + tl + u * cstep;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (u == 0 && c0 == wave * 8) {
                        qu[u][r] = q[r];
                        wsu[u][r] = ws[r];
                    } else {
                        qu[u][r] = c < nchunk ? *reinterpret_cast<const uint4*>(rp[r] + 16 * c) : make_uint4(0, 0, 0, 0);
                        wsu[u][r] = c < nchunk ? h2f(sp[r][c >> 1]) : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c0 + u * cstep >= nchunk) break;                 // wave-uniform
                const int c = c0 + tl + u * cstep;
                const bool valid = c < nchunk;
                const int round = (c0 - wave * 8) / cstep + u;
                uint32_t dp0[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    // last dword of the left neighbour's chunk (same team when c is odd)
                    const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)qu[u][r].w, 0x111, 0xf, 0xf, true);
                    dp0[r] = (c & 1) ? left : 0u;
                }
                int hi[R][BS], lo[R][BS];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < BS; ++b) { hi[r][b] = 0; lo[r][b] = 0; }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    uint32_t P[R][4];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t w4[4] = {qu[u][r].x, qu[u][r].y, qu[u][r].z, qu[u][r].w};
                        planes_of(w4[m], m == 0 ? dp0[r] : w4[m - 1], P[r]);
                    }
#pragma unroll
                    for (int b = 0; b < BS; ++b) {
                        if (b < bs) {
                            const uint4* xp = reinterpret_cast<const uint4*>(wlds + b * bregion + 1024 * round +
                                                                             128 * tl + 32 * m);
                            const uint4 xh = xp[0], xl = xp[1];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                int h = hi[r][b], l = lo[r][b];
                                h = __builtin_amdgcn_sdot4((int)P[r][0], (int)xh.x, h, false);
                                l = __builtin_amdgcn_sdot4((int)P[r][0], (int)xl.x, l, false);
                                h = __builtin_amdgcn_sdot4((int)P[r][1], (int)xh.y, h, false);
                                l = __builtin_amdgcn_sdot4((int)P[r][1], (int)xl.y, l, false);
                                h = __builtin_amdgcn_sdot4((int)P[r][2], (int)xh.z, h, false);
                                l = __builtin_amdgcn_sdot4((int)P[r][2], (int)xl.z, l, false);
                                h = __builtin_amdgcn_sdot4((int)P[r][3], (int)xh.w, h, false);
                                l = __builtin_amdgcn_sdot4((int)P[r][3], (int)xl.w, l, false);
                                hi[r][b] = h;
                                lo[r][b] = l;
                            }
                        }
                    }
                }
                if (valid) {
#pragma unroll
                    for (int b = 0; b < BS; ++b) {
                        if (b < bs) {
                            const uint8_t* sx_base = wlds + b * bregion + 1024 * L.rounds;
                            const float sxv = reinterpret_cast<const float*>(sx_base)[c >> 1];
                            const int qs = reinterpret_cast<const int*>(sx_base + k / 32)[c];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                const int t = 2 * (hi[r][b] * 256 + lo[r][b]) - 7 * qs;
                                acc[r][b] += (wsu[u][r] * sxv) * (float)t;
                            }
                        }
                    }
                }
            }
        }
        // team sums (lanes tl = 0..7), then wave partials through LDS
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < BS; ++b) {
                float v = acc[r][b];
                v += xor_lane<4>(v, lane);
                v += xor_lane<2>(v, lane);
                v += xor_lane<1>(v, lane);
                if (tl == 0) red[((wave * 8 + team) * R + r) * BS + b] = v;
            }
        __syncthreads();
        for (int o = tid; o < 8 * R * BS; o += nthr) {
            const int b = o % BS, r = (o / BS) % R, t = o / (BS * R);
            float v = 0.0f;
            for (int w = 0; w < W; ++w) v += red[((w * 8 + t) * R + r) * BS + b];
            const int row = blockIdx.x * 8 * R + t * R + r;
            if (row < n && b < bs) y[(int64_t)(b0 + b) * n + row] = v;
        }
    }
}

// ------------------------------------------------ fused stage of a stack
// y = W~ . R . n(x) in one launch: the activation rotation (with the RMS
// normalisation and fp16 rounding of PG_FLAG_RMSNORM) is the product's
// prologue.  One workgroup per CU owns R consecutive weight rows with all of
// their k columns, so the launch is one pass over the codes and each lane
// waits for memory once:
//   1. the input row is copied to LDS (direct global -> LDS copies) and then
//      every code chunk of the lane is requested; waiting until only the code
//      requests are outstanding means x has arrived (memory operations of a
//      wave complete in order);
//   2. the RMS of x is summed, and the normalised, sign-flipped values are
//      staged in LDS as fp16 (exact: n() rounds to fp16, and fp16 inputs are
//      exact), one 128-block per 272-byte row;
//   3. the Hadamard products run on the matrix cores: v_mfma_f32_32x32x16_f16
//      with the +-1 entries of H as the A operand (built from bit patterns in
//      registers, no memory), 32 blocks per tile.  The rows of H are ordered
//      so that each lane's four accumulators r = 4i .. 4i + 3 are the four
//      groups of one position in a PG_Q16-style digit dword;
//   4. each wave quantises its 32 x 32 tile (one scale per 32 elements, from
//      the tile's own maximum, so no other wave is waited for): q =
//      rint(v * 32512 / max) by one fma with 1.5 * 2^23, which leaves q as a
//      16-bit two's complement integer in the low half of the float's bits;
//      byte permutes split it into a signed high digit floor(q / 256) and an
//      unsigned low digit q mod 256, four groups per dword;
//   5. team T of 8 lanes takes column group cg = T % CG (chunks 8 cg .. 8 cg
//      + 7, one 128-byte line of a row per team) and rows rp, rp + RP, ...
//      (rp = T / CG); a lane reads its chunk's digits once per batch row and
//      uses them for all of its rows: levels come from bit planes (planes_of)
//      and meet the digits in v_dot4 (signed for the high digit, unsigned for
//      the low one);
//   6. team sums go to LDS per (row, column group) and are added in column
//      group order.
// Launch shape (host): W waves, R rows per workgroup, CG = ceil(k/512),
// RP = 8W / CG, at most RS rows per lane and XG 8-value groups of x per
// thread.
struct FusedShape {
    int W, R, CG, RP, RS, XG;
    int BT, BTM;         // batch rows per launch, and the kernel's compile-time bound on them
};

constexpr int FS_PITCH = 144;      // LDS bytes per 64-value chunk of digits (128 + 16 against bank conflicts)
constexpr int FS_XPITCH = 272;     // LDS bytes per staged fp16 128-block (256 + 16)

// LDS bytes per batch row: digits, then per 32-value quarter its scale and
// its sum of q
__host__ __device__ inline int fused_row_bytes(int k) { return ((k / 64) * FS_PITCH + (k / 32) * 8 + 15) & ~15; }
// one input row as given (fp32 or fp16), and its fp16 blocks
__host__ __device__ inline int fused_xrow_bytes(int k, int esz) { return (k * esz + 15) & ~15; }
__host__ __device__ inline int fused_xhrow_bytes(int k) { return (k / 128) * FS_XPITCH; }

// LDS of one launch: BT rows of x, of fp16 blocks and of digits, the sign
// bits, the team sums and the per-wave sums of squares
__host__ inline size_t fused_lds_bytes(int k, int esz, const FusedShape& S) {
    return (size_t)S.BT * (fused_xrow_bytes(k, esz) + fused_xhrow_bytes(k) + fused_row_bytes(k)) +
           (size_t)((k / 8 + 15) & ~15) + (size_t)S.BT * S.R * S.CG * 4 + (size_t)S.BT * S.W * 4;
}

// s_waitcnt operand: at most n vector-memory operations of this wave still
// outstanding, the other counters unrestricted (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Element of a 128-block held by accumulator row M = 8 i + 4 h + r of row
// tile mt: quarter mt, part i / 2 of the quarter, group r, position
// 2 (i % 2) + h.
__device__ __forceinline__ int fs_elem(int mt, int M) {
    const int i = M >> 3, h = (M >> 2) & 1, r = M & 3;
    return 32 * mt + 16 * (i >> 1) + 4 * r + 2 * (i & 1) + h;
}

typedef _Float16 fs_f16x8 __attribute__((ext_vector_type(8)));

// Instances that loop over batch tiles themselves (the codes stay in
// registers); the others get one launch per tile.  The loop keeps more
// values live, so only instances with registers to spare have it.
__host__ __device__ constexpr bool fused_loops(int RS, int BTM) {
    return BTM > 1 && RS * BTM <= 16 && !(RS == 2 && BTM == 8);
}

template <int XDT, int XG, int RS, int BTM>
__global__ __launch_bounds__(512) void k_rot_qgemv(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int n, int k,
                                                    const void* __restrict__ x, int64_t ldx,
                                                    const uint8_t* __restrict__ sign_bits, uint32_t flags,
                                                    int batch, float* __restrict__ y, int R, int CG, int RP,
                                                    int BT) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // every argument is fetched by one scalar load burst here: loads left to
    // the point of first use each cost a full round trip, and a scalar load
    // in flight also holds back every later wait for LDS
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(ldx), "s"(sign_bits), "s"(flags),
                 "s"(batch), "s"(y), "s"(R), "s"(CG), "s"(RP), "s"(BT));
    constexpr int nthr = 512, W = 8;                           // the launch shape is fixed
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int T = wave * 8 + (lane >> 3), tl = lane & 7;
    const int kg = k >> 2, nchunk = k >> 6, nbk = k >> 7, ngr = k >> 3;
    const int row0 = blockIdx.x * R;
    const int bt0 = batch < BT ? batch : BT;                 // batch rows of the first tile (<= BT <= BTM)
    const int esz = XDT == PG_F32 ? 4 : 2;
    const int xrow = fused_xrow_bytes(k, esz), xhrow = fused_xhrow_bytes(k), rb = fused_row_bytes(k);
    uint8_t* xbuf = lds;                                     // [BT][xrow] x as given
    uint8_t* xh = xbuf + (size_t)BT * xrow;                  // [BT][nbk][FS_XPITCH] fp16 blocks
    uint8_t* sbuf = xh + (size_t)BT * xhrow;                 // sign bits
    uint8_t* rows_lds = sbuf + ((k / 8 + 15) & ~15);         // [BT][rb] digits, scales, sums
    float* part = reinterpret_cast<float*>(rows_lds + (size_t)BT * rb);   // [BT][R][CG]
    float* wsum = part + (size_t)BT * R * CG;                             // [BT][W]
    const bool norm = (flags & PG_FLAG_RMSNORM) != 0;

    // this lane's column of chunks and its rows
    const int cg = T % CG, rp = T / CG;
    const int c = 8 * cg + tl;
    const bool col_ok = rp < RP && c < nchunk;
    const int cc = c < nchunk ? c : nchunk - 1;

    // ---- 1. x rows to LDS (16 bytes per lane), sign bits, then all code chunks
    auto copy_x = [&](int b0, int bt) {
        for (int b = 0; b < bt; ++b) {
            const uint8_t* src = (const uint8_t*)x + (int64_t)(b0 + b) * ldx * esz;
            const int bytes = k * esz;
            for (int o = wave * 1024; o < bytes; o += W * 1024)
                if (o + 16 * lane < bytes)
                    __builtin_amdgcn_global_load_lds(src + o + 16 * lane, xbuf + (size_t)b * xrow + o, 16, 0, 0);
        }
    };
    copy_x(0, bt0);
    uint32_t sg = 0;
    const bool sg_on = tid < k / 32;
    if (sg_on) sg = reinterpret_cast<const uint32_t*>(sign_bits)[tid];
    asm volatile("" ::: "memory");
    // The scale of a chunk comes with its neighbour in one aligned dword (the
    // half is picked where it is used, so nothing converts it early).
    uint4 q[RS];
    uint32_t wsr[RS];
    bool rok[RS], whi[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
        const int r = rp + j * RP;
        rok[j] = col_ok && r < R && row0 + r < n;
        const int row = rok[j] ? row0 + r : (row0 < n ? row0 : n - 1);
        q[j] = *reinterpret_cast<const uint4*>(codes + (int64_t)row * kg + 16 * cc);
        const int64_t si = (int64_t)row * nbk + (cc >> 1);
        whi[j] = (si & 1) != 0;
        wsr[j] = reinterpret_cast<const uint32_t*>(scales)[si >> 1];
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * RS));      // x copies and sign loads done
    if (sg_on) reinterpret_cast<uint32_t*>(sbuf)[tid] = sg;
    __syncthreads();

    // A operand patterns of the Hadamard product (see fs_elem): lane l holds
    // row M = l % 32 and inputs 8 (l / 32) + t of a 16-wide step; the entry is
    //   (-1)^popcount(e & 7 & t) (-1)^(bit 3 of e & l / 32)   (fixed per lane)
    //   (-1)^(bit 4 of e & step % 2)                            (odd steps)
    //   (-1)^popcount(mt & step / 2)                            (uniform)
    uint32_t apat[2][4];
    {
        const int e0 = fs_elem(0, lane & 31);
        const int ha = lane >> 5;
        const bool f_lane = ((e0 >> 3) & 1) & ha;
        const bool f_odd = (e0 >> 4) & 1;
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
            const bool n0 = (__builtin_popcount(e0 & 7 & t) & 1) ^ f_lane;
            const bool n1 = (__builtin_popcount(e0 & 7 & (t + 1)) & 1) ^ f_lane;
            const uint32_t wv = (n0 ? 0xBC00u : 0x3C00u) | ((n1 ? 0xBC00u : 0x3C00u) << 16);
            apat[0][t >> 1] = wv;
            apat[1][t >> 1] = f_odd ? (wv ^ 0x80008000u) : wv;
        }
    }
    const int ntile = (nbk + 31) >> 5;

    // ---- 2.-6. one tile of at most BT batch rows, x already in LDS; the
    // codes stay in registers from one tile to the next
    auto tile = [&](int b0, int bt) {
        // ---- 2. sums of squares of every batch row: thread t takes 8-value
        // groups t + nthr u, then wave sums
        auto read8 = [&](int b, int gi, float v[8]) {
            const uint8_t* xr = xbuf + (size_t)b * xrow;
            if (XDT == PG_F32) {
                const float4 v0 = *reinterpret_cast<const float4*>(xr + 32 * gi);
                const float4 v1 = *reinterpret_cast<const float4*>(xr + 32 * gi + 16);
                v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
                v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
            } else {
                const uint4 w = *reinterpret_cast<const uint4*>(xr + 16 * gi);
                const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
    #pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[2 * t] = h2f((uint16_t)(w4[t] & 0xffffu));
                    v[2 * t + 1] = h2f((uint16_t)(w4[t] >> 16));
                }
            }
        };
        if (norm) {
            for (int b = 0; b < bt; ++b) {
                float ss = 0.0f;
    #pragma unroll
                for (int u = 0; u < XG; ++u) {
                    const int gi = tid + nthr * u;
                    if (gi < ngr) {
                        float v[8];
                        read8(b, gi, v);
    #pragma unroll
                        for (int t = 0; t < 8; ++t) ss += v[t] * v[t];
                    }
                }
                ss = wave_sum(ss);
                if (lane == 0) wsum[b * W + wave] = ss;
            }
            __syncthreads();
        }
        // ---- 3. normalised, sign-flipped fp16 blocks of every batch row
        for (int b = 0; b < bt; ++b) {
            float inv = 1.0f;
            if (norm) {
                float tot = 0.0f;
                for (int w = 0; w < W; ++w) tot += wsum[b * W + w];
                inv = __builtin_amdgcn_rsqf(tot * __builtin_amdgcn_rcpf((float)k) + 1e-6f);
            }
    #pragma unroll
            for (int u = 0; u < XG; ++u) {
                const int gi = tid + nthr * u;
                if (gi < ngr) {
                    float v[8];
                    read8(b, gi, v);
                    const uint32_t s8 = sbuf[gi];
                    uint32_t hw[4];
    #pragma unroll
                    for (int t = 0; t < 8; t += 2) {
                        uint32_t h0 = f2h(norm ? v[t] * inv : v[t]);
                        uint32_t h1 = f2h(norm ? v[t + 1] * inv : v[t + 1]);
                        h0 ^= ((s8 >> t) & 1u) << 15;
                        h1 ^= ((s8 >> (t + 1)) & 1u) << 15;
                        hw[t >> 1] = h0 | (h1 << 16);
                    }
                    *reinterpret_cast<uint4*>(xh + (size_t)b * xhrow + (gi >> 4) * FS_XPITCH + (gi & 15) * 16) =
                        make_uint4(hw[0], hw[1], hw[2], hw[3]);
                }
            }
        }
        __syncthreads();
        // ---- 4. Hadamard tiles on the matrix cores, quantised per 32 values
        for (int job = wave; job < bt * 4 * ntile; job += W) {
            const int b = job / (4 * ntile), jj = job - b * 4 * ntile;
            const int nt = jj >> 2, mt = jj & 3;
            const int blk = nt * 32 + (lane & 31);
            const bool bok = blk < nbk;
            uint8_t* dig = rows_lds + (size_t)b * rb;
            float* sxq = reinterpret_cast<float*>(dig + nchunk * FS_PITCH);
            int* sqq = reinterpret_cast<int*>(dig + nchunk * FS_PITCH + (k / 32) * 4);
            const uint8_t* xr = xh + (size_t)b * xhrow + (bok ? blk : 0) * FS_XPITCH + 16 * (lane >> 5);
            f32x16 acc;
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            uint4 bv[8];                                         // all B operands first: one LDS wait
    #pragma unroll
            for (int st = 0; st < 8; ++st) bv[st] = *reinterpret_cast<const uint4*>(xr + 32 * st);
    #pragma unroll
            for (int st = 0; st < 8; ++st) {
                const uint4 bw = bok ? bv[st] : make_uint4(0, 0, 0, 0);
                const uint32_t fl = (__builtin_popcount(mt & (st >> 1)) & 1) ? 0x80008000u : 0u;
                const uint32_t* av = apat[st & 1];
                const uint4 aw = make_uint4(av[0] ^ fl, av[1] ^ fl, av[2] ^ fl, av[3] ^ fl);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(fs_f16x8, aw),
                                                             __builtin_bit_cast(fs_f16x8, bw), acc, 0, 0, 0);
            }
            // quarter maximum: 16 values per lane, then the lane pair (l, l + 32)
            float mx = 0.0f;
    #pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(acc[r]));
            mx = fmaxf(mx, xor_lane32(mx, lane));
            const float s = mx > 0.0f ? (float)Q16_MAXQ * __builtin_amdgcn_rcpf(mx) : 0.0f;
            const int ch = 2 * blk + (mt >> 1);                  // chunk of this quarter
            uint8_t* dq = dig + (bok ? ch : 0) * FS_PITCH + 32 * 2 * (mt & 1) + 4 * (lane >> 5);
            int shi = 0, slo = 0;
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t bits[4];
    #pragma unroll
                for (int r = 0; r < 4; ++r) bits[r] = __builtin_bit_cast(uint32_t, fmaf(acc[4 * i + r], s, 12582912.0f));
                const uint32_t t01 = __builtin_amdgcn_perm(bits[1], bits[0], 0x05040100u);
                const uint32_t t23 = __builtin_amdgcn_perm(bits[3], bits[2], 0x05040100u);
                const uint32_t dl = __builtin_amdgcn_perm(t23, t01, 0x06040200u);   // q mod 256 of groups 0..3
                const uint32_t dh = __builtin_amdgcn_perm(t23, t01, 0x07050301u);   // floor(q / 256)
                shi = __builtin_amdgcn_sdot4((int)dh, 0x01010101, shi, false);
                slo = (int)__builtin_amdgcn_udot4(dl, 0x01010101u, (uint32_t)slo, false);
                // part 2 (mt % 2) + i / 2 of the chunk, position 2 (i % 2) + l / 32
                if (bok) {
                    uint8_t* dd = dq + 32 * (i >> 1) + 8 * (i & 1);
                    *reinterpret_cast<uint32_t*>(dd) = dh;
                    *reinterpret_cast<uint32_t*>(dd + 16) = dl;
                }
            }
            int qs = 256 * shi + slo;
            qs += __builtin_bit_cast(int, xor_lane32(__builtin_bit_cast(float, qs), lane));
            if (bok && lane < 32) {
                sxq[4 * blk + mt] = mx * (0.08838834764831845f / (float)Q16_MAXQ);   // 2^-3.5 max / 32512
                sqq[4 * blk + mt] = qs;
            }
        }
        __syncthreads();
        // ---- 5. decode and dot products: the planes of a code dword are built
        // once and used for every batch row
        {
            // codes and scales are used only here, through copies passed through
            // an opaque move: that keeps the compiler from hoisting their decode
            // above the rotation (which would wait for every code request first)
            uint4 qb[RS];
            uint32_t wb[RS];
    #pragma unroll
            for (int j = 0; j < RS; ++j) {
                qb[j] = q[j];
                wb[j] = wsr[j];
                asm volatile("" : "+v"(qb[j].x), "+v"(qb[j].y), "+v"(qb[j].z), "+v"(qb[j].w), "+v"(wb[j]));
            }
            float sx0[BTM], sx1[BTM];
            int sq0[BTM], sq1[BTM];
    #pragma unroll
            for (int b = 0; b < BTM; ++b) {
                const uint8_t* dig = rows_lds + (size_t)(b < bt ? b : 0) * rb;
                const float* sxq = reinterpret_cast<const float*>(dig + nchunk * FS_PITCH);
                const int* sqq = reinterpret_cast<const int*>(dig + nchunk * FS_PITCH + (k / 32) * 4);
                sx0[b] = sxq[2 * cc];
                sx1[b] = sxq[2 * cc + 1];
                sq0[b] = sqq[2 * cc];
                sq1[b] = sqq[2 * cc + 1];
            }
            float tq[RS][BTM];
            int hi[RS][BTM], lo[RS][BTM];
    #pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m == 0 || m == 2)
    #pragma unroll
                    for (int j = 0; j < RS; ++j)
    #pragma unroll
                        for (int b = 0; b < BTM; ++b) { hi[j][b] = 0; lo[j][b] = 0; }
                uint4 xh4[BTM], xl4[BTM];
    #pragma unroll
                for (int b = 0; b < BTM; ++b) {
                    const uint8_t* dig = rows_lds + (size_t)(b < bt ? b : 0) * rb + cc * FS_PITCH + 32 * m;
                    xh4[b] = *reinterpret_cast<const uint4*>(dig);
                    xl4[b] = *reinterpret_cast<const uint4*>(dig + 16);
                }
    #pragma unroll
                for (int j = 0; j < RS; ++j) {
                    const uint32_t w4[4] = {qb[j].x, qb[j].y, qb[j].z, qb[j].w};
                    uint32_t prev;
                    if (m == 0) {
                        // last dword of the left neighbour's chunk (same row, chunk c - 1)
                        const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb[j].w, 0x111, 0xf, 0xf, true);
                        prev = (c & 1) ? left : 0u;
                    } else {
                        prev = w4[m - 1];
                    }
                    uint32_t P[4];
                    planes_of(w4[m], prev, P);
    #pragma unroll
                    for (int b = 0; b < BTM; ++b) {
                        if (BTM > 1 && b >= bt) break;                 // uniform
                        int h = hi[j][b];
                        uint32_t l = (uint32_t)lo[j][b];
                        h = __builtin_amdgcn_sdot4((int)P[0], (int)xh4[b].x, h, false);
                        l = __builtin_amdgcn_udot4(P[0], xl4[b].x, l, false);
                        h = __builtin_amdgcn_sdot4((int)P[1], (int)xh4[b].y, h, false);
                        l = __builtin_amdgcn_udot4(P[1], xl4[b].y, l, false);
                        h = __builtin_amdgcn_sdot4((int)P[2], (int)xh4[b].z, h, false);
                        l = __builtin_amdgcn_udot4(P[2], xl4[b].z, l, false);
                        h = __builtin_amdgcn_sdot4((int)P[3], (int)xh4[b].w, h, false);
                        l = __builtin_amdgcn_udot4(P[3], xl4[b].w, l, false);
                        hi[j][b] = h;
                        lo[j][b] = (int)l;
                    }
                }
                // quarter done: sum level * q = 2 (256 hi + lo) - 7 sum q
                if (m == 1)
    #pragma unroll
                    for (int j = 0; j < RS; ++j)
    #pragma unroll
                        for (int b = 0; b < BTM; ++b) tq[j][b] = sx0[b] * (float)(2 * (hi[j][b] * 256 + lo[j][b]) - 7 * sq0[b]);
                if (m == 3)
    #pragma unroll
                    for (int j = 0; j < RS; ++j)
    #pragma unroll
                        for (int b = 0; b < BTM; ++b) tq[j][b] += sx1[b] * (float)(2 * (hi[j][b] * 256 + lo[j][b]) - 7 * sq1[b]);
            }
    #pragma unroll
            for (int j = 0; j < RS; ++j) {
                const float wsc = h2f((uint16_t)(whi[j] ? wb[j] >> 16 : wb[j]));
    #pragma unroll
                for (int b = 0; b < BTM; ++b) {
                    if (BTM > 1 && b >= bt) break;                     // uniform
                    float v = rok[j] ? wsc * tq[j][b] : 0.0f;
                    v += xor_lane<4>(v, lane);
                    v += xor_lane<2>(v, lane);
                    v += xor_lane<1>(v, lane);
                    if (tl == 0 && rp < RP && rp + j * RP < R) part[((size_t)b * R + rp + j * RP) * CG + cg] = v;
                }
            }
        }
        __syncthreads();
        for (int o = tid; o < bt * R; o += nthr) {
            const int b = o / R, r = o - b * R;
            if (row0 + r >= n) continue;
            const float* pr = part + ((size_t)b * R + r) * CG;
            float v = 0.0f;
            for (int g = 0; g < CG; ++g) v += pr[g];
            y[(int64_t)(b0 + b) * n + row0 + r] = v;
        }
    };
    tile(0, bt0);
    if constexpr (fused_loops(RS, BTM))
    for (int b0 = BT; b0 < batch; b0 += BT) {
        // further tiles (when the LDS holds fewer rows than the batch): the
        // same codes against the next rows of x, no second pass over memory
        const int bt = batch - b0 < BT ? batch - b0 : BT;
        __syncthreads();                                     // last tile's sums read
        copy_x(b0, bt);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        tile(b0, bt);
    }
}

// ------------------------------------------------------------------- qgemm
// Prompt product Y[m][n] on the matrix cores.  Workgroup tile: 128 rows of X
// by 128 weight rows, K advanced 64 at a time (half a scale block).  Each
// step copies the bf16 X tile to LDS and decodes the weight tile to LDS as
// bf16 levels (small odd integers, exact in bf16).  Four waves each own a
// 64x64 output block of 2x2 v_mfma_f32_32x32x16_bf16 tiles; the matrix cores
// accumulate one 128-block's levels . x in fp32, which is then multiplied by
// the block scale of its weight row and added to the running fp32 sum.
constexpr int QG_BM = 128, QG_BN = 128, QG_BK = 64, QG_LDK = QG_BK + 8;   // padded LDS row (bf16)

__global__ __launch_bounds__(256) void k_qgemm_v1(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const uint16_t* __restrict__ x, int m,
                                                  float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[QG_BM * QG_LDK];
    __shared__ __attribute__((aligned(16))) uint16_t ws[QG_BN * QG_LDK];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;          // wave's 64x64 block
    const int m0 = blockIdx.y * QG_BM, n0 = blockIdx.x * QG_BN;
    const int kg = k >> 2, nbk = k >> 7;
    f32x16 acc[2][2], bacc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[i][j][r] = 0.0f; bacc[i][j][r] = 0.0f; }

    // decode assignment: thread -> (weight row, 8 code bytes) of the 16-byte step
    const int drow = tid >> 1, dsub = tid & 1;
    const int wrow = n0 + drow < n ? n0 + drow : n - 1;
    const uint8_t* wrp = codes + (int64_t)wrow * kg;
    for (int kb = 0; kb < k; kb += QG_BK) {
        // X tile: 128 rows x 64 bf16 = 8 x 16 B per row; 256 threads x 4 loads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i;             // 0..1023
            const int r = idx >> 3, cc = idx & 7;
            const int gr = m0 + r < m ? m0 + r : m - 1;
            const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)gr * k + kb + 8 * cc);
            *reinterpret_cast<uint4*>(xs + r * QG_LDK + 8 * cc) = v;
        }
        // weight tile: this thread's 8 bytes of row drow, groups kb/4 + 8*dsub ...
        {
            const int g0 = (kb >> 2) + 8 * dsub;       // first group index in the row
            const int gb = g0 & 31;                    // position inside the 32-group block
            const uint2 v = *reinterpret_cast<const uint2*>(wrp + g0);
            uint32_t s = 0;
            if (gb >= 3) {
                const uint32_t u1 = wrp[g0 - 1] & 1u, u2 = wrp[g0 - 2] & 1u, u3 = wrp[g0 - 3] & 1u;
                s = u1 | (u2 << 1) | (u3 << 2);
            }
            const uint32_t words[2] = {v.x, v.y};
            uint16_t* dst = ws + drow * QG_LDK + 32 * dsub;
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const uint32_t byte = (words[g >> 2] >> (8 * (g & 3))) & 0xffu;
                int lv[4];
                levels_of(s, byte, lv);
                s = ((s << 1) | (byte & 1u)) & 7u;
                uint2 pk;
                pk.x = (uint32_t)f2bf((float)lv[0]) | ((uint32_t)f2bf((float)lv[1]) << 16);
                pk.y = (uint32_t)f2bf((float)lv[2]) | ((uint32_t)f2bf((float)lv[3]) << 16);
                *reinterpret_cast<uint2*>(dst + 4 * g) = pk;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < QG_BK; kk += 16) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8*>(xs + r * QG_LDK + kk + 8 * (lane >> 5));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8*>(ws + r * QG_LDK + kk + 8 * (lane >> 5));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], bacc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (((kb + QG_BK) & 127) == 0) {               // end of a 128-block: apply its scales
            const int blk = kb >> 7;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                const int colc = col < n ? col : n - 1;
                const float sc = h2f(scales[(int64_t)colc * nbk + blk]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[i][j][r] += sc * bacc[i][j][r];
                        bacc[i][j][r] = 0.0f;
                    }
            }
        }
    }
    // accumulator layout of a 32x32 tile: value r of lane l is
    // row 8*(r/4) + 4*(l/32) + (r%4), column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (rr < m && col < n) y[(int64_t)rr * n + col] = acc[i][j][r];
            }
        }
}

// Pipelined prompt product for large m.  Workgroup tile: 256 rows of X by 128
// weight rows, K advanced 64 at a time; 8 waves, each a 64x64 block of 2x2
// v_mfma_f32_32x32x16_bf16 tiles.  Per step s the workgroup
//   - copies the X tile of step s + 2 to LDS with direct global -> LDS copies
//     (three X buffers) and requests the code dwords of step s + 2;
//   - runs the matrix cores on step s (X buffer s % 3, level buffer s % 2);
//   - decodes the codes of step s + 1 into the other level buffer: thread t
//     takes code dword t % 4 of weight row t / 4 (16 weights), builds its bit
//     planes (planes_of), transposes them to per-group byte order and turns
//     P = (level + 7) / 2 into bf16 bits with two byte-permute lookups;
//   - at the end of each 128-block adds scale * (block sum) to the result.
// LDS rows are 128 bytes; 16-byte chunk c of row r sits at c ^ ((r / 2) & 7),
// so that the 16 rows an operand read touches at once fall on distinct banks.
constexpr int Q2_BM = 256, Q2_BN = 128, Q2_BK = 64;
constexpr int Q2_XBYTES = Q2_BM * Q2_BK * 2, Q2_WBYTES = Q2_BN * Q2_BK * 2;

__device__ __forceinline__ int q2_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(512) void k_qgemm_v2(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const uint16_t* __restrict__ x, int m,
                                                  float* __restrict__ y, int tiles_n, int remap) {
    // one object per buffer, and the step loop unrolled by 6 so that every
    // access names its buffer statically: the compiler then sees that the
    // direct copies in flight never touch the buffers being read or written
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];      // X, 256 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs2[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[Q2_WBYTES];      // levels, 128 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t ws1[Q2_WBYTES];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // tiles of one XCD are consecutive in (n, m) order, so that they share X rows in L2
    int t = blockIdx.x;
    if (remap) t = (t & 7) * (gridDim.x >> 3) + (t >> 3);
    const int n0 = (t % tiles_n) * Q2_BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7, steps = k / Q2_BK;

    // X copies: wave w, copy i covers slots (4 w + i) * 64 + lane; slot j is
    // row j / 8, chunk position j % 8, which holds logical chunk q2_chunk(row, j % 8)
    const uint16_t* xtile = x + (int64_t)m0 * k;
    int xoff[4];                                        // element offsets from row m0 (< 256 k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (4 * wave + i) * 64 + lane;
        const int r = j >> 3, c = q2_chunk(r, j & 7);
        const int gr = m0 + r < m ? r : m - 1 - m0;
        xoff[i] = gr * k + 8 * c;
    }
    auto copy_x = [&](int st, uint8_t* dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(xtile + xoff[i] + st * Q2_BK, dst + (4 * wave + i) * 1024, 16, 0, 0);
    };
    // codes: thread t takes dword t % 4 of weight row t / 4 of the step
    const int nr = tid >> 2, dm = tid & 3;
    const int wrow = n0 + nr < n ? n0 + nr : n - 1;
    const uint32_t* csrc = reinterpret_cast<const uint32_t*>(codes + (int64_t)wrow * kg) + dm;

    uint32_t dprev = 0;                                 // this thread's dword of the previous step
    auto decode = [&](bool second_half, uint32_t d, uint8_t* wdst) {
        const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x111, 0xf, 0xf, true);      // lane - 1
        const uint32_t back = (uint32_t)__builtin_amdgcn_mov_dpp((int)dprev, 0x103, 0xf, 0xf, true);  // lane + 3
        const uint32_t dp = dm != 0 ? left : (second_half ? back : 0u);   // nothing before a block start
        dprev = d;
        uint32_t P[4];
        planes_of(d, dp, P);
        // byte transpose: Qg holds P of weights 4 g .. 4 g + 3
        const uint32_t t0 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
        const uint32_t u0 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);
        const uint32_t u1 = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
        const uint32_t Q[4] = {__builtin_amdgcn_perm(u0, t0, 0x05040100u), __builtin_amdgcn_perm(u0, t0, 0x07060302u),
                               __builtin_amdgcn_perm(u1, t1, 0x05040100u), __builtin_amdgcn_perm(u1, t1, 0x07060302u)};
        // bf16 of 2 P - 7 for P = 0..7: low bytes E0 A0 40 80 80 40 A0 E0,
        // high bytes C0 C0 C0 BF 3F 40 40 40
        uint32_t o[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t lo = __builtin_amdgcn_perm(0xE0A04080u, 0x8040A0E0u, Q[g]);
            const uint32_t hi = __builtin_amdgcn_perm(0x4040403Fu, 0xBFC0C0C0u, Q[g]);
            o[2 * g] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            o[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
        uint8_t* row = wdst + nr * 128;
        *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    };

    f32x16 acc[2][2], bacc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[i][j][r] = 0.0f; bacc[i][j][r] = 0.0f; }
    int scol[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + (lane & 31);
        scol[j] = col < n ? col : n - 1;
    }

    // prologue: codes and X of steps 0 and 1, levels of step 0
    const uint32_t c0 = csrc[0];
    copy_x(0, xs0);
    const int s1 = steps > 1 ? 1 : 0;
    uint32_t c1 = csrc[4 * s1];
    copy_x(s1, xs1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    decode(false, c0, ws0);
    __syncthreads();

    uint32_t sc_cur[2] = {0, 0};                        // fp16 bits, one register each
    // Step st = 6 i + J uses X buffer J % 3 and level buffer J % 2.  Each
    // step requests the codes and X copies of step st + 2 and, at a block
    // start, the block's scales; past the last step the requests repeat the
    // last step into a buffer nobody reads again, so that every step makes
    // the same number of requests and the waits below have fixed counts.
    auto body = [&](auto J, int st) {
        constexpr int j6 = decltype(J)::value;
        uint8_t* xcur = j6 % 3 == 0 ? xs0 : j6 % 3 == 1 ? xs1 : xs2;
        uint8_t* xnext2 = j6 % 3 == 0 ? xs2 : j6 % 3 == 1 ? xs0 : xs1;
        uint8_t* wcur = j6 % 2 == 0 ? ws0 : ws1;
        uint8_t* wnext = j6 % 2 == 0 ? ws1 : ws0;
        constexpr bool half2 = (j6 & 1) != 0;                   // second half of a 128-block
        const int sn = st + 2 < steps ? st + 2 : steps - 1;
        const uint32_t c2 = csrc[4 * sn];
        copy_x(sn, xnext2);
        if (!half2)
#pragma unroll
            for (int j = 0; j < 2; ++j) sc_cur[j] = scales[(int64_t)scol[j] * nbk + (st >> 1)];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 64 * wm + 32 * i + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8*>(xcur + r * 128 + 16 * q2_chunk(r, c));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 64 * wn + 32 * j + (lane & 31);
                b[j] = *reinterpret_cast<const bf16x8*>(wcur + r * 128 + 16 * q2_chunk(r, c));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], bacc[i][j], 0, 0, 0);
        }
        // everything but this step's requests (5, or 7 with scales) has
        // landed: the codes of step st + 1 and, for the barrier below, its X
        // copies
        if (half2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(7));
        if (st + 1 < steps) decode(!half2, c1, wnext);           // levels of step st + 1
        c1 = c2;
        if (half2) {                                            // end of a 128-block
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float sc = h2f((uint16_t)sc_cur[j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[i][j][r] += sc * bacc[i][j][r];
                        bacc[i][j][r] = 0.0f;
                    }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);                     // lgkmcnt(0): level writes, operand reads
        __builtin_amdgcn_s_barrier();
    };
    for (int st = 0; st < steps; st += 6) {                     // steps is even (k % 128 == 0)
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
        if (st + 2 >= steps) break;
        body(std::integral_constant<int, 2>(), st + 2);
        body(std::integral_constant<int, 3>(), st + 3);
        if (st + 4 >= steps) break;
        body(std::integral_constant<int, 4>(), st + 4);
        body(std::integral_constant<int, 5>(), st + 5);
    }
    // value r of lane l of a 32x32 tile: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 64 * wn + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) y[(int64_t)row * n + col] = acc[i][j][r];
            }
        }
}

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(PG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return PG_OK;
}

}  // namespace

int launch_decode(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, float* w,
                  pg_stream_t s) {
    const int64_t total = n * (k / 4);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_decode, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)s, codes, scales, total,
                       (int)(k / 4), w);
    return hip_check(hipGetLastError(), "pg_decode launch");
}

int launch_fwht(const void* x, int in_dt, void* y, int out_dt, const uint8_t* sign_bits, int64_t rows,
                int64_t k, uint32_t flags, pg_stream_t s) {
    if (rows > 65535) return fail(PG_ERR_UNSUPPORTED, "rows > 65535");
    const dim3 grid((unsigned)((k / 128 + 3) / 4), (unsigned)rows);
    hipLaunchKernelGGL(k_fwht, grid, dim3(256), 0, (hipStream_t)s, x, in_dt, y, out_dt, sign_bits, (int)k, flags,
                       (int64_t)q16_row_bytes(k));
    return hip_check(hipGetLastError(), "pg_fwht_rotate launch");
}

namespace {

template <int BS>
int launch_q16_bs(int R, int W, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                  const uint8_t* xq, int stride, int batch, float* y, hipStream_t st) {
    const int rows_per_wg = 8 * R;
    const dim3 grid((unsigned)((n + rows_per_wg - 1) / rows_per_wg));
    const Q16Layout L = q16_layout((int)k, W, BS);
    const size_t lds = (size_t)W * L.wave_bytes + (size_t)W * 8 * R * BS * 4;
    if (R == 2)
        hipLaunchKernelGGL((k_qgemv_q16<BS, 2>), grid, dim3(64 * W), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y);
    else
        hipLaunchKernelGGL((k_qgemv_q16<BS, 1>), grid, dim3(64 * W), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y);
    return hip_check(hipGetLastError(), "pg_qgemv launch");
}

}  // namespace

int launch_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                 int x_dt, int batch, float* y, pg_stream_t s) {
    if (x_dt == PG_Q16) {
        const int stride = (int)q16_row_bytes(k);
        // rows per workgroup 8*R; waves per workgroup W split each row's
        // 64-weight chunks, chosen so that the launch has about 2048+ waves
        // while every lane still gets at least one chunk
        int R = 1;
        const int64_t wgs = (n + 7) / 8;
        int W = 1;
        while (W < 8 && wgs * W < 2048 && (k / 64) >= 16 * W) W *= 2;
        const char* env = getenv("PG_QGEMV_SHAPE");          // development override "R,W"
        if (env) { int a = 0, b = 0; if (sscanf(env, "%d,%d", &a, &b) == 2 && (a == 1 || a == 2) && (b == 1 || b == 2 || b == 4 || b == 8)) { R = a; W = b; } }
        // batch rows per pass: the staged activations fit the LDS budget
        const size_t budget = 96 * 1024;
        int bs = 1;
        while (bs < 8 && bs < batch && (size_t)W * q16_layout((int)k, W, 2 * bs).wave_bytes + (size_t)W * 8 * R * 2 * bs * 4 <= budget) bs *= 2;
        if ((size_t)W * q16_layout((int)k, W, 1).wave_bytes + (size_t)W * 8 * R * 4 > budget)
            return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the PG_Q16 path", (long long)k);
        hipStream_t st = (hipStream_t)s;
        const uint8_t* xq = (const uint8_t*)x;
        if (bs >= 8) return launch_q16_bs<8>(R, W, codes, scales, n, k, xq, stride, batch, y, st);
        if (bs >= 4) return launch_q16_bs<4>(R, W, codes, scales, n, k, xq, stride, batch, y, st);
        if (bs >= 2) return launch_q16_bs<2>(R, W, codes, scales, n, k, xq, stride, batch, y, st);
        return launch_q16_bs<1>(R, W, codes, scales, n, k, xq, stride, batch, y, st);
    }
    // activations of a tile of batch rows live in LDS as fp32 (<= 64 KiB)
    const int64_t per_row = k * 4;
    int bt = (int)(65536 / per_row);
    if (bt < 1) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the batch path", (long long)k);
    const dim3 grid((unsigned)((n + 31) / 32));
    hipStream_t st = (hipStream_t)s;
    if (bt >= 8 && batch > 4) {
        hipLaunchKernelGGL(k_qgemv_v1<8>, grid, dim3(256), 8 * per_row, st, codes, scales, (int)n, (int)k, x, x_dt, batch, y);
    } else if (bt >= 4 && batch > 2) {
        hipLaunchKernelGGL(k_qgemv_v1<4>, grid, dim3(256), 4 * per_row, st, codes, scales, (int)n, (int)k, x, x_dt, batch, y);
    } else if (bt >= 2 && batch > 1) {
        hipLaunchKernelGGL(k_qgemv_v1<2>, grid, dim3(256), 2 * per_row, st, codes, scales, (int)n, (int)k, x, x_dt, batch, y);
    } else {
        hipLaunchKernelGGL(k_qgemv_v1<1>, grid, dim3(256), per_row, st, codes, scales, (int)n, (int)k, x, x_dt, batch, y);
    }
    return hip_check(hipGetLastError(), "pg_qgemv launch");
}

namespace {

template <int XDT, int XG, int RS, int BTM>
int launch_fused_t(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                   const void* x, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                   hipStream_t st) {
    const dim3 grid((unsigned)((n + S.R - 1) / S.R));
    const int esz = XDT == PG_F32 ? 4 : 2;
    const int tile = fused_loops(RS, BTM) ? batch : S.BT;  // rows handed to one launch
    for (int b0 = 0; b0 < batch; b0 += tile) {
        const int bt = batch - b0 < tile ? batch - b0 : tile;
        const void* xb = (const uint8_t*)x + (int64_t)b0 * ldx * esz;
        hipLaunchKernelGGL((k_rot_qgemv<XDT, XG, RS, BTM>), grid, dim3(64 * S.W), fused_lds_bytes((int)k, esz, S),
                           st, codes, scales, (int)n, (int)k, xb, ldx, sign_bits, flags, bt, y + (int64_t)b0 * n,
                           S.R, S.CG, S.RP, S.BT);
        const int rc = hip_check(hipGetLastError(), "pg_rot_qgemv launch");
        if (rc != PG_OK) return rc;
    }
    return PG_OK;
}

// (rows per lane, batch rows per launch) combinations that fit the register
// budget (RS * BTM <= 32, and RS <= 2 for 8 rows)
template <int XDT, int XG>
int launch_fused_rs(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                    const void* x, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                    hipStream_t st) {
#define PG_FUSED(RS_, BTM_) return launch_fused_t<XDT, XG, RS_, BTM_>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st)
    if (S.BTM == 1) {                  // rows per lane as exact as possible: each one costs a full decode
        if (S.RS <= 1) PG_FUSED(1, 1);
        if (S.RS <= 2) PG_FUSED(2, 1);
        if (S.RS <= 3) PG_FUSED(3, 1);
        if (S.RS <= 4) PG_FUSED(4, 1);
        if (S.RS <= 5) PG_FUSED(5, 1);
        if (S.RS <= 6) PG_FUSED(6, 1);
        if (S.RS <= 7) PG_FUSED(7, 1);
        if (S.RS <= 8) PG_FUSED(8, 1);
        if (S.RS <= 10) PG_FUSED(10, 1);
        if (S.RS <= 12) PG_FUSED(12, 1);
        if (S.RS <= 14) PG_FUSED(14, 1);
        PG_FUSED(16, 1);
    }
    if (S.BTM == 2) {
        if (S.RS <= 8) PG_FUSED(8, 2);
        PG_FUSED(16, 2);
    }
    if (S.BTM == 4) {
        if (S.RS <= 2) PG_FUSED(2, 4);
        if (S.RS <= 4) PG_FUSED(4, 4);
        PG_FUSED(8, 4);
    }
    if (S.RS <= 1) PG_FUSED(1, 8);
    PG_FUSED(2, 8);
#undef PG_FUSED
}

int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

}  // namespace

// Launch shape of the fused stage: about one workgroup per CU, each with
// all of its rows' codes in registers (at most 16 rows per lane).
int fused_shape(int64_t n, int64_t k, int batch, FusedShape* out) {
    FusedShape S;
    S.W = 8;                                           // the kernel assumes 512 threads
    int R_req = 0;
    if (const char* e = getenv("PG_FUSED_ROWS")) {     // rows per workgroup, for tuning sweeps
        const int r2 = atoi(e);
        if (r2 > 0) R_req = r2;
    }
    const int nchunk = (int)(k / 64), nbk = (int)(k / 128);
    S.CG = (nchunk + 7) / 8;
    if (S.CG > 8 * S.W) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    S.RP = 8 * S.W / S.CG;
    S.XG = (int)((k / 8 + 64 * S.W - 1) / (64 * S.W));   // 8-value groups of x per thread
    if (k / 32 > 64 * S.W || S.XG > 4)
        return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    (void)nbk;
    const int64_t cus = compute_units();
    int64_t R = R_req > 0 ? R_req : (n + cus - 1) / cus;
    if (R > 16 * S.RP) R = 16 * S.RP;                      // at most 16 rows per lane
    if (R > n) R = n;
    S.R = (int)R;
    S.RS = (S.R + S.RP - 1) / S.RP;
    // batch rows per tile: as many as the LDS holds, up to the template's bound
    // BTM (registers: RS * BTM <= 32, RS <= 2 for 8 rows); with fewer rows
    // per tile than the batch, the kernel loops over tiles itself where its
    // registers allow (fused_loops), else one launch per tile
    const size_t budget = 150 * 1024;
    int bt_lds = 1;                                    // rows of x the LDS holds at once
    for (;;) {
        FusedShape T = S;
        T.BTM = T.BT = bt_lds + 1;
        if (bt_lds >= 8 || fused_lds_bytes((int)k, 4, T) > budget) break;
        ++bt_lds;
    }
    const int t = batch < bt_lds ? batch : bt_lds;
    S.BTM = batch <= 1 ? 1 : S.RS <= 2 ? (t > 4 ? 8 : 4) : S.RS <= 4 ? 4 : S.RS <= 8 ? (t <= 2 ? 2 : 4) : 2;
    S.BT = t < S.BTM ? t : S.BTM;
    if (fused_lds_bytes((int)k, 4, S) > budget) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    *out = S;
    return PG_OK;
}

int launch_rot_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                     int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                     pg_stream_t s) {
    FusedShape S;
    const int rc = fused_shape(n, k, batch, &S);
    if (rc != PG_OK) return rc;
    hipStream_t st = (hipStream_t)s;
    if (x_dt == PG_F32) {
        if (!(flags & PG_FLAG_RMSNORM))
            return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv: fp32 input needs PG_FLAG_RMSNORM (its rotation runs in fp16)");
        if (S.XG <= 1) return launch_fused_rs<PG_F32, 1>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
        if (S.XG <= 2) return launch_fused_rs<PG_F32, 2>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
        return launch_fused_rs<PG_F32, 4>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    }
    if (S.XG <= 1) return launch_fused_rs<PG_F16, 1>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    if (S.XG <= 2) return launch_fused_rs<PG_F16, 2>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    return launch_fused_rs<PG_F16, 4>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
}

int launch_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x,
                 int64_t m, float* y, pg_stream_t s) {
    const int64_t tn = (n + Q2_BN - 1) / Q2_BN, tm = (m + Q2_BM - 1) / Q2_BM;
    // the pipelined kernel is the product; PG_QGEMM_KERNEL=1 selects the
    // plain one-buffer kernel (kept as a second implementation for tests)
    const char* e = getenv("PG_QGEMM_KERNEL");
    if (!(e && atoi(e) == 1)) {
        if (tn * tm > (1 << 30)) return fail(PG_ERR_UNSUPPORTED, "m too large");
        const int remap = (tn * tm) % 8 == 0 ? 1 : 0;
        hipLaunchKernelGGL(k_qgemm_v2, dim3((unsigned)(tn * tm)), dim3(512), 0, (hipStream_t)s, codes, scales,
                           (int)n, (int)k, x, (int)m, y, (int)tn, remap);
        return hip_check(hipGetLastError(), "pg_qgemm launch");
    }
    const dim3 grid((unsigned)((n + QG_BN - 1) / QG_BN), (unsigned)((m + QG_BM - 1) / QG_BM));
    if (grid.y > 65535) return fail(PG_ERR_UNSUPPORTED, "m too large");
    hipLaunchKernelGGL(k_qgemm_v1, grid, dim3(256), 0, (hipStream_t)s, codes, scales, (int)n, (int)k, x, (int)m, y);
    return hip_check(hipGetLastError(), "pg_qgemm launch");
}

}  // namespace pg
