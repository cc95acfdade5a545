// Device helpers shared by the HIP kernels of libpingala (gfx950, wave64):
// number conversions, the decode of one code byte, cross-lane exchanges and
// reductions, the bit planes of a code dword, and waitcnt operands.
//
// Format: P8F v1 ("Pingala-8" landing page, section "How it works": an
// 8-state trellis over groups of 4 weights); bit layout in include/pingala.h.
#pragma once
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
__device__ __forceinline__ int wave_xor(int v) {
    const int lane = threadIdx.x & 63;
    v ^= xor_lane_i<1>(v, lane);
    v ^= xor_lane_i<2>(v, lane);
    v ^= xor_lane_i<4>(v, lane);
    v ^= xor_lane_i<8>(v, lane);
    v ^= __builtin_bit_cast(int, xor_lane16(__builtin_bit_cast(float, v), lane));
    v ^= __builtin_bit_cast(int, xor_lane32(__builtin_bit_cast(float, v), lane));
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

// The stack normalisation's factor for a row of k values whose squares sum
// to ss (rk = 1/k rounded to fp32): the hardware reciprocal square root of
// fma(ss, rk, 1e-6).  Every kernel that normalises calls this, so that n(v) =
// fp16_RNE(v * rms_inv(ss, rk)) has one definition.
__device__ __forceinline__ float rms_inv(float ss, float rk) { return __builtin_amdgcn_rsqf(fmaf(ss, rk, 1e-6f)); }

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

// s_waitcnt operand: at most n vector-memory operations of this wave still
// outstanding, the other counters unrestricted (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(PG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return PG_OK;
}


// Workgroup barrier that waits only for this wave's LDS accesses (not for
// its global loads or direct-to-LDS copies in flight, which __syncthreads'
// fences would wait for).  The builtin barrier alone is no compiler fence:
// the empty asm statements with a memory clobber keep every memory access
// on its side.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// compute units of the current device (cached per device)
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
}  // namespace pg
