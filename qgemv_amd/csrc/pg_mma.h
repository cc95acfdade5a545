// The block step shared by the batched products on the gfx950 int8 matrix
// cores (k_qgemv_mma, k_rot_qmma): one 128-block of 16 weight rows against
// up to 16 batch rows of 16-bit activation digits.
//
// v_mfma_i32_16x16x64_i8: D[b][r] += sum_k A[b][k] B[k][r], A = activation
// digits (row b = batch row), B = bit planes P = (level + 7) / 2 of the
// weight rows.  Lane l supplies A row / B column l % 16 and the k slice
// l / 16 (16 bytes) and receives D[4 (l / 16) + i][l % 16], i = 0..3.  Lane
// group kq = l / 16 takes code dwords 2 kq and 2 kq + 1 of the block: the
// product mm = 0, 1 pairs dword 2 kq + mm of every lane group, so two
// products cover the block's 8 dwords.  The digits of code dword d sit in
// plane order (byte 4 j + g is group g, position j; 16 hi digits, then 16 lo
// digits), the order of the planes, so both operands are 16 bytes as stored.
// Per block, exactly in int32,
//   sum level q = 2 (256 H + L) - 7 sum q,  H = sum P hi,  L = sum P lo,
// then y[b][r] += sw[r] * sx[b] * that, in fp32.
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode);
// bit layout: include/pingala.h.
#pragma once
#include "pg_device.h"

namespace pg {
namespace {

typedef int mma_v4i __attribute__((ext_vector_type(4)));
typedef unsigned int mma_v4u __attribute__((ext_vector_type(4)));

// Codes travel in tiles of 16 rows x 4 blocks (128 bytes of each row, one
// cache line), read by eight lanes per row and stored to a small LDS area of
// the wave, from which each lane takes its 8 bytes of a block (reading those
// straight from memory would touch 16 lines per 512 bytes).
constexpr int MMA_CPITCH = 144;              // LDS bytes per row of a code tile (128 + 16)
constexpr int MMA_TILE_BYTES = 16 * MMA_CPITCH;

// the wave's tile to LDS: ct0 holds row lane / 8, ct1 row 8 + lane / 8,
// bytes 16 (lane % 8) .. of the 128 (LDS accesses of a wave run in order)
__device__ __forceinline__ void mma_put_tile(uint8_t* ctile, int lane, mma_v4u ct0, mma_v4u ct1) {
    *reinterpret_cast<mma_v4u*>(ctile + (lane >> 3) * MMA_CPITCH + 16 * (lane & 7)) = ct0;
    *reinterpret_cast<mma_v4u*>(ctile + (8 + (lane >> 3)) * MMA_CPITCH + 16 * (lane & 7)) = ct1;
}

// Block j of the tile in LDS for this lane (weight row r16 = lane % 16,
// lane group kq), with its digit operands d (hi and lo of dwords 2 kq and
// 2 kq + 1), the table entries t = (2 sx, -7 sx sum q) of batch rows
// 4 kq .. 4 kq + 3 and the weight scale sw: adds the block to acc.
__device__ __forceinline__ void mma_block(const uint8_t* ctile, int r16, int kq, int j, const uint4 (&d)[4],
                                          const float4 (&t)[2], float sw, float acc[4]) {
    const uint8_t* cr = ctile + r16 * MMA_CPITCH + 32 * j;
    const uint2 cd = *reinterpret_cast<const uint2*>(cr + 8 * kq);
    const uint32_t pv = *reinterpret_cast<const uint32_t*>(cr + (kq > 0 ? 8 * kq - 4 : 0));
    const uint32_t prev = kq > 0 ? pv : 0u;                  // a block starts the trellis at state 0
    uint32_t P0[4], P1[4];
    planes_of(cd.x, prev, P0);
    planes_of(cd.y, cd.x, P1);
    const mma_v4i b0 = {(int)P0[0], (int)P0[1], (int)P0[2], (int)P0[3]};
    const mma_v4i b1 = {(int)P1[0], (int)P1[1], (int)P1[2], (int)P1[3]};
    mma_v4i H = {0, 0, 0, 0}, L = {0, 0, 0, 0};
    H = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[0]), b0, H, 0, 0, 0);
    L = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[1]), b0, L, 0, 0, 0);
    H = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[2]), b1, H, 0, 0, 0);
    L = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[3]), b1, L, 0, 0, 0);
    const float tx[4] = {t[0].x, t[0].z, t[1].x, t[1].z};
    const float ty[4] = {t[0].y, t[0].w, t[1].y, t[1].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float f = (float)(H[e] * 256 + L[e]);
        acc[e] = fmaf(fmaf(f, tx[e], ty[e]), sw, acc[e]);
    }
}

}  // namespace
}  // namespace pg
