// Fused stage of a stack for batch 2..8 on the gfx950 matrix cores: RMS
// normalisation, the random Hadamard rotation and the product y = W~ . R . n(x)
// of every batch row in one launch.  The rotation runs on the f16 matrix
// cores as in k_rot_qgemv; the product is the int8 block step of pg_mma.h,
// so the activations are quantised to 16 bits with one scale per 128-block
// (the block's largest value), held in LDS as signed digit pairs.
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode,
// random Hadamard rotation); bit layout: include/pingala.h.
#include "pg_fused.h"
#include "pg_mma.h"

namespace pg {
namespace {

constexpr int RQ_MAX_BATCH = 8;               // one wave per batch row while staging
constexpr int RQ_MAX_K = 4096;                // 8 groups of 8 values per lane; one row of 32 blocks per tile
constexpr int RQ_MAX_ITEMS = 256;             // items per workgroup: at most 8 code tiles per wave
constexpr size_t RQ_LDS_LIMIT = 160 * 1024;

// LDS of one launch
struct RqLayout {
    size_t xh, tab, yw, swt, ctile, total;
};
__host__ __device__ inline RqLayout rq_layout(int k, int R, int batch) {
    const int nbk = k / 128, nbk4 = (nbk + 3) & ~3;
    RqLayout L;
    L.xh = 0;                                                         // [batch][nbk][272]: fp16 blocks, then digits
    L.tab = L.xh + (size_t)batch * nbk * FS_XPITCH;                  // [nbk][16] float2
    L.yw = L.tab + (size_t)nbk * 16 * 8;                             // [8][R][16] float
    L.swt = L.yw + (size_t)8 * R * 16 * 4;                           // [R][nbk4] fp16 bits
    L.ctile = L.swt + (((size_t)R * nbk4 * 2 + 15) & ~(size_t)15);   // [8][16][144]
    L.total = L.ctile + (size_t)8 * MMA_TILE_BYTES;
    return L;
}

// Workgroup of 8 waves over R = 16 NRT rows and all k columns:
//   1. requests: wave w reads batch row w of x (8-value groups lane + 64 u)
//      and its sign bytes, then the weight scales of the rows and the code
//      tiles (16 rows x 4 blocks, as k_qgemv_mma), which stay in flight;
//   2. wave w sums its row's squares (RMS norm) and stages the normalised,
//      sign-flipped fp16 blocks in LDS;
//   3.-5. wave w < batch, after a barrier: the rotation tiles of row w (all
//      four quarters of its 32-block tile) on the f16 matrix cores, kept in
//      registers; the block maxima in registers; q = rint(v * 32512 / block
//      max) as digits hi = floor((q + 128) / 256), lo = q - 256 hi (signed),
//      written over the row's fp16 blocks in code-dword plane order; the
//      block sums of q; the row's table entries (2 sx, -7 sx sum q);
//   6. after a barrier, the items of k_qgemv_mma, digits from LDS;
//   7. the waves' sums in wave order.
// Every reduction has a fixed order or is exact (integer adds, maxima), so
// the result does not depend on timing.
template <int XDT, int TPW>
__global__ __launch_bounds__(512) void k_rot_qmma(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales,
                                                  const void* __restrict__ x,
                                                  const uint8_t* __restrict__ sign_bits,
                                                  float* __restrict__ y, int n, int k, int ldx32, uint32_t bword) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // 14 argument dwords, all preloaded into scalar registers (launch_rq_x)
    const int R = (int)(bword & 0xffffu), batch = (int)((bword >> 16) & 0xffu);
    const uint32_t flags = ((bword >> 24) & 1u) ? (uint32_t)PG_FLAG_RMSNORM : 0u;
    const int64_t ldx = ldx32;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = k >> 2, nbk = k >> 7, nbk4 = (nbk + 3) & ~3, tpr = nbk4 >> 2, ngr = k >> 3;
    const int row0 = blockIdx.x * R;
    const int tiles = (R >> 4) * tpr;
    const int r16 = lane & 15, kq = lane >> 4;
    const RqLayout Ly = rq_layout(k, R, batch);
    const size_t xrowb = (size_t)nbk * FS_XPITCH;            // LDS bytes per batch row of blocks
    uint8_t* xh = lds + Ly.xh;
    float2* tab = reinterpret_cast<float2*>(lds + Ly.tab);
    float* yw = reinterpret_cast<float*>(lds + Ly.yw);
    float* ywv = yw + (size_t)wave * R * 16;
    uint16_t* swt = reinterpret_cast<uint16_t*>(lds + Ly.swt);
    uint8_t* ctile = lds + Ly.ctile + (size_t)wave * MMA_TILE_BYTES;
    const bool norm = (flags & PG_FLAG_RMSNORM) != 0;
    float rk = 1.0f / (float)k;
    asm volatile("" : "+v"(rk));                      // computed here, before any wait (the
                                                      // compiler would sink it past the barrier)
    constexpr int esz = XDT == PG_F32 ? 4 : 2;

    // ---- 1. requests (past the end: repeats of valid addresses)
    constexpr int KV = RQ_MAX_K / 512;                       // 8-value groups per lane, at most
    const bool rowon = wave < batch;                         // uniform
    const uint8_t* xr = reinterpret_cast<const uint8_t*>(x) + (int64_t)(rowon ? wave : 0) * ldx * esz;
    float xv[KV][8];
    uint32_t sgb[KV];
    if (rowon)                                               // waves past the batch load no row
#pragma unroll
    for (int u = 0; u < KV; ++u) {
        if (64 * u >= ngr) continue;                         // uniform: no group of this round in the row
        const int g = lane + 64 * u, gc = g < ngr ? g : ngr - 1;
        if constexpr (XDT == PG_F32) {
            const float4 v0 = *reinterpret_cast<const float4*>(xr + 32 * gc);
            const float4 v1 = *reinterpret_cast<const float4*>(xr + 32 * gc + 16);
            xv[u][0] = v0.x; xv[u][1] = v0.y; xv[u][2] = v0.z; xv[u][3] = v0.w;
            xv[u][4] = v1.x; xv[u][5] = v1.y; xv[u][6] = v1.z; xv[u][7] = v1.w;
        } else {
            const uint4 w = *reinterpret_cast<const uint4*>(xr + 16 * gc);
            const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xv[u][2 * t] = h2f((uint16_t)(w4[t] & 0xffffu));
                xv[u][2 * t + 1] = h2f((uint16_t)(w4[t] >> 16));
            }
        }
        sgb[u] = sign_bits[gc];
    }
    constexpr int SWU = TPW;                                 // weight scales per thread: R nbk4 <= 512 TPW
    const int nsw = R * nbk;
    uint32_t swv[SWU];
#pragma unroll
    for (int u = 0; u < SWU; ++u) {
        const int e = tid + 512 * u, ec = e < nsw ? e : nsw - 1;
        const int r = ec / nbk;
        const int row = row0 + r < n ? row0 + r : n - 1;
        swv[u] = scales[(int64_t)row * nbk + (ec - r * nbk)];
    }
    asm volatile("" ::: "memory");
    // wave w takes tiles w, w + 8, ... (at most TPW; the waves' counts differ
    // by one at most); its row tiles never decrease, so a running sum per row
    // tile is enough
    const int mine = wave < tiles ? (tiles - wave + 7) >> 3 : 0;     // uniform
    auto tile_of = [&](int i) { const int t = wave + 8 * i; return t < tiles ? t : tiles - 1; };
    mma_v4u ct[TPW][2];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = tile_of(i);
        const int rt = t / tpr, tb = t - rt * tpr;
        int off = 128 * tb + 16 * (lane & 7);
        if (off > kg - 16) off = kg - 16;                    // past the row's end (nbk % 4 != 0): unused
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * rt + 8 * h + (lane >> 3);
            const int row = row0 + r < n ? row0 + r : n - 1;
            ct[i][h] = *reinterpret_cast<const mma_v4u*>(codes + (int64_t)row * kg + off);
        }
    }
    asm volatile("" ::: "memory");

    // ---- 2. LDS set-up; normalised, sign-flipped fp16 blocks of row `wave`
    for (int e = tid; e < nbk * 16; e += 512) tab[e] = make_float2(0.0f, 0.0f);   // batch slots past the batch
#pragma unroll
    for (int u = 0; u < SWU; ++u) {                          // past the end: the last entry again, same place
        const int e = tid + 512 * u, ec = e < nsw ? e : nsw - 1;
        const int r = ec / nbk;
        swt[r * nbk4 + (ec - r * nbk)] = (uint16_t)swv[u];
    }
    for (int e = lane; e < R * 4; e += 64) reinterpret_cast<float4*>(ywv)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rowon) {
        float inv = 1.0f;
        if (norm) {
            float ss = 0.0f;
#pragma unroll
            for (int u = 0; u < KV; ++u)
                if (lane + 64 * u < ngr)
#pragma unroll
                    for (int t = 0; t < 8; ++t) ss += xv[u][t] * xv[u][t];
            ss = wave_sum(ss);
            inv = rms_inv(ss, rk);
        }
#pragma unroll
        for (int u = 0; u < KV; ++u) {
            const int g = lane + 64 * u;
            if (g < ngr) {
                uint32_t hw[4];
#pragma unroll
                for (int t = 0; t < 8; t += 2) {
                    uint32_t h0 = f2h(norm ? xv[u][t] * inv : xv[u][t]);
                    uint32_t h1 = f2h(norm ? xv[u][t + 1] * inv : xv[u][t + 1]);
                    h0 ^= ((sgb[u] >> t) & 1u) << 15;
                    h1 ^= ((sgb[u] >> (t + 1)) & 1u) << 15;
                    hw[t >> 1] = h0 | (h1 << 16);
                }
                *reinterpret_cast<uint4*>(xh + (size_t)wave * xrowb + (g >> 4) * FS_XPITCH + (g & 15) * 16) =
                    make_uint4(hw[0], hw[1], hw[2], hw[3]);
            }
        }
    }
    lds_barrier();                                           // LDS only: the code requests stay in flight

    // ---- 3.-5. wave w < batch: the rotation tiles of batch row w, all four
    // quarters from one read of each block's B operand (their A operands
    // differ only in sign); the block maxima and sums of q in registers; the
    // digits written over the row's fp16 blocks (only this wave reads them)
    // and the row's table entries (2 sx, -7 sx sum q), sx = max 2^-3.5 / 32512
    uint32_t apat[2][4];
    fs_apat(lane, apat);
    const int blk = lane & 31;
    const bool bok = blk < nbk;
    if (wave < batch) {                                      // uniform
        const int b = wave;
        f32x16 acc_r[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_r[mt][r] = 0.0f;
        const uint8_t* xb = xh + (size_t)b * xrowb + (bok ? blk : 0) * FS_XPITCH + 16 * (lane >> 5);
        uint4 bv[8];                                         // the block's B operands, one LDS wait
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const uint4 v = *reinterpret_cast<const uint4*>(xb + 32 * st);
            bv[st] = bok ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const uint32_t* av = apat[st & 1];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint32_t fl = (__builtin_popcount(mt & (st >> 1)) & 1) ? 0x80008000u : 0u;
                const uint4 aw = make_uint4(av[0] ^ fl, av[1] ^ fl, av[2] ^ fl, av[3] ^ fl);
                acc_r[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(fs_f16x8, aw),
                                                                   __builtin_bit_cast(fs_f16x8, bv[st]), acc_r[mt], 0, 0, 0);
            }
        }
        // block maximum: a lane holds 16 values of each quarter of block
        // lane % 32, the lane pair (l, l + 32) all 128
        float mx = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(acc_r[mt][r]));
        mx = fmaxf(mx, xor_lane32(mx, lane));
        const float s = mx > 0.0f ? (float)Q16_MAXQ * __builtin_amdgcn_rcpf(mx) : 0.0f;
        int qsum = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            // value 16 p + 4 g + j of the block at byte 32 p + 4 j + g (hi), + 16 (lo):
            // accumulator row 8 i + 4 h + r is part 2 mt + i / 2, position 2 (i % 2) + h
            uint8_t* dq = xh + (size_t)b * xrowb + (bok ? blk : 0) * FS_XPITCH + 64 * mt + 4 * (lane >> 5);
            int shi = 0, slo = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t bits[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    bits[r] = __builtin_bit_cast(uint32_t, fmaf(acc_r[mt][4 * i + r], s, 12582912.0f + 128.0f));
                // the low 16 bits are q + 128: hi = its high byte, lo = its low byte - 128
                const uint32_t t01 = __builtin_amdgcn_perm(bits[1], bits[0], 0x05040100u);
                const uint32_t t23 = __builtin_amdgcn_perm(bits[3], bits[2], 0x05040100u);
                const uint32_t dl = __builtin_amdgcn_perm(t23, t01, 0x06040200u) ^ 0x80808080u;
                const uint32_t dh = __builtin_amdgcn_perm(t23, t01, 0x07050301u);
                shi = __builtin_amdgcn_sdot4((int)dh, 0x01010101, shi, false);
                slo = __builtin_amdgcn_sdot4((int)dl, 0x01010101, slo, false);
                if (bok) {
                    uint8_t* dd = dq + 32 * (i >> 1) + 8 * (i & 1);
                    *reinterpret_cast<uint32_t*>(dd) = dh;
                    *reinterpret_cast<uint32_t*>(dd + 16) = dl;
                }
            }
            qsum += 256 * shi + slo;
        }
        qsum += __builtin_bit_cast(int, xor_lane32(__builtin_bit_cast(float, qsum), lane));
        if (bok && lane < 32) {
            const float sx = mx * (0.08838834764831845f / (float)Q16_MAXQ);
            tab[16 * blk + b] = make_float2(2.0f * sx, -7.0f * sx * (float)qsum);
        }
    }
    lds_barrier();                                           // LDS only: the code requests stay in flight

    // ---- 6. items (as k_qgemv_mma; digits of block blk of batch row b at
    // xh + b xrowb + 272 blk, code dword d's 32 bytes at 32 d)
    const int bcol = r16 < batch ? r16 : 0;
    const uint8_t* drow = xh + (size_t)bcol * xrowb + 64 * kq;
    uint4 dg[2][4];
    float4 tb2[2][2];
    auto blk_of = [&](int m) {
        const int t = tile_of(m >> 2);
        const int bb = 4 * (t - (t / tpr) * tpr) + (m & 3);
        return bb < nbk ? bb : nbk - 1;
    };
    auto request = [&](int m, int slot) {
        const int bb = blk_of(m);
        const uint4* p = reinterpret_cast<const uint4*>(drow + FS_XPITCH * bb);
        dg[slot][0] = p[0];
        dg[slot][1] = p[1];
        dg[slot][2] = p[2];
        dg[slot][3] = p[3];
        const float4* tq = reinterpret_cast<const float4*>(tab + 16 * bb + 4 * kq);
        tb2[slot][0] = tq[0];
        tb2[slot][1] = tq[1];
    };
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    request(0, 0);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        if (i < mine) {                                      // uniform
            const int t = tile_of(i);
            const int rt = t / tpr, tb = t - rt * tpr;
            mma_put_tile(ctile, lane, ct[i][0], ct[i][1]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 4 * i + j;
                request(m + 1, (m + 1) & 1);
                const int bb = 4 * tb + j;
                const float sw = bb < nbk ? h2f(swt[(16 * rt + r16) * nbk4 + bb]) : 0.0f;   // uniform test
                mma_block(ctile, r16, kq, j, dg[m & 1], tb2[m & 1], sw, acc);
            }
            *reinterpret_cast<float4*>(ywv + 16 * (16 * rt + r16) + 4 * kq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            if (i + 1 < TPW && tile_of(i + 1) / tpr != rt) {  // uniform: a new row tile starts from zero
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
            }
        }
    }
    lds_barrier();                                           // LDS only: the code requests stay in flight

    // ---- 7. the waves' sums in wave order
    for (int e = tid; e < R * batch; e += 512) {
        const int b = e / R, r = e - b * R;
        if (row0 + r >= n) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) v += yw[((size_t)w * R + r) * 16 + b];
        y[(int64_t)b * n + row0 + r] = v;
    }
}

template <int XDT>
int launch_rq_x(int tpw, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y, int R, size_t lds,
                hipStream_t st) {
    const dim3 grid((unsigned)((n + R - 1) / R));
    // R (16 bits), the batch (8) and the RMS flag in one dword, ldx in 32
    // bits: with 14 argument dwords the hardware preloads every argument into
    // scalar registers (the build asks for preloading; the argument-segment
    // pointer takes 2 of the 16 user registers), so no wave waits for a
    // scalar load before its first requests
    if (R >= 65536 || batch > 255 || ldx < 0 || ldx > 0x7fffffff)
        return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv: shape n=%lld k=%lld ldx=%lld out of the kernel's range",
                    (long long)n, (long long)k, (long long)ldx);
    const uint32_t bword = (uint32_t)R | ((uint32_t)batch << 16) | ((flags & PG_FLAG_RMSNORM) ? 1u << 24 : 0u);
#define PG_RQ(T) hipLaunchKernelGGL((k_rot_qmma<XDT, T>), grid, dim3(512), lds, st, codes, scales, x, sign_bits, y, \
                                    (int)n, (int)k, (int)ldx, bword)
    switch (tpw) {
        case 1: PG_RQ(1); break;
        case 2: PG_RQ(2); break;
        case 3: PG_RQ(3); break;
        case 4: PG_RQ(4); break;
        case 5: PG_RQ(5); break;
        case 6: PG_RQ(6); break;
        case 7: PG_RQ(7); break;
        default: PG_RQ(8); break;
    }
#undef PG_RQ
    return hip_check(hipGetLastError(), "pg_rot_qgemv launch");
}

}  // namespace

int launch_rot_qmma(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dt,
                    int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y, hipStream_t st) {
    if (batch > RQ_MAX_BATCH || k > RQ_MAX_K || (flags & PG_FLAG_CARRY_STATE)) return PG_ERR_UNSUPPORTED;
    const int cus = compute_units();
    const int nbk4 = (int)((k / 128 + 3) & ~3);
    int64_t per = (n + cus - 1) / cus;
    int64_t R = 16 * ((per + 15) / 16);
    if (R > 128) R = 128;
    while (R > 16 && (R / 16) * nbk4 > RQ_MAX_ITEMS) R -= 16;
    while (R > 16 && rq_layout((int)k, (int)R, batch).total > RQ_LDS_LIMIT) R -= 16;
    const size_t lds = rq_layout((int)k, (int)R, batch).total;
    if (lds > RQ_LDS_LIMIT || (R / 16) * nbk4 > RQ_MAX_ITEMS) return PG_ERR_UNSUPPORTED;
    const int tpw = (int)(((R / 16) * (nbk4 / 4) + 7) / 8);
    if (x_dt == PG_F32)
        return launch_rq_x<PG_F32>(tpw, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, (int)R, lds, st);
    return launch_rq_x<PG_F16>(tpw, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, (int)R, lds, st);
}

}  // namespace pg
