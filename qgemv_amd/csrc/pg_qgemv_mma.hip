// Batched product on PG_Q16 activations with the gfx950 int8 matrix cores
// (batch 2..8 of pg_qgemv).  The VALU path (k_qgemv_q16) pays two v_dot4 per
// code dword for every batch row; here the bit planes of a code dword are the
// B operand of v_mfma_i32_16x16x64_i8 and up to 16 batch rows share them, so
// the vector work per weight stays that of the decode.
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode,
// rotation before coding); batched generation is the case the same page's
// section on limits calls weakest.  Bit layout and PG_Q16: include/pingala.h.
#include "pg_mma.h"

namespace pg {
namespace {

// One item = (16 weight rows, one 128-block): the matrix-core block step of
// pg_mma.h, with the PG_Q16 digits of the batch rows as the A operand
// (PG_Q16 chunk 8 blk + d holds code dword d's 16 values in plane order).
//
// Workgroup: 8 waves over R = 16 NRT rows and all k columns, the codes in
// tiles of 16 rows x 4 blocks (pg_mma.h).  Each wave takes a consecutive run of
// tiles (row tile t / (nbk / 4), blocks 4 (t % (nbk / 4)) ..), all requested
// at entry; the weight scales of the workgroup's rows are copied to LDS once.
// The activation digits, which every workgroup reads, are copied to LDS at
// entry when all batch rows fit (STAGE), else read from the L2 an item ahead.
// Each wave adds its items into its own LDS rows [R][16]; the waves' sums
// are added in wave order at the end, so the result does not depend on
// timing.
constexpr int MMA_PITCH_PAD = 16;            // staged digit row: 2k + 16 bytes, so that the 16-byte reads of
                                             // 8 consecutive batch rows fall in distinct banks
constexpr int MMA_STAGE_BYTES = 80 * 1024;   // staged digits, at most (10 chunks of 16 bytes per thread)
constexpr int MMA_MAX_ITEMS = 256;           // items per workgroup: at most 8 tiles of 4 per wave
constexpr size_t MMA_LDS_LIMIT = 160 * 1024;

// LDS of one launch: block table, the waves' partial rows, the weight scales
// of the workgroup's rows, one code tile per wave and (STAGE) the digits
struct MmaLayout {
    size_t tab, yw, swt, ctile, stage, total;
};
__host__ __device__ inline MmaLayout mma_layout(int k, int R, int batch, bool stage) {
    const int nbk = k / 128, nbk4 = (nbk + 3) & ~3;
    MmaLayout L;
    L.tab = 0;                                                       // [nbk][16] float2
    L.yw = L.tab + (size_t)nbk * 16 * 8;                             // [8][R][16] float
    L.swt = L.yw + (size_t)8 * R * 16 * 4;                           // [R][nbk4] fp16 bits
    L.ctile = L.swt + (((size_t)R * nbk4 * 2 + 15) & ~(size_t)15);   // [8][16][144]
    L.stage = L.ctile + (size_t)8 * MMA_TILE_BYTES;                  // [batch][2k + 16]
    L.total = L.stage + (stage ? (size_t)batch * (size_t)(2 * k + MMA_PITCH_PAD) : 0);
    return L;
}

template <int TPW, bool STAGE>
__global__ __launch_bounds__(512) void k_qgemv_mma(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int n, int k,
                                                   const uint8_t* __restrict__ xq, int stride, int batch,
                                                   float* __restrict__ y, int R) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(xq), "s"(stride), "s"(batch), "s"(y), "s"(R));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = k >> 2, nbk = k >> 7, nbk4 = (nbk + 3) & ~3, tpr = nbk4 >> 2;
    const int row0 = blockIdx.x * R;
    const int tiles = (R >> 4) * tpr;
    const int r16 = lane & 15, kq = lane >> 4;
    const MmaLayout Ly = mma_layout(k, R, batch, STAGE);
    float2* tab = reinterpret_cast<float2*>(lds + Ly.tab);
    float* yw = reinterpret_cast<float*>(lds + Ly.yw);
    float* ywv = yw + (size_t)wave * R * 16;
    uint16_t* swt = reinterpret_cast<uint16_t*>(lds + Ly.swt);
    uint8_t* ctile = lds + Ly.ctile + (size_t)wave * MMA_TILE_BYTES;
    uint8_t* stage = lds + Ly.stage;
    const int pitch = 2 * k + MMA_PITCH_PAD;

    // ---- requests, in this order: staged digits, block table, weight
    // scales, code tiles.  Memory operations of a wave complete in order, so
    // waiting for the first three (before the barrier) leaves the codes in
    // flight.  Past the end every request repeats a valid address.
    constexpr int SU = STAGE ? MMA_STAGE_BYTES / 16 / 512 : 1;
    const int rchunks = k / 8, schunks = batch * rchunks;   // 16-byte digit chunks per row, in all
    mma_v4u sv[SU];
    if constexpr (STAGE) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int c = tid + 512 * u, cc = c < schunks ? c : schunks - 1;
            const int b = cc / rchunks;
            sv[u] = *reinterpret_cast<const mma_v4u*>(xq + (int64_t)b * stride + 16 * (cc - b * rchunks));
        }
    }
    constexpr int TPT = 4;                                   // table entries per thread, at most (k <= 16384)
    float tsx[TPT];
    int tsq0[TPT], tsq1[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int e = tid + 512 * u;
        const int blk = e >> 4 < nbk ? e >> 4 : nbk - 1, b = (e & 15) < batch ? (e & 15) : 0;
        const uint8_t* xr = xq + (int64_t)b * stride + 2 * k;
        tsx[u] = reinterpret_cast<const float*>(xr)[blk];
        const int* hs = reinterpret_cast<const int*>(xr + k / 32);
        tsq0[u] = hs[2 * blk];
        tsq1[u] = hs[2 * blk + 1];
    }
    constexpr int SWU = MMA_MAX_ITEMS * 16 / 512;            // weight scales per thread, at most
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

    // ---- LDS: block table, weight scales, staged digits, own partial rows
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int e = tid + 512 * u;
        const float sx = (e & 15) < batch ? tsx[u] : 0.0f;
        if (e < nbk * 16) tab[e] = make_float2(2.0f * sx, -7.0f * sx * (float)(tsq0[u] + tsq1[u]));
    }
#pragma unroll
    for (int u = 0; u < SWU; ++u) {                          // past the end: the last entry again, same place
        const int e = tid + 512 * u, ec = e < nsw ? e : nsw - 1;
        const int r = ec / nbk;
        swt[r * nbk4 + (ec - r * nbk)] = (uint16_t)swv[u];
    }
    if constexpr (STAGE) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int c = tid + 512 * u, cc = c < schunks ? c : schunks - 1;
            const int b = cc / rchunks;
            *reinterpret_cast<mma_v4u*>(stage + (size_t)b * pitch + 16 * (cc - b * rchunks)) = sv[u];
        }
    }
    for (int e = lane; e < R * 4; e += 64) reinterpret_cast<float4*>(ywv)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    lds_barrier();

    // ---- items: the digits and table entries of the next item are requested
    // ahead (from LDS, or for unstaged digits from the L2)
    const int bcol = r16 < batch ? r16 : 0;                  // batch row of this lane's A operand
    const uint8_t* drow = (STAGE ? stage + (size_t)bcol * pitch : xq + (int64_t)bcol * stride) + 64 * kq;
    uint4 dg[2][4];
    float4 tb2[2][2];                                        // (2 sx, -7 sx sum q) of batch rows 4 kq .. 4 kq + 3
    auto blk_of = [&](int m) {                               // block of item m (4 per tile), clamped to the row
        const int t = tile_of(m >> 2);
        const int b = 4 * (t - (t / tpr) * tpr) + (m & 3);
        return b < nbk ? b : nbk - 1;
    };
    auto request = [&](int m, int slot) {
        const int blk = blk_of(m);
        const uint4* p = reinterpret_cast<const uint4*>(drow + 256 * blk);
        dg[slot][0] = p[0];                                  // hi, dword 2 kq
        dg[slot][1] = p[1];                                  // lo
        dg[slot][2] = p[2];                                  // hi, dword 2 kq + 1
        dg[slot][3] = p[3];                                  // lo
        const float4* tq = reinterpret_cast<const float4*>(tab + 16 * blk + 4 * kq);
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
                // this lane: batch rows 4 kq .. 4 kq + 3 of weight row 16 rt + r16
                const int blk = 4 * tb + j;
                const float sw = blk < nbk ? h2f(swt[(16 * rt + r16) * nbk4 + blk]) : 0.0f;   // uniform test
                mma_block(ctile, r16, kq, j, dg[m & 1], tb2[m & 1], sw, acc);
            }
            // a tile's running sums go to the wave's slot of its row tile; they
            // carry on into the next tile of the same row tile (the last store
            // of a slot holds all of it)
            *reinterpret_cast<float4*>(ywv + 16 * (16 * rt + r16) + 4 * kq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            if (i + 1 < TPW && tile_of(i + 1) / tpr != rt) {  // uniform
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
            }
        }
    }
    __syncthreads();

    // ---- the waves' sums in wave order
    for (int e = tid; e < R * batch; e += 512) {
        const int b = e / R, r = e - b * R;
        if (row0 + r >= n) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) v += yw[((size_t)w * R + r) * 16 + b];
        y[(int64_t)b * n + row0 + r] = v;
    }
}

template <int TPW>
int launch_mma_t(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint8_t* xq, int stride,
                 int batch, float* y, int R, hipStream_t st) {
    const dim3 grid((unsigned)((n + R - 1) / R));
    const bool stage = batch * 2 * k <= MMA_STAGE_BYTES && mma_layout((int)k, R, batch, true).total <= MMA_LDS_LIMIT;
    const size_t lds = mma_layout((int)k, R, batch, stage).total;
    if (stage)
        hipLaunchKernelGGL((k_qgemv_mma<TPW, true>), grid, dim3(512), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y, R);
    else
        hipLaunchKernelGGL((k_qgemv_mma<TPW, false>), grid, dim3(512), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y, R);
    return hip_check(hipGetLastError(), "pg_qgemv launch");
}

}  // namespace

// Rows per workgroup: a multiple of 16 near n / CUs, so that one round of
// workgroups covers the matrix, with at most 8 tiles per wave.
int launch_qgemv_mma(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint8_t* xq,
                     int batch, float* y, pg_stream_t s) {
    const int cus = compute_units();
    const int nbk = (int)(k / 128), nbk4 = (nbk + 3) & ~3;
    if (nbk * 16 > 512 * 4 || nbk4 > MMA_MAX_ITEMS)
        return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the batched PG_Q16 path", (long long)k);
    int64_t per = (n + cus - 1) / cus;
    int64_t R = 16 * ((per + 15) / 16);
    if (R > 128) R = 128;                                    // 8 waves x R x 64 B of partial sums
    while (R > 16 && (R / 16) * nbk4 > MMA_MAX_ITEMS) R -= 16;
    const int tpw = (int)(((R / 16) * (nbk4 / 4) + 7) / 8);
    const int stride = (int)q16_row_bytes(k);
    hipStream_t st = (hipStream_t)s;
    switch (tpw) {
        case 1: return launch_mma_t<1>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 2: return launch_mma_t<2>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 3: return launch_mma_t<3>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 4: return launch_mma_t<4>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 5: return launch_mma_t<5>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 6: return launch_mma_t<6>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        case 7: return launch_mma_t<7>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
        default: return launch_mma_t<8>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    }
}

}  // namespace pg
