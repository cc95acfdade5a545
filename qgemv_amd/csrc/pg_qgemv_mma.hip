// Batched product on PG_Q16 activations with the gfx950 int8 matrix cores
// (batch 2..8 of pg_qgemv).  The VALU path (k_qgemv_q16) pays two v_dot4 per
// code dword for every batch row; here the bit planes of a code dword are the
// B operand of v_mfma_i32_16x16x64_i8 and up to 16 batch rows share them, so
// the vector work per weight stays that of the decode.
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode,
// rotation before coding); batched generation is the case the same page's
// section on limits calls weakest.  Bit layout and PG_Q16: include/pingala.h.
#include "pg_device.h"

namespace pg {
namespace {

typedef int mma_v4i __attribute__((ext_vector_type(4)));

// One item = (tile of 16 weight rows, 128-block).  For every item the
// 16 x 16 x 64 int8 product
//   D[b][r] += sum_k A[b][k] B[k][r]
// takes A = activation digits (row b = batch row, 16 rows of which the first
// `batch` are real) and B = bit planes P = (level + 7) / 2 of the weight rows.
// Lane l supplies A row / B column l % 16 and the k slice l / 16 (16 bytes);
// it receives D[4 (l / 16) + i][l % 16], i = 0..3.  Lane group kq = l / 16
// takes code dwords 2 kq and 2 kq + 1 of the block: the product mm = 0, 1
// pairs dword 2 kq + mm of every lane group, so two products cover the
// block's 8 dwords.  PG_Q16 chunk 8 blk + d holds dword d's 16 values in
// plane order (byte 4 j + g is group g, position j; hi digits, then lo), the
// order of the planes, so both operands are 16 bytes as stored.  Per block,
// exactly in int32,
//   sum level q = 2 (256 H + L) - 7 sum q,  H = sum P hi,  L = sum P lo,
// then y[b][r] += sw[r][blk] * sx[b][blk] * that, in fp32.
//
// Workgroup: 8 waves over R = 16 NRT rows and all k columns; items g (row
// tile g / nbk, block g % nbk) in consecutive runs, one run per wave.  All code dwords and weight scales
// of a wave's items are requested at entry; the activation digits (read by
// every workgroup, so they come from the L2) are copied to LDS at entry
// when all batch rows fit (STAGE), else requested a pair of items ahead.
// Each wave adds its items into its own LDS rows [R][16]; the waves' sums
// are added in wave order at the end, so the result does not depend on
// timing.
constexpr int MMA_PITCH_PAD = 16;      // LDS row pitch of staged digits: 2k + 16 bytes, so that the 16-byte
                                       // reads of 8 consecutive batch rows fall in distinct banks

template <int IPW, bool STAGE>
__global__ __launch_bounds__(512) void k_qgemv_mma(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int n, int k,
                                                   const uint8_t* __restrict__ xq, int stride, int batch,
                                                   float* __restrict__ y, int R) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(xq), "s"(stride), "s"(batch), "s"(y), "s"(R));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = k >> 2, nbk = k >> 7;
    const int row0 = blockIdx.x * R;
    const int items = (R >> 4) * nbk;
    const int r16 = lane & 15, kq = lane >> 4;
    float2* tab = reinterpret_cast<float2*>(lds);                          // [nbk][16]: (2 sx, -7 sx sum q)
    float* yw = reinterpret_cast<float*>(lds + (size_t)nbk * 16 * 8);      // [8][R][16]
    float* ywv = yw + (size_t)wave * R * 16;
    uint8_t* stage = lds + (size_t)nbk * 16 * 8 + (size_t)8 * R * 16 * 4;   // [batch][2k + 64] digits
    const int pitch = 2 * k + MMA_PITCH_PAD;

    // ---- staged digits: every batch row's 2k digit bytes, 1 KiB per wave
    // and copy (direct global -> LDS)
    if (STAGE) {
        for (int b = 0; b < batch; ++b)
            for (int o = wave * 1024; o < 2 * k; o += 8 * 1024)
                if (o + 16 * lane < 2 * k)
                    __builtin_amdgcn_global_load_lds(xq + (int64_t)b * stride + o + 16 * lane, stage + (size_t)b * pitch + o,
                                                     16, 0, 0);
    }

    // ---- block scales and sums of every batch row (issued first: the wait
    // for them below leaves the code requests in flight)
    constexpr int TPT = 4;                                   // table entries per thread, at most
    float tsx[TPT];
    int tsq0[TPT], tsq1[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        // every lane loads (from a valid address); entries past the batch
        // are zeroed when written
        const int e = tid + 512 * u;
        const int blk = e >> 4 < nbk ? e >> 4 : nbk - 1, b = (e & 15) < batch ? (e & 15) : 0;
        const uint8_t* xr = xq + (int64_t)b * stride + 2 * k;
        tsx[u] = reinterpret_cast<const float*>(xr)[blk];
        const int* hs = reinterpret_cast<const int*>(xr + k / 32);
        tsq0[u] = hs[2 * blk];
        tsq1[u] = hs[2 * blk + 1];
    }
    asm volatile("" ::: "memory");

    // ---- every item's code dwords and weight scale
    // item i of this wave: row tile and block (uniform; past the end a repeat
    // of the last item, requested but never used)
    // a wave's items are consecutive (blocks of a row tile in order), so the
    // 4 blocks of a 128-byte line of codes come in back-to-back requests
    const int per = (items + 7) >> 3;                        // items of a wave, at most
    const int first = wave * per;
    const int mine = items - first < per ? (items - first > 0 ? items - first : 0) : per;
    auto item_g = [&](int i) { const int g = first + i; return g < items ? g : items - 1; };
    auto item_rt = [&](int i) { return item_g(i) / nbk; };
    auto item_blk = [&](int i) { const int g = item_g(i); return g - (g / nbk) * nbk; };
    uint2 cd[IPW];
    uint32_t wsr[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int blk = item_blk(i);
        int row = row0 + 16 * item_rt(i) + r16;
        if (row >= n) row = n - 1;
        const uint8_t* cb = codes + (int64_t)row * kg + 32 * blk;
        cd[i] = *reinterpret_cast<const uint2*>(cb + 8 * kq);
        wsr[i] = scales[(int64_t)row * nbk + blk];          // 16-bit load into a whole register
    }
    asm volatile("" ::: "memory");

    // ---- activation digits and block table entries, a pair of items ahead
    const int bcol = r16 < batch ? r16 : 0;                  // batch row of this lane's A operand
    const uint8_t* xrow = xq + (int64_t)bcol * stride + 64 * kq;
    const uint8_t* srow = stage + (size_t)bcol * pitch + 64 * kq;
    uint4 dg[2][2][4];                                       // [pair slot][item of the pair][operand]
    float4 tb[2][2][2];                                      // (2 sx, -7 sx sum q) of batch rows 4 kq .. 4 kq + 3
    auto request_digits = [&](int pr, int slot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4* q4 = reinterpret_cast<const uint4*>((STAGE ? srow : xrow) + 256 * item_blk(2 * pr + h));
            dg[slot][h][0] = q4[0];                          // hi, dword 2 kq
            dg[slot][h][1] = q4[1];                          // lo
            dg[slot][h][2] = q4[2];                          // hi, dword 2 kq + 1
            dg[slot][h][3] = q4[3];                          // lo
        }
    };
    auto request_tab = [&](int pr, int slot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4* tq = reinterpret_cast<const float4*>(tab + 16 * item_blk(2 * pr + h) + 4 * kq);
            tb[slot][h][0] = tq[0];
            tb[slot][h][1] = tq[1];
        }
    };
    if (!STAGE) request_digits(0, 0);                        // staged digits are read after the barrier

    // tables to LDS (the compiler's wait for them counts the later requests
    // as still in flight), own partial rows cleared
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int e = tid + 512 * u;
        const float sx = (e & 15) < batch ? tsx[u] : 0.0f;
        if (e < nbk * 16) tab[e] = make_float2(2.0f * sx, -7.0f * sx * (float)(tsq0[u] + tsq1[u]));
    }
    for (int e = lane; e < R * 4; e += 64) reinterpret_cast<float4*>(ywv)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    lds_barrier();

    // one item: planes of the lane's two code dwords, four products, and the
    // block's contribution added to the running sums of the row tile, which
    // are stored to the wave's slot of that tile after every item (the last
    // store of a tile holds all of it; items past the wave's run add zero)
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto item = [&](int i, const uint4 (&d)[4], const float4 (&t)[2]) {
        // dword 2 kq - 1 is the second dword of lane l - 16 (a block starts the
        // trellis at state 0)
        const uint32_t left = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (lane - 16), (int)cd[i].y);
        const uint32_t prev = kq > 0 ? left : 0u;
        uint32_t P0[4], P1[4];
        planes_of(cd[i].x, prev, P0);
        planes_of(cd[i].y, cd[i].x, P1);
        const mma_v4i b0 = {(int)P0[0], (int)P0[1], (int)P0[2], (int)P0[3]};
        const mma_v4i b1 = {(int)P1[0], (int)P1[1], (int)P1[2], (int)P1[3]};
        mma_v4i H = {0, 0, 0, 0}, L = {0, 0, 0, 0};
        H = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[0]), b0, H, 0, 0, 0);
        L = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[1]), b0, L, 0, 0, 0);
        H = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[2]), b1, H, 0, 0, 0);
        L = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(mma_v4i, d[3]), b1, L, 0, 0, 0);
        // this lane: batch rows 4 kq .. 4 kq + 3 of weight row 16 rt + r16
        const float sw = i < mine ? h2f((uint16_t)(wsr[i] & 0xffffu)) : 0.0f;   // uniform choice
        const float tx[4] = {t[0].x, t[0].z, t[1].x, t[1].z}, ty[4] = {t[0].y, t[0].w, t[1].y, t[1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float f = (float)(H[j] * 256 + L[j]);
            acc[j] = fmaf(fmaf(f, tx[j], ty[j]), sw, acc[j]);
        }
        *reinterpret_cast<float4*>(ywv + 16 * (16 * item_rt(i) + r16) + 4 * kq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        const bool next_tile = i + 1 < IPW && item_rt(i + 1) != item_rt(i);   // uniform
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = next_tile ? 0.0f : acc[j];
    };

    if (STAGE) request_digits(0, 0);
    request_tab(0, 0);
#pragma unroll
    for (int pr = 0; pr < IPW / 2; ++pr) {
        // the next pair's operands first (also past this wave's run: valid
        // repeats, so that the wait counts stay fixed)
        if (pr + 1 < IPW / 2) {
            request_digits(pr + 1, (pr + 1) & 1);
            request_tab(pr + 1, (pr + 1) & 1);
        }
        asm volatile("" ::: "memory");                       // keeps the requests here, ahead of their use
        // two independent items in one block, for the scheduler to interleave
        item(2 * pr, dg[pr & 1][0], tb[pr & 1][0]);
        item(2 * pr + 1, dg[pr & 1][1], tb[pr & 1][1]);
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

// LDS of one launch: the block table, the waves' partial rows and (STAGE)
// the digits of every batch row
inline size_t mma_lds_bytes(int64_t k, int R, int batch, bool stage) {
    return (size_t)(k / 128) * 16 * 8 + (size_t)8 * R * 16 * 4 +
           (stage ? (size_t)batch * (size_t)(2 * k + MMA_PITCH_PAD) : 0);
}

template <int IPW>
int launch_mma_t(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint8_t* xq, int stride,
                 int batch, float* y, int R, hipStream_t st) {
    const dim3 grid((unsigned)((n + R - 1) / R));
    const bool stage = batch * (2 * k + MMA_PITCH_PAD) <= 96 * 1024;
    const size_t lds = mma_lds_bytes(k, R, batch, stage);
    if (stage)
        hipLaunchKernelGGL((k_qgemv_mma<IPW, true>), grid, dim3(512), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y, R);
    else
        hipLaunchKernelGGL((k_qgemv_mma<IPW, false>), grid, dim3(512), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y, R);
    return hip_check(hipGetLastError(), "pg_qgemv launch");
}

}  // namespace

// Rows per workgroup: a multiple of 16 near n / CUs, so that one round of
// workgroups covers the matrix, with at most 32 items per wave.
int launch_qgemv_mma(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint8_t* xq,
                     int batch, float* y, pg_stream_t s) {
    const int cus = compute_units();
    const int nbk = (int)(k / 128);
    if (nbk * 16 > 512 * 4) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the batched PG_Q16 path", (long long)k);
    int64_t per = (n + cus - 1) / cus;
    int64_t R = 16 * ((per + 15) / 16);
    if (const char* e = getenv("PG_MMA_ROWS")) {             // rows per workgroup, for tuning sweeps
        const int r2 = atoi(e);
        if (r2 >= 16) R = 16 * (r2 / 16);
    }
    if (R > 128) R = 128;                                    // 8 waves x R x 64 B of partial sums
    while (R > 16 && (R / 16) * nbk > 8 * 28) R -= 16;
    if ((R / 16) * nbk > 8 * 28) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the batched PG_Q16 path", (long long)k);
    const int ipw = (int)(((R / 16) * nbk + 7) / 8);
    const int stride = (int)q16_row_bytes(k);
    hipStream_t st = (hipStream_t)s;
    if (ipw <= 2) return launch_mma_t<2>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 4) return launch_mma_t<4>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 6) return launch_mma_t<6>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 8) return launch_mma_t<8>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 10) return launch_mma_t<10>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 12) return launch_mma_t<12>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 14) return launch_mma_t<14>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 16) return launch_mma_t<16>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 20) return launch_mma_t<20>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    if (ipw <= 24) return launch_mma_t<24>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
    return launch_mma_t<28>(codes, scales, n, k, xq, stride, batch, y, (int)R, st);
}

}  // namespace pg
