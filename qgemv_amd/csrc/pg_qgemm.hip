// Prompt product of libpingala on the gfx950 matrix cores: Y = X . W~^T for
// m rows of bf16 activations X against P8F v1 codes, the weights decoded
// tile by tile into LDS as bf16 levels (small odd integers, exact in bf16).
//
// Method: "Pingala-8" landing page, section "How it works" (the trellis
// decode); bit layout in include/pingala.h.
#include <algorithm>
#include <mutex>

#include "pg_device.h"

namespace pg {
namespace {

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
// Split K: workgroups 0 .. t_full - 1 take tiles 0 .. t_full - 1 whole; the
// workgroups after them take the other nrem = tiles - t_full tiles S ways,
// workgroup t_full + i covering tile t_full + i % nrem over the 128-blocks
// [s nbk / S, (s + 1) nbk / S) of split s = i / nrem.  Split 0 writes y;
// split s > 0 writes its 256 x 128 block to part s - 1 of the workspace
// ([S - 1][nrem][256][128] fp32), which k_qgemm_sum then adds to y.  Each
// range is XCD-grouped by itself (remap bit 0: the whole tiles, bit 1: the
// splits), so that the whole tiles are dispatched first and the short split
// workgroups fill the last round.
// LDS rows are 128 bytes; 16-byte chunk c of row r sits at c ^ ((r / 2) & 7),
// so that the 16 rows an operand read touches at once fall on distinct banks.
constexpr int Q2_BM = 256, Q2_BN = 128, Q2_BK = 64;
constexpr int Q2_XBYTES = Q2_BM * Q2_BK * 2, Q2_WBYTES = Q2_BN * Q2_BK * 2;

__device__ __forceinline__ int q2_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(512) void k_qgemm_v2(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const uint16_t* __restrict__ x, int m,
                                                  float* __restrict__ y, int tiles_n, int remap, int tiles,
                                                  int t_full, int splits, float* __restrict__ ws) {
    // one object per buffer, and the step loop unrolled by 6 so that every
    // access names its buffer statically: the compiler then sees that the
    // direct copies in flight never touch the buffers being read or written
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];      // X, 256 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs2[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[Q2_WBYTES];      // levels, 128 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t ws1[Q2_WBYTES];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap),
                 "s"(tiles), "s"(t_full), "s"(splits), "s"(ws));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // tiles of one XCD are consecutive in (n, m) order, so that they share X rows in L2
    int t, split = 0, nsplit = 1;
    const int nrem = tiles - t_full;
    if ((int)blockIdx.x < t_full) {
        t = blockIdx.x;
        if (remap & 1) t = (t & 7) * (t_full >> 3) + (t >> 3);
    } else {
        int i = blockIdx.x - t_full;
        const int cnt = gridDim.x - t_full;
        if (remap & 2) i = (i & 7) * (cnt >> 3) + (i >> 3);
        split = i / nrem;
        t = t_full + (i - split * nrem);
        nsplit = splits;
    }
    const int n0 = (t % tiles_n) * Q2_BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7;
    // this split's steps [st0, st_end): whole 128-blocks, so st0 is even
    const int st0 = 2 * (int)((int64_t)split * nbk / nsplit);
    const int st_end = 2 * (int)((int64_t)(split + 1) * nbk / nsplit);
    // output: y itself, or this split's tile block of the workspace
    float* __restrict__ out = y;
    int64_t ld = n;
    int rb = 0, cb = 0;
    if (split > 0) {
        out = ws + ((int64_t)(split - 1) * nrem + (t - t_full)) * (Q2_BM * Q2_BN);
        ld = Q2_BN;
        rb = m0;
        cb = n0;
    }

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

    // prologue: codes and X of steps st0 and st0 + 1, levels of step st0
    const uint32_t c0 = csrc[4 * st0];
    copy_x(st0, xs0);
    const int s1 = st0 + 1;                             // a split holds at least one block
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
        const int sn = st + 2 < st_end ? st + 2 : st_end - 1;
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
        if (st + 1 < st_end) decode(!half2, c1, wnext);          // levels of step st + 1
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
        lds_barrier();                                          // level writes and operand reads done
    };
    for (int st = st0; st < st_end; st += 6) {                  // whole blocks: an even count of steps
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
        if (st + 2 >= st_end) break;
        body(std::integral_constant<int, 2>(), st + 2);
        body(std::integral_constant<int, 3>(), st + 3);
        if (st + 4 >= st_end) break;
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
                if (row < m) out[(int64_t)(row - rb) * ld + (col - cb)] = acc[i][j][r];
            }
        }
}

// Warp-specialised prompt product: the tile, buffers, decode and split-K
// plan of k_qgemm_v2, with the work split by role.  Waves 0..7 (consumers)
// only read operands from LDS, run the matrix cores and apply the per-block
// scales; waves 8..11 (producers) issue the X copies of step s + 2 and the
// code loads, and decode the levels of step s + 1 (two code dwords per
// thread).  One barrier per step, so between barriers the consumers' matrix
// work on step s runs beside the producers' copies and decode on the other
// waves of the same SIMDs.  The producers wait for their own copies (vmcnt)
// before the barrier; the consumers issue no copies, so none of their LDS
// reads waits for one.
__global__ __launch_bounds__(768) void k_qgemm_v3(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const uint16_t* __restrict__ x, int m,
                                                  float* __restrict__ y, int tiles_n, int remap, int tiles,
                                                  int t_full, int splits, float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs2[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[Q2_WBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws1[Q2_WBYTES];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap),
                 "s"(tiles), "s"(t_full), "s"(splits), "s"(ws));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int t, split = 0, nsplit = 1;
    const int nrem = tiles - t_full;
    if ((int)blockIdx.x < t_full) {
        t = blockIdx.x;
        if (remap & 1) t = (t & 7) * (t_full >> 3) + (t >> 3);
    } else {
        int i = blockIdx.x - t_full;
        const int cnt = gridDim.x - t_full;
        if (remap & 2) i = (i & 7) * (cnt >> 3) + (i >> 3);
        split = i / nrem;
        t = t_full + (i - split * nrem);
        nsplit = splits;
    }
    const int n0 = (t % tiles_n) * Q2_BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7;
    const int st0 = 2 * (int)((int64_t)split * nbk / nsplit);
    const int st_end = 2 * (int)((int64_t)(split + 1) * nbk / nsplit);

    if (wave >= 8) {
        // ---------------------------------------------------------- producers
        const int pw = wave - 8, pt = tid - 512;
        const uint16_t* xtile = x + (int64_t)m0 * k;
        int xoff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = (8 * pw + i) * 64 + lane;
            const int r = j >> 3, c = q2_chunk(r, j & 7);
            const int gr = m0 + r < m ? r : m - 1 - m0;
            xoff[i] = gr * k + 8 * c;
        }
        auto copy_x = [&](int st, uint8_t* dst) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_global_load_lds(xtile + xoff[i] + st * Q2_BK, dst + (8 * pw + i) * 1024, 16, 0, 0);
        };
        // code dwords: rows pt / 4 and pt / 4 + 64 of the tile, dword pt % 4 of the step
        const int nr = pt >> 2, dm = pt & 3;
        const int wrow0 = n0 + nr < n ? n0 + nr : n - 1;
        const int wrow1 = n0 + nr + 64 < n ? n0 + nr + 64 : n - 1;
        const uint32_t* csrc0 = reinterpret_cast<const uint32_t*>(codes + (int64_t)wrow0 * kg) + dm;
        const uint32_t* csrc1 = reinterpret_cast<const uint32_t*>(codes + (int64_t)wrow1 * kg) + dm;
        uint32_t dprev[2] = {0u, 0u};
        auto decode = [&](bool second_half, uint32_t d, int h, uint8_t* wdst) {
            const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x111, 0xf, 0xf, true);          // lane - 1
            const uint32_t back = (uint32_t)__builtin_amdgcn_mov_dpp((int)dprev[h], 0x103, 0xf, 0xf, true);   // lane + 3
            const uint32_t dp = dm != 0 ? left : (second_half ? back : 0u);
            dprev[h] = d;
            uint32_t P[4];
            planes_of(d, dp, P);
            const uint32_t t0 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
            const uint32_t u0 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
            const uint32_t t1 = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);
            const uint32_t u1 = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
            const uint32_t Q[4] = {__builtin_amdgcn_perm(u0, t0, 0x05040100u), __builtin_amdgcn_perm(u0, t0, 0x07060302u),
                                   __builtin_amdgcn_perm(u1, t1, 0x05040100u), __builtin_amdgcn_perm(u1, t1, 0x07060302u)};
            uint32_t o[8];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t lo = __builtin_amdgcn_perm(0xE0A04080u, 0x8040A0E0u, Q[g]);
                const uint32_t hi = __builtin_amdgcn_perm(0x4040403Fu, 0xBFC0C0C0u, Q[g]);
                o[2 * g] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
                o[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
            }
            const int rr = nr + 64 * h;
            uint8_t* row = wdst + rr * 128;
            *reinterpret_cast<uint4*>(row + 16 * q2_chunk(rr, 2 * dm)) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint4*>(row + 16 * q2_chunk(rr, 2 * dm + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
        };
        // prologue: codes and X of steps st0 and st0 + 1, levels of step st0
        const uint32_t a0 = csrc0[4 * st0], b0 = csrc1[4 * st0];
        copy_x(st0, xs0);
        const int s1 = st0 + 1;
        uint32_t a1 = csrc0[4 * s1], b1 = csrc1[4 * s1];
        copy_x(s1, xs1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        decode(false, a0, 0, ws0);
        decode(false, b0, 1, ws0);
        lds_barrier();
        auto body = [&](auto J, int st) {
            constexpr int j6 = decltype(J)::value;
            uint8_t* xnext2 = j6 % 3 == 0 ? xs2 : j6 % 3 == 1 ? xs0 : xs1;
            uint8_t* wnext = j6 % 2 == 0 ? ws1 : ws0;
            constexpr bool half2 = (j6 & 1) != 0;
            const int sn = st + 2 < st_end ? st + 2 : st_end - 1;
            const uint32_t a2 = csrc0[4 * sn], b2 = csrc1[4 * sn];
            copy_x(sn, xnext2);
            // all but this step's 10 requests have landed: the codes and X copies of step st + 1
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
            if (st + 1 < st_end) {
                decode(!half2, a1, 0, wnext);
                decode(!half2, b1, 1, wnext);
            }
            a1 = a2;
            b1 = b2;
            lds_barrier();
        };
        for (int st = st0; st < st_end; st += 6) {
            body(std::integral_constant<int, 0>(), st);
            body(std::integral_constant<int, 1>(), st + 1);
            if (st + 2 >= st_end) break;
            body(std::integral_constant<int, 2>(), st + 2);
            body(std::integral_constant<int, 3>(), st + 3);
            if (st + 4 >= st_end) break;
            body(std::integral_constant<int, 4>(), st + 4);
            body(std::integral_constant<int, 5>(), st + 5);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));               // the repeated copies past the end
        return;
    }

    // -------------------------------------------------------------- consumers
    const int wm = wave >> 1, wn = wave & 1;
    float* __restrict__ out = y;
    int64_t ld = n;
    int rb = 0, cb = 0;
    if (split > 0) {
        out = ws + ((int64_t)(split - 1) * nrem + (t - t_full)) * (Q2_BM * Q2_BN);
        ld = Q2_BN;
        rb = m0;
        cb = n0;
    }
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
    uint32_t sc_cur[2] = {0, 0};
    lds_barrier();                                              // the producers' prologue
    auto body = [&](auto J, int st) {
        constexpr int j6 = decltype(J)::value;
        uint8_t* xcur = j6 % 3 == 0 ? xs0 : j6 % 3 == 1 ? xs1 : xs2;
        uint8_t* wcur = j6 % 2 == 0 ? ws0 : ws1;
        constexpr bool half2 = (j6 & 1) != 0;
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
        if (half2) {
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
        lds_barrier();
    };
    for (int st = st0; st < st_end; st += 6) {
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
        if (st + 2 >= st_end) break;
        body(std::integral_constant<int, 2>(), st + 2);
        body(std::integral_constant<int, 3>(), st + 3);
        if (st + 4 >= st_end) break;
        body(std::integral_constant<int, 4>(), st + 4);
        body(std::integral_constant<int, 5>(), st + 5);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 64 * wn + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) out[(int64_t)(row - rb) * ld + (col - cb)] = acc[i][j][r];
            }
        }
}

// Producer/consumer prompt product with the block scales carried in the
// running sum: the tile, buffers and split plans of k_qgemm_v2 in 1024
// threads, waves 0..7 consumers (operand reads and matrix cores only) and
// waves 8..15 producers (X copies, code loads, decode; one code dword per
// thread as in k_qgemm_v2).  Instead of a per-block partial sum, a
// consumer keeps acc = sum over the blocks so far of (s_b / s_cur) * S_b,
// with s_cur the scale of its column's current block: at each block end it
// multiplies acc by s_cur / s_next and at the end by s_cur, so the matrix
// cores accumulate straight into acc and a consumer holds one set of
// accumulators, which leaves registers for four waves per SIMD.  A block
// of zero scale is decoded as zero levels and keeps s_cur (no division by
// zero; an all-zero prefix multiplies zeros).
__global__ __launch_bounds__(1024) void k_qgemm_v4(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, int n, int k,
                                                   const uint16_t* __restrict__ x, int m,
                                                   float* __restrict__ y, int tiles_n, int remap, int tiles,
                                                   int t_full, int splits, float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t xs2[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[Q2_WBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws1[Q2_WBYTES];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap),
                 "s"(tiles), "s"(t_full), "s"(splits), "s"(ws));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int t, split = 0, nsplit = 1;
    const int nrem = tiles - t_full;
    if ((int)blockIdx.x < t_full) {
        t = blockIdx.x;
        if (remap & 1) t = (t & 7) * (t_full >> 3) + (t >> 3);
    } else {
        int i = blockIdx.x - t_full;
        const int cnt = gridDim.x - t_full;
        if (remap & 2) i = (i & 7) * (cnt >> 3) + (i >> 3);
        split = i / nrem;
        t = t_full + (i - split * nrem);
        nsplit = splits;
    }
    const int n0 = (t % tiles_n) * Q2_BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7;
    const int st0 = 2 * (int)((int64_t)split * nbk / nsplit);
    const int st_end = 2 * (int)((int64_t)(split + 1) * nbk / nsplit);

    if (wave >= 8) {
        // ---------------------------------------------------------- producers
        const int pw = wave - 8, pt = tid - 512;
        const uint16_t* xtile = x + (int64_t)m0 * k;
        int xoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = (4 * pw + i) * 64 + lane;
            const int r = j >> 3, c = q2_chunk(r, j & 7);
            const int gr = m0 + r < m ? r : m - 1 - m0;
            xoff[i] = gr * k + 8 * c;
        }
        auto copy_x = [&](int st, uint8_t* dst) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds(xtile + xoff[i] + st * Q2_BK, dst + (4 * pw + i) * 1024, 16, 0, 0);
        };
        const int nr = pt >> 2, dm = pt & 3;
        const int wrow = n0 + nr < n ? n0 + nr : n - 1;
        const uint32_t* csrc = reinterpret_cast<const uint32_t*>(codes + (int64_t)wrow * kg) + dm;
        const uint16_t* srow = scales + (int64_t)wrow * nbk;
        uint32_t dprev = 0;
        auto decode = [&](bool second_half, uint32_t d, bool zero, uint8_t* wdst) {
            const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x111, 0xf, 0xf, true);
            const uint32_t back = (uint32_t)__builtin_amdgcn_mov_dpp((int)dprev, 0x103, 0xf, 0xf, true);
            const uint32_t dp = dm != 0 ? left : (second_half ? back : 0u);
            dprev = d;
            uint32_t P[4];
            planes_of(d, dp, P);
            const uint32_t t0 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
            const uint32_t u0 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
            const uint32_t t1 = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);
            const uint32_t u1 = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
            const uint32_t Q[4] = {__builtin_amdgcn_perm(u0, t0, 0x05040100u), __builtin_amdgcn_perm(u0, t0, 0x07060302u),
                                   __builtin_amdgcn_perm(u1, t1, 0x05040100u), __builtin_amdgcn_perm(u1, t1, 0x07060302u)};
            const uint32_t keep = zero ? 0u : ~0u;           // a zero-scale block: zero levels
            uint32_t o[8];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t lo = __builtin_amdgcn_perm(0xE0A04080u, 0x8040A0E0u, Q[g]);
                const uint32_t hi = __builtin_amdgcn_perm(0x4040403Fu, 0xBFC0C0C0u, Q[g]);
                o[2 * g] = __builtin_amdgcn_perm(hi, lo, 0x05010400u) & keep;
                o[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u) & keep;
            }
            uint8_t* row = wdst + nr * 128;
            *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm)) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
        };
        // prologue: codes, block scale and X of steps st0, st0 + 1; levels of step st0
        // (the scale travels with the codes: a zero-scale block decodes to zero levels)
        const uint32_t c0 = csrc[4 * st0];
        const uint32_t z0 = srow[st0 >> 1];
        copy_x(st0, xs0);
        const int s1 = st0 + 1;
        uint32_t c1 = csrc[4 * s1];
        uint32_t z1 = srow[s1 >> 1];
        copy_x(s1, xs1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        decode(false, c0, (z0 & 0x7fffu) == 0, ws0);
        lds_barrier();
        auto body = [&](auto J, int st) {
            constexpr int j6 = decltype(J)::value;
            uint8_t* xnext2 = j6 % 3 == 0 ? xs2 : j6 % 3 == 1 ? xs0 : xs1;
            uint8_t* wnext = j6 % 2 == 0 ? ws1 : ws0;
            constexpr bool half2 = (j6 & 1) != 0;
            const int sn = st + 2 < st_end ? st + 2 : st_end - 1;
            const uint32_t c2 = csrc[4 * sn];
            const uint32_t z2 = srow[sn >> 1];
            copy_x(sn, xnext2);
            // all but this step's 6 requests have landed: codes, scale and X copies of step st + 1
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
            if (st + 1 < st_end) decode(!half2, c1, (z1 & 0x7fffu) == 0, wnext);
            c1 = c2;
            z1 = z2;
            lds_barrier();
        };
        for (int st = st0; st < st_end; st += 6) {
            body(std::integral_constant<int, 0>(), st);
            body(std::integral_constant<int, 1>(), st + 1);
            if (st + 2 >= st_end) break;
            body(std::integral_constant<int, 2>(), st + 2);
            body(std::integral_constant<int, 3>(), st + 3);
            if (st + 4 >= st_end) break;
            body(std::integral_constant<int, 4>(), st + 4);
            body(std::integral_constant<int, 5>(), st + 5);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        return;
    }

    // -------------------------------------------------------------- consumers
    const int wm = wave >> 1, wn = wave & 1;
    float* __restrict__ out = y;
    int64_t ld = n;
    int rb = 0, cb = 0;
    if (split > 0) {
        out = ws + ((int64_t)(split - 1) * nrem + (t - t_full)) * (Q2_BM * Q2_BN);
        ld = Q2_BN;
        rb = m0;
        cb = n0;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    int scol[2];
    float scur[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + (lane & 31);
        scol[j] = col < n ? col : n - 1;
        scur[j] = h2f(scales[(int64_t)scol[j] * nbk + (st0 >> 1)]);
    }
    uint32_t snx[2] = {0, 0};
    lds_barrier();                                              // the producers' prologue
    auto body = [&](auto J, int st) {
        constexpr int j6 = decltype(J)::value;
        uint8_t* xcur = j6 % 3 == 0 ? xs0 : j6 % 3 == 1 ? xs1 : xs2;
        uint8_t* wcur = j6 % 2 == 0 ? ws0 : ws1;
        constexpr bool half2 = (j6 & 1) != 0;
        // the next block's scales, requested a step ahead
        if (!half2 && st + 2 < st_end)
#pragma unroll
            for (int j = 0; j < 2; ++j) snx[j] = scales[(int64_t)scol[j] * nbk + (st >> 1) + 1];
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
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (half2 && st + 1 < st_end) {                         // block end: carry into the next block's scale
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float sn = h2f((uint16_t)snx[j]);
                const float snew = sn != 0.0f ? sn : scur[j];
                const float r = snew != 0.0f ? scur[j] / snew : 1.0f;
                scur[j] = snew;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[i][j][q] *= r;
            }
        }
        lds_barrier();
    };
    for (int st = st0; st < st_end; st += 6) {
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
        if (st + 2 >= st_end) break;
        body(std::integral_constant<int, 2>(), st + 2);
        body(std::integral_constant<int, 3>(), st + 3);
        if (st + 4 >= st_end) break;
        body(std::integral_constant<int, 4>(), st + 4);
        body(std::integral_constant<int, 5>(), st + 5);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 64 * wn + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) out[(int64_t)(row - rb) * ld + (col - cb)] = acc[i][j][r] * scur[j];
            }
        }
}

// Wide-tile prompt product: 256 x 256 output tiles (X rows x weight rows),
// whole K, with the decode and copies of k_qgemm_v2 and the carried block
// scales of k_qgemm_v4.  Per 64-wide K step the tile does twice the matrix
// work of the 256 x 128 tile for the same 32 KB of X copied into the LDS, and
// its 128 x 64 wave tiles (4 x 2 products of 32 x 32) read 0.75 KB of
// operands from the LDS per product instead of 1 KB.  512 threads, two waves
// per SIMD; every thread copies four X chunks per step and decodes the code
// dwords of weight rows tid / 4 and tid / 4 + 128.  X is copied one step
// ahead into two buffers, codes and scales are loaded two steps ahead.  At a
// block's first step the decoding threads also store each row's block scale
// in the LDS, and at the next step the waves rescale their running sums by
// s_prev / s_new before the block's products (at the end they multiply by the
// last scale), so no second set of accumulators is held.  A zero-scale block
// is decoded as zero levels and keeps the previous scale.  Every output is
// summed in the order of k_qgemm_v4, so the two give equal results.
constexpr int Q6_BN = 256;
constexpr int Q6_WBYTES = Q6_BN * Q2_BK * 2;

__global__ __launch_bounds__(512) void k_qgemm_v6(const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scales, int n, int k,
                                                  const uint16_t* __restrict__ x, int m,
                                                  float* __restrict__ y, int tiles_n, int remap, int tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];      // X, 256 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[Q6_WBYTES];      // levels, 256 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t ws1[Q6_WBYTES];
    __shared__ float scl[2][Q6_BN];                                      // row scales, by block parity
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap),
                 "s"(tiles));
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int t = blockIdx.x;
    if (remap) t = (t & 7) * (tiles >> 3) + (t >> 3);            // tiles of one XCD share X rows in L2
    const int n0 = (t % tiles_n) * Q6_BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7;
    const int st_end = 2 * nbk;

    // X copies: copy i of wave w fills slot (4 w + i) * 64 + lane: row slot / 8, chunk position slot % 8
    const uint16_t* xtile = x + (int64_t)m0 * k;
    int xoff[4];
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
    // codes: dword tid % 4 of the step, weight rows tid / 4 and tid / 4 + 128 of the tile
    const int nr0 = tid >> 2, dm = tid & 3;
    const uint32_t* csrc[2];
    const uint16_t* srow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int wrow = n0 + nr0 + 128 * h < n ? n0 + nr0 + 128 * h : n - 1;
        csrc[h] = reinterpret_cast<const uint32_t*>(codes + (int64_t)wrow * kg) + dm;
        srow[h] = scales + (int64_t)wrow * nbk;
    }
    uint32_t dprev[2] = {0u, 0u};                       // this thread's dwords of the previous step
    auto decode = [&](bool second_half, uint32_t d, uint32_t z, int h, uint8_t* wdst) {
        const int nr = nr0 + 128 * h;
        const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x111, 0xf, 0xf, true);       // lane - 1
        const uint32_t back = (uint32_t)__builtin_amdgcn_mov_dpp((int)dprev[h], 0x103, 0xf, 0xf, true); // lane + 3
        const uint32_t dp = dm != 0 ? left : (second_half ? back : 0u);   // nothing before a block start
        dprev[h] = d;
        uint32_t P[4];
        planes_of(d, dp, P);
        const uint32_t t0 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
        const uint32_t u0 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);
        const uint32_t u1 = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
        const uint32_t Q[4] = {__builtin_amdgcn_perm(u0, t0, 0x05040100u), __builtin_amdgcn_perm(u0, t0, 0x07060302u),
                               __builtin_amdgcn_perm(u1, t1, 0x05040100u), __builtin_amdgcn_perm(u1, t1, 0x07060302u)};
        const uint32_t keep = (z & 0x7fffu) == 0 ? 0u : ~0u;             // a zero-scale block: zero levels
        uint32_t o[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t lo = __builtin_amdgcn_perm(0xE0A04080u, 0x8040A0E0u, Q[g]);
            const uint32_t hi = __builtin_amdgcn_perm(0x4040403Fu, 0xBFC0C0C0u, Q[g]);
            o[2 * g] = __builtin_amdgcn_perm(hi, lo, 0x05010400u) & keep;
            o[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u) & keep;
        }
        uint8_t* row = wdst + nr * 128;
        *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(row + 16 * q2_chunk(nr, 2 * dm + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    };

    // prologue: codes, scales and X of step 0, codes and scales of step 1; levels and row scales of step 0.
    // Codes and scales of odd steps are held in cA, zA, of even steps in cB, zB.
    uint32_t cA[2], cB[2];
    uint16_t zA[2], zB[2];
    {
        uint32_t c0[2];
        uint16_t z0[2];
        copy_x(0, xs0);
#pragma unroll
        for (int h = 0; h < 2; ++h) { c0[h] = csrc[h][0]; z0[h] = srow[h][0]; }
#pragma unroll
        for (int h = 0; h < 2; ++h) { cA[h] = csrc[h][4]; zA[h] = srow[h][0]; }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            decode(false, c0[h], z0[h], h, ws0);
            if (dm == 0) scl[0][nr0 + 128 * h] = h2f(z0[h]);
        }
    }
    lds_barrier();

    const int wm = wave >> 2, wn = wave & 3;             // 128-row half of X, 64-row quarter of the weights
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    float scur[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) scur[j] = scl[0][64 * wn + 32 * j + (lane & 31)];

    // Step st uses buffers st % 2.  Each step copies X of step st + 1 (past
    // the end: the last step again, into the buffer nobody reads) and then
    // loads the codes and scales of step st + 2 (clamped the same way), so
    // that every step makes 8 requests and the wait below has a fixed count.
    auto body = [&](auto J, int st) {
        constexpr int j2 = decltype(J)::value;
        constexpr bool half2 = j2 == 1;                 // second half of a 128-block
        uint8_t* xcur = j2 == 0 ? xs0 : xs1;
        uint8_t* xnext = j2 == 0 ? xs1 : xs0;
        uint8_t* wcur = j2 == 0 ? ws0 : ws1;
        uint8_t* wnext = j2 == 0 ? ws1 : ws0;
        copy_x(st + 1 < st_end ? st + 1 : st_end - 1, xnext);
        asm volatile("" ::: "memory");                  // the copies are issued before the loads below,
        const int sn = st + 2 < st_end ? st + 2 : st_end - 1;
        uint32_t* cn = j2 == 0 ? cB : cA;               // step st + 2
        uint16_t* zn = j2 == 0 ? zB : zA;
#pragma unroll
        for (int h = 0; h < 2; ++h) { cn[h] = csrc[h][4 * sn]; zn[h] = srow[h][sn >> 1]; }
        asm volatile("" ::: "memory");                  // and these before the operand reads
        const uint32_t* c1 = j2 == 0 ? cA : cB;         // step st + 1
        const uint16_t* z1 = j2 == 0 ? zA : zB;
        if (!half2 && st > 0) {                         // a block start: carry the sums into its scale
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float sn_ = scl[(st >> 1) & 1][64 * wn + 32 * j + (lane & 31)];
                const float snew = sn_ != 0.0f ? sn_ : scur[j];
                const float r = snew != 0.0f ? scur[j] / snew : 1.0f;
                scur[j] = snew;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[i][j][q] *= r;
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8 a[4], b[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 128 * wm + 32 * i + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8*>(xcur + r * 128 + 16 * q2_chunk(r, c));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 64 * wn + 32 * j + (lane & 31);
                b[j] = *reinterpret_cast<const bf16x8*>(wcur + r * 128 + 16 * q2_chunk(r, c));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        // all but this step's 4 code and scale requests have landed: the X of
        // step st + 1 and the codes and scales of step st + 1
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        if (st + 1 < st_end) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                decode(!half2, c1[h], z1[h], h, wnext);
                // step st + 1 starts a block: its row scales, read after the barrier
                if (half2 && dm == 0) scl[((st + 1) >> 1) & 1][nr0 + 128 * h] = h2f(z1[h]);
            }
        }
        lds_barrier();                                  // level, scale and X writes and operand reads done
    };
    for (int st = 0; st < st_end; st += 2) {            // whole blocks: an even count of steps
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
    }
    // value r of lane l of a 32x32 tile: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 64 * wn + 32 * j + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) y[(int64_t)row * n + col] = acc[i][j][r] * scur[j];
            }
        }
}

// Prompt product with the weight operand decoded in registers (k_qgemm_v7):
// the carried block scales of k_qgemm_v4, but each wave decodes the levels of
// its own weight rows straight into the matrix cores' B operands, so that
// only X passes through the LDS (copied one step ahead, 64 KB in two buffers)
// and one barrier per step hands the X buffers over.  Template parameters:
// NW waves over a 256 x BN output tile, each wave MI x (8 / MI) products of
// 32 x 32.  <4, 8, 256>: 128 x 64 wave tiles (two waves decode each weight
// row); <8, 8, 256>: 256 x 32 wave tiles (each weight row decoded once, twice
// the X operand reads); <8, 4, 128>: the same wave tiles in 4-wave
// workgroups over k_qgemm_v2's tiles and split plans, two workgroups per
// compute unit (the library's kernel).  Within a 64-wide K step the products
// take K in a permuted order, the same for both operands: product kk of lane
// half h (lanes 32 h .. 32 h + 31) covers step positions 32 h + 8 kk .. + 7,
// so that a lane needs code dwords 2 h and 2 h + 1 of its row's step and the
// dword before them (the trellis state), 12 bytes it loads itself two steps
// ahead.
__device__ __forceinline__ void levels_bf16(uint32_t d, uint32_t dp, uint32_t keep, uint32_t o[8]) {
    uint32_t P[4];
    planes_of(d, dp, P);
    // byte transpose: Qg holds P of weights 4 g .. 4 g + 3
    const uint32_t t0 = __builtin_amdgcn_perm(P[1], P[0], 0x05010400u);
    const uint32_t u0 = __builtin_amdgcn_perm(P[3], P[2], 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(P[1], P[0], 0x07030602u);
    const uint32_t u1 = __builtin_amdgcn_perm(P[3], P[2], 0x07030602u);
    const uint32_t Q[4] = {__builtin_amdgcn_perm(u0, t0, 0x05040100u), __builtin_amdgcn_perm(u0, t0, 0x07060302u),
                           __builtin_amdgcn_perm(u1, t1, 0x05040100u), __builtin_amdgcn_perm(u1, t1, 0x07060302u)};
    // bf16 of 2 P - 7 for P = 0..7 (as in k_qgemm_v2's decode)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t lo = __builtin_amdgcn_perm(0xE0A04080u, 0x8040A0E0u, Q[g]);
        const uint32_t hi = __builtin_amdgcn_perm(0x4040403Fu, 0xBFC0C0C0u, Q[g]);
        o[2 * g] = __builtin_amdgcn_perm(hi, lo, 0x05010400u) & keep;
        o[2 * g + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u) & keep;
    }
}

template <int MI, int NW, int BN>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_qgemm_v7(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales, int n, int k,
                                                      const uint16_t* __restrict__ x, int m,
                                                      float* __restrict__ y, int tiles_n, int remap, int tiles,
                                                      int t_full, int splits, float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) uint8_t xs0[Q2_XBYTES];      // X, 256 rows x 128 B
    __shared__ __attribute__((aligned(16))) uint8_t xs1[Q2_XBYTES];
    asm volatile("" ::"s"(codes), "s"(scales), "s"(n), "s"(k), "s"(x), "s"(m), "s"(y), "s"(tiles_n), "s"(remap),
                 "s"(tiles), "s"(t_full), "s"(splits), "s"(ws));
    // wave tile: MI row tiles of 32 (X rows) by NJ column groups of 32 (weight rows)
    constexpr int WM = 8 / MI, WN = NW / WM, NJ = BN / (32 * WN);
    static_assert(WM * WN == NW && NJ * 32 * WN == BN && NJ >= 1, "wave grid");
    constexpr int XC = 32 / NW;                          // X copies per thread and step (2048 16-byte slots)
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // tile and split as in k_qgemm_v2: tiles 0..t_full-1 whole, the others `splits` ways
    int t, split = 0, nsplit = 1;
    const int nrem = tiles - t_full;
    if ((int)blockIdx.x < t_full) {
        t = blockIdx.x;
        if (remap & 1) t = (t & 7) * (t_full >> 3) + (t >> 3);   // tiles of one XCD share X rows in L2
    } else {
        int i = blockIdx.x - t_full;
        const int cnt = gridDim.x - t_full;
        if (remap & 2) i = (i & 7) * (cnt >> 3) + (i >> 3);
        split = i / nrem;
        t = t_full + (i - split * nrem);
        nsplit = splits;
    }
    const int n0 = (t % tiles_n) * BN, m0 = (t / tiles_n) * Q2_BM;
    const int kg = k >> 2, nbk = k >> 7;
    const int st0 = 2 * (int)((int64_t)split * nbk / nsplit);
    const int st_end = 2 * (int)((int64_t)(split + 1) * nbk / nsplit);
    // output: y itself, or this split's tile block of the workspace
    float* __restrict__ out = y;
    int64_t ld = n;
    int rb = 0, cb = 0;
    if (split > 0) {
        out = ws + ((int64_t)(split - 1) * nrem + (t - t_full)) * (Q2_BM * BN);
        ld = BN;
        rb = m0;
        cb = n0;
    }
    const int wm = wave / WN, wn = wave % WN;
    const int hf = lane >> 5;                            // which half of each step this lane's operands hold

    // X copies: copy i of wave w fills slot (XC w + i) * 64 + lane: row slot / 8, chunk position slot % 8
    // (the copies' operands are kept free of the template parameters: a
    // direct-to-LDS copy whose operands depend on them is not instantiated
    // for the host side, and the launch then has no stub)
    const uint16_t* xtile = x + (int64_t)m0 * k;
    int xslot = XC * wave;
    int xoff[8];
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int j = (xslot + i) * 64 + lane;
        const int r = j >> 3, c = q2_chunk(r, j & 7);
        const int gr = m0 + r < m ? r : m - 1 - m0;
        xoff[i] = gr * k + 8 * c;
    }
    auto copy_x = [&](int st, uint8_t* dst) {
#pragma unroll
        for (int i = 0; i < XC; ++i)
            __builtin_amdgcn_global_load_lds(xtile + xoff[i] + st * Q2_BK, dst + (xslot + i) * 1024, 16, 0, 0);
    };
    // codes and scales of weight rows n0 + 32 (NJ wn + j) + lane % 32, j < NJ
    const uint8_t* crow[NJ];
    const uint16_t* srow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = n0 + 32 * (NJ * wn + j) + (lane & 31);
        const int wrow = col < n ? col : n - 1;
        crow[j] = codes + (int64_t)wrow * kg;
        srow[j] = scales + (int64_t)wrow * nbk;
    }
    // the 12 bytes at step st: dwords 2 hf - 1 .. 2 hf + 1 of the step (dword
    // -1 is the previous step's dword 3), or dwords 0..2 at a block start for
    // hf = 0 (nothing before it; the first word is then not used)
    auto load_codes = [&](int st, uint3* c, uint16_t* z) {
        const int off = 16 * st + 8 * hf - ((hf != 0 || (st & 1) != 0) ? 4 : 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            c[j] = *reinterpret_cast<const uint3*>(crow[j] + off);
            z[j] = srow[j][st >> 1];
        }
    };
    // B operands of step st for column group j: o[0..3] product 0, o[4..7]
    // product 1 (from dword 2 hf), p[0..3] product 2, p[4..7] product 3
    auto decode_b = [&](int st, const uint3& c, uint16_t z, uint32_t o[8], uint32_t p[8]) {
        const bool start = hf == 0 && (st & 1) == 0;
        const uint32_t prev = start ? 0u : c.x;
        const uint32_t d0 = start ? c.x : c.y;
        const uint32_t d1 = start ? c.y : c.z;
        const uint32_t keep = (z & 0x7fffu) == 0 ? 0u : ~0u;       // a zero-scale block: zero levels
        levels_bf16(d0, prev, keep, o);
        levels_bf16(d1, d0, keep, p);
    };

    // prologue: X of step 0; codes and scales of steps 0 and 1 (even steps in
    // set A, odd steps in set B)
    uint3 cA[NJ], cB[NJ];
    uint16_t zA[NJ], zB[NJ];
    copy_x(st0, xs0);
    asm volatile("" ::: "memory");
    load_codes(st0, cA, zA);
    load_codes(st0 + 1 < st_end ? st0 + 1 : st0, cB, zB);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    float scur[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) scur[j] = h2f(zA[j]);
    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Step st reads X buffer st % 2 and code set st % 2.  It copies X of step
    // st + 1 (past the end: the last step again, into the buffer nobody
    // reads) and, once its own codes are decoded, loads the codes and scales
    // of step st + 2 (clamped the same way) into the set it used, so every
    // step makes 8 requests and the wait below has a fixed count.
    auto body = [&](auto J, int st) {
        constexpr int j2 = decltype(J)::value;
        uint8_t* xcur = j2 == 0 ? xs0 : xs1;
        uint8_t* xnext = j2 == 0 ? xs1 : xs0;
        uint3* cs = j2 == 0 ? cA : cB;
        uint16_t* zs = j2 == 0 ? zA : zB;
        copy_x(st + 1 < st_end ? st + 1 : st_end - 1, xnext);
        asm volatile("" ::: "memory");                  // the copies are issued before the code loads
        // everything but these copies has landed: the codes and scales of
        // steps st and st + 1 (those of st + 1 were requested a step ago)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(XC));
        if (j2 == 0 && st > st0) {                      // a block start: carry the sums into its scale
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float s_ = h2f(zs[j]);
                const float snew = s_ != 0.0f ? s_ : scur[j];
                const float r = snew != 0.0f ? scur[j] / snew : 1.0f;
                scur[j] = snew;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[i][j][q] *= r;
            }
        }
        uint32_t bo[NJ][8], bp[NJ][8];
#pragma unroll
        for (int j = 0; j < NJ; ++j) decode_b(st, cs[j], zs[j], bo[j], bp[j]);
        const int sn = st + 2 < st_end ? st + 2 : st_end - 1;
        load_codes(sn, cs, zs);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 4 * hf + kk;
            bf16x8 a[MI], b[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = 32 * (MI * wm + i) + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8*>(xcur + r * 128 + 16 * q2_chunk(r, c));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t* src = kk < 2 ? bo[j] + 4 * kk : bp[j] + 4 * (kk - 2);
                const uint4 v = make_uint4(src[0], src[1], src[2], src[3]);
                b[j] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        // all but this step's 2 NJ code and scale requests have landed: X of step st + 1
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NJ));
        lds_barrier();                                  // X copies and operand reads done
    };
    for (int st = st0; st < st_end; st += 2) {          // whole blocks: an even count of steps
        body(std::integral_constant<int, 0>(), st);
        body(std::integral_constant<int, 1>(), st + 1);
    }
    // value r of lane l of a 32x32 tile: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = n0 + 32 * (NJ * wn + j) + (lane & 31);
            if (col >= n) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * (MI * wm + i) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) out[(int64_t)(row - rb) * ld + (col - cb)] = acc[i][j][r] * scur[j];
            }
        }
}


// y += part 0 + part 1 + ... over the split tiles: thread q takes values
// 4 (q % 8192) .. + 3 of tile block q / 8192 (tile t_full + q / 8192, 256 x
// 128 values, row-major) from every part in part order; values outside y
// (ragged edges) are skipped.
__global__ __launch_bounds__(256) void k_qgemm_sum(float* __restrict__ y, const float* __restrict__ ws, int m,
                                                   int n, int tiles_n, int t_full, int nrem, int parts) {
    constexpr int TB = Q2_BM * Q2_BN;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)nrem * (TB / 4)) return;
    const int u = (int)(q / (TB / 4)), e = 4 * (int)(q % (TB / 4));
    const int t = t_full + u;
    const int row = (t / tiles_n) * Q2_BM + e / Q2_BN, col = (t % tiles_n) * Q2_BN + e % Q2_BN;
    if (row >= m || col >= n) return;
    const float* src = ws + (int64_t)u * TB + e;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float* yr = y + (int64_t)row * n + col;
    const bool whole = (n & 3) == 0 && col + 4 <= n;
    if (whole) {
        a = *reinterpret_cast<const float4*>(yr);
    } else {
        a.x = yr[0];
        if (col + 1 < n) a.y = yr[1];
        if (col + 2 < n) a.z = yr[2];
        if (col + 3 < n) a.w = yr[3];
    }
    for (int p = 0; p < parts; ++p) {
        const float4 b = *reinterpret_cast<const float4*>(src + (int64_t)p * nrem * TB);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    if (whole) {
        *reinterpret_cast<float4*>(yr) = a;
    } else {
        yr[0] = a.x;
        if (col + 1 < n) yr[1] = a.y;
        if (col + 2 < n) yr[2] = a.z;
        if (col + 3 < n) yr[3] = a.w;
    }
}

}  // namespace

// How the 256 x 128-tile kernels split K: the first t_full tiles whole, the
// other tiles `splits` ways (splits = 1: no split, t_full = all tiles).
// Chosen by a cost model in microseconds fitted to k_qgemm_v2's timings on
// the Qwen3-4B-shaped launches at m = 512 and 4096 (split counts 1..8
// forced): workgroups run in rounds of one per compute unit; a round costs
// 10 us (start, pipeline fill and drain, output stores) plus 2.2 us per
// 128-block of its workgroups; a split adds the sum launch, 2 us plus S + 1
// reads or writes of the split tiles' fp32 values at 5 TB/s.  The
// candidates: no split; every tile split S ways; the tiles of the full rounds
// whole and those of the last, partial round split S ways (run after the
// full rounds, they fill it).  A split is taken when the model gives 8% or
// more.  The 4-wave kernel (two workgroups per unit) takes the same plans:
// timed with them it is ahead of k_qgemm_v2 on every Qwen3-4B product at
// m = 4096 and level at m = 512, and the plans keep the workspace of every
// Qwen3-4B product at m = 512 within the allocation-free scratch.
QgPlan qgemm_plan(int64_t n, int64_t k, int64_t m, size_t ws_bytes) {
    const int64_t tiles = ((n + Q2_BN - 1) / Q2_BN) * ((m + Q2_BM - 1) / Q2_BM), nbk = k / 128;
    const int64_t cus = compute_units();
    const double per_block = 2.2;
    const double tb = (double)Q2_BM * Q2_BN * 4;                   // bytes of a tile block
    const QgPlan none = {tiles, 1};
    auto fits = [&](int64_t t_full, int64_t sp) {
        return sp >= 1 && sp <= std::min<int64_t>(8, nbk) && t_full >= 0 && t_full < tiles &&
               (double)(sp - 1) * (double)(tiles - t_full) * tb <= (double)ws_bytes;
    };
    auto rt = [&](double blocks) { return 10.0 + per_block * blocks; };
    auto per = [&](int64_t sp) { return (double)((nbk + sp - 1) / sp); };
    auto sum_cost = [&](int64_t nrem, int64_t sp) { return 2.0 + (double)(sp + 1) * (double)nrem * tb / 5e6; };
    const double c1 = (double)((tiles + cus - 1) / cus) * rt((double)nbk);
    QgPlan best = none;
    double cbest = c1;
    for (int64_t sp = 2; sp <= 8; ++sp) {
        if (fits(0, sp)) {                                          // every tile
            const double c = (double)((tiles * sp + cus - 1) / cus) * rt(per(sp)) + sum_cost(tiles, sp);
            if (c < cbest) { cbest = c; best = {0, (int)sp}; }
        }
        const int64_t full = (tiles / cus) * cus, rem = tiles - full;
        if (full > 0 && rem > 0 && fits(full, sp)) {                // the last round's tiles
            const double c = (double)(full / cus) * rt((double)nbk) +
                             (double)((rem * sp + cus - 1) / cus) * rt(per(sp)) + sum_cost(rem, sp);
            if (c < cbest) { cbest = c; best = {full, (int)sp}; }
        }
    }
    return cbest <= 0.92 * c1 ? best : none;
}

// A given plan (pg_qgemm_tune): tiles t_full.. split `splits` ways, the split
// count lowered until it fits the 128-blocks, 8 and the workspace.
QgPlan qgemm_forced(int64_t n, int64_t k, int64_t m, size_t ws_bytes, int splits, int64_t t_full) {
    const int64_t tiles = ((n + Q2_BN - 1) / Q2_BN) * ((m + Q2_BM - 1) / Q2_BM), nbk = k / 128;
    const double tb = (double)Q2_BM * Q2_BN * 4;
    if (t_full < 0 || t_full >= tiles) return QgPlan{tiles, 1};
    int64_t sp = std::min<int64_t>(splits, std::min<int64_t>(8, nbk));
    while (sp > 1 && (double)(sp - 1) * (double)(tiles - t_full) * tb > (double)ws_bytes) --sp;
    return sp > 1 ? QgPlan{t_full, (int)sp} : QgPlan{tiles, 1};
}

size_t qgemm_workspace_bytes(int64_t n, int64_t k, int64_t m) {
    const int64_t tiles = ((n + Q2_BN - 1) / Q2_BN) * ((m + Q2_BM - 1) / Q2_BM);
    const QgPlan p = qgemm_plan(n, k, m, (size_t)-1 / 2);
    return (size_t)(p.splits - 1) * (size_t)(tiles - p.t_full) * (size_t)(Q2_BM * Q2_BN) * 4;
}

int launch_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x,
                 int64_t m, float* y, void* workspace, size_t ws_bytes, pg_stream_t s, int kernel, int splits,
                 int64_t first_split) {
    const int64_t tn = (n + Q2_BN - 1) / Q2_BN, tm = (m + Q2_BM - 1) / Q2_BM, tiles = tn * tm;

    // kernel 1, the plain one-buffer kernel (a second implementation, for
    // tests), has its own tiles; every other kernel takes a split plan
    if (kernel != 1) {
        const QgPlan p = !workspace ? QgPlan{tiles, 1}
                         : splits >= 1 ? qgemm_forced(n, k, m, ws_bytes, splits, first_split)
                                       : qgemm_plan(n, k, m, ws_bytes);
        const int64_t nrem = tiles - p.t_full, grid = p.t_full + nrem * p.splits;
        if (grid > (1 << 30)) return fail(PG_ERR_UNSUPPORTED, "m too large");
        const int remap = (p.t_full % 8 == 0 ? 1 : 0) | ((nrem * p.splits) % 8 == 0 ? 2 : 0);
        // The library's choice: the 4-wave 256 x 128-tile kernel with
        // register-decoded operands, two workgroups per compute unit (timed
        // interleaved with the others, medians of five rounds: ahead of
        // k_qgemm_v2 on the Qwen3-4B layer at m = 4096 by 15%, equal at
        // m = 512)
        const int64_t tiles6 = ((n + Q6_BN - 1) / Q6_BN) * tm;
        if (kernel == 0) kernel = 8;
        if (kernel == 6 || kernel == 7) {               // operands decoded in registers: no split, no workspace
            if (tiles6 > (1 << 30)) return fail(PG_ERR_UNSUPPORTED, "m too large");
            const int tn6 = (int)((n + Q6_BN - 1) / Q6_BN), rm6 = tiles6 % 8 == 0 ? 1 : 0;
            if (kernel == 6)
                k_qgemm_v7<4, 8, Q6_BN><<<dim3((unsigned)tiles6), dim3(512), 0, (hipStream_t)s>>>(
                    codes, scales, (int)n, (int)k, x, (int)m, y, tn6, rm6, (int)tiles6, (int)tiles6, 1, nullptr);
            else
                k_qgemm_v7<8, 8, Q6_BN><<<dim3((unsigned)tiles6), dim3(512), 0, (hipStream_t)s>>>(
                    codes, scales, (int)n, (int)k, x, (int)m, y, tn6, rm6, (int)tiles6, (int)tiles6, 1, nullptr);
            return hip_check(hipGetLastError(), "pg_qgemm launch");
        }
        if (kernel == 5) {                              // wide tiles, whole K: no split, no workspace
            if (tiles6 > (1 << 30)) return fail(PG_ERR_UNSUPPORTED, "m too large");
            hipLaunchKernelGGL(k_qgemm_v6, dim3((unsigned)tiles6), dim3(512), 0, (hipStream_t)s, codes, scales,
                               (int)n, (int)k, x, (int)m, y, (int)((n + Q6_BN - 1) / Q6_BN),
                               tiles6 % 8 == 0 ? 1 : 0, (int)tiles6);
            return hip_check(hipGetLastError(), "pg_qgemm launch");
        }
        if (kernel == 8)                                // 256 x 128 tiles of 4 waves, operands decoded in registers
            k_qgemm_v7<8, 4, Q2_BN><<<dim3((unsigned)grid), dim3(256), 0, (hipStream_t)s>>>(
                codes, scales, (int)n, (int)k, x, (int)m, y, (int)tn, remap, (int)tiles, (int)p.t_full, p.splits,
                static_cast<float*>(workspace));
        else if (kernel == 3)
            hipLaunchKernelGGL(k_qgemm_v4, dim3((unsigned)grid), dim3(1024), 0, (hipStream_t)s, codes, scales,
                               (int)n, (int)k, x, (int)m, y, (int)tn, remap, (int)tiles, (int)p.t_full, p.splits,
                               static_cast<float*>(workspace));
        else if (kernel == 2)
            hipLaunchKernelGGL(k_qgemm_v3, dim3((unsigned)grid), dim3(768), 0, (hipStream_t)s, codes, scales,
                               (int)n, (int)k, x, (int)m, y, (int)tn, remap, (int)tiles, (int)p.t_full, p.splits,
                               static_cast<float*>(workspace));
        else
            hipLaunchKernelGGL(k_qgemm_v2, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)s, codes, scales,
                               (int)n, (int)k, x, (int)m, y, (int)tn, remap, (int)tiles, (int)p.t_full, p.splits,
                               static_cast<float*>(workspace));
        const int rc = hip_check(hipGetLastError(), "pg_qgemm launch");
        if (rc != PG_OK || p.splits == 1) return rc;
        const int64_t blocks = nrem * (Q2_BM * Q2_BN / 4) / 256;
        hipLaunchKernelGGL(k_qgemm_sum, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)s, y,
                           static_cast<const float*>(workspace), (int)m, (int)n, (int)tn, (int)p.t_full, (int)nrem,
                           p.splits - 1);
        return hip_check(hipGetLastError(), "pg_qgemm split sum launch");
    }
    const dim3 grid((unsigned)((n + QG_BN - 1) / QG_BN), (unsigned)((m + QG_BM - 1) / QG_BM));
    if (grid.y > 65535) return fail(PG_ERR_UNSUPPORTED, "m too large");
    hipLaunchKernelGGL(k_qgemm_v1, grid, dim3(256), 0, (hipStream_t)s, codes, scales, (int)n, (int)k, x, (int)m, y);
    return hip_check(hipGetLastError(), "pg_qgemm launch");
}

// ---------------------------------------------------- allocation-free variant
// The split-K workspace of pg_qgemm_noalloc: a device array in the library's
// code object, one copy per GPU the library runs on, held until the process
// ends.  In host code `scratch` is only a stand-in for the symbol; its device
// address is looked up once per device (hipGetSymbolAddress) and only that
// address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[QGEMM_SCRATCH_BYTES];

namespace {
std::mutex scratch_mu;
void* scratch_addr[64] = {};
}  // namespace

int qgemm_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PG_ERR_HIP, "pg_qgemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(PG_ERR_UNSUPPORTED, "pg_qgemm_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PG_ERR_HIP, "pg_qgemm_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return PG_OK;
}

}  // namespace pg
