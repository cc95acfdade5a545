// Prompt product of libpingala on the gfx950 matrix cores: Y = X . W~^T for
// m rows of bf16 activations X against P8F v1 codes, the weights decoded
// tile by tile into LDS as bf16 levels (small odd integers, exact in bf16).
//
// Method: "Pingala-8" landing page, section "How it works" (the trellis
// decode); bit layout in include/pingala.h.
#include <algorithm>

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

// How the pipelined kernel splits K: the first t_full tiles whole, the other
// tiles `splits` ways (splits = 1: no split, t_full = all tiles).  Chosen by a
// cost model in microseconds fitted to kernel timings of the Qwen3-4B-shaped
// launches at m = 512 and 4096 (split counts 1..8 forced): workgroups run in
// rounds of one per compute unit (the kernel's LDS holds one workgroup per
// unit); a round costs 10 us (start, pipeline fill and drain, output stores)
// plus 2.2 us per 128-block of its workgroups; a split adds the sum launch,
// 2 us plus S + 1 reads or writes of the split tiles' fp32 values at 5 TB/s.
// The candidates: no split; every tile split S ways; the tiles of the full
// rounds whole and those of the last, partial round split S ways (run after
// the full rounds, they fill it).  A split is taken when the model gives 8%
// or more.  PG_QGEMM_SPLITS=S (every tile) or S:T (tiles T.. only) forces a
// plan, still within the 128-blocks and the workspace.
QgPlan qgemm_plan(int64_t n, int64_t k, int64_t m, size_t ws_bytes) {
    const int64_t tiles = ((n + Q2_BN - 1) / Q2_BN) * ((m + Q2_BM - 1) / Q2_BM), nbk = k / 128;
    const int64_t cus = compute_units();
    const double tb = (double)Q2_BM * Q2_BN * 4;                   // bytes of a tile block
    const QgPlan none = {tiles, 1};
    auto fits = [&](int64_t t_full, int64_t sp) {
        return sp >= 1 && sp <= std::min<int64_t>(8, nbk) && t_full >= 0 && t_full < tiles &&
               (double)(sp - 1) * (double)(tiles - t_full) * tb <= (double)ws_bytes;
    };
    if (const char* e = getenv("PG_QGEMM_SPLITS")) {
        long long sp = 0, tf = 0;
        const int got = sscanf(e, "%lld:%lld", &sp, &tf);
        if (got >= 1 && sp > 1) {
            if (got < 2) tf = 0;
            sp = std::min<long long>(sp, std::min<int64_t>(8, nbk));
            while (sp > 1 && !fits(tf, sp)) --sp;
            return sp > 1 ? QgPlan{tf, (int)sp} : none;
        }
        if (got >= 1 && sp == 1) return none;
    }
    auto rt = [](double blocks) { return 10.0 + 2.2 * blocks; };
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

size_t qgemm_workspace_bytes(int64_t n, int64_t k, int64_t m) {
    const int64_t tiles = ((n + Q2_BN - 1) / Q2_BN) * ((m + Q2_BM - 1) / Q2_BM);
    const QgPlan p = qgemm_plan(n, k, m, (size_t)-1 / 2);
    return (size_t)(p.splits - 1) * (size_t)(tiles - p.t_full) * (size_t)(Q2_BM * Q2_BN) * 4;
}

int launch_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x,
                 int64_t m, float* y, void* workspace, size_t ws_bytes, pg_stream_t s) {
    const int64_t tn = (n + Q2_BN - 1) / Q2_BN, tm = (m + Q2_BM - 1) / Q2_BM, tiles = tn * tm;
    // the pipelined kernel is the product; PG_QGEMM_KERNEL=1 selects the
    // plain one-buffer kernel (kept as a second implementation for tests)
    const char* e = getenv("PG_QGEMM_KERNEL");
    if (!(e && atoi(e) == 1)) {
        const QgPlan p = workspace ? qgemm_plan(n, k, m, ws_bytes) : QgPlan{tiles, 1};
        const int64_t nrem = tiles - p.t_full, grid = p.t_full + nrem * p.splits;
        if (grid > (1 << 30)) return fail(PG_ERR_UNSUPPORTED, "m too large");
        const int remap = (p.t_full % 8 == 0 ? 1 : 0) | ((nrem * p.splits) % 8 == 0 ? 2 : 0);
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

}  // namespace pg
