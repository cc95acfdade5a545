// HIP kernels of libpingala for gfx950 (MI355X, wave64): trellis decode,
// the run-time Hadamard rotation, the batch-1..8 product (qgemv) and the
// prompt product on the matrix cores (qgemm).
//
// Method: "Pingala-8" landing page, section "How it works" -- an 8-state
// Ungerboeck trellis over groups of 4 weights, the state carried from group
// to group choosing the value set of the next group, plus a random Hadamard
// rotation.  Bit layout: format P8F v1 as stated in include/pingala.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// One workgroup (4 waves) per row.  Each wave transforms whole 128-blocks:
// lane l holds elements l and l+64, the first butterfly stage (distance 64)
// is inside the lane, the other six use lane exchanges.  Optional RMS
// normalisation with fp16 rounding first (PG_FLAG_RMSNORM).
__global__ __launch_bounds__(256) void k_fwht(const void* __restrict__ x, int in_dt, void* __restrict__ y,
                                              int out_dt, const uint8_t* __restrict__ sign_bits, int k,
                                              uint32_t flags) {
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t base = row * (int64_t)k;
    __shared__ float red[4];
    float inv = 1.0f;
    if (flags & PG_FLAG_RMSNORM) {
        float ss = 0.0f;
        for (int i = threadIdx.x; i < k; i += 256) {
            const float v = load_elem(x, in_dt, base + i);
            ss += v * v;
        }
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        inv = 1.0f / sqrtf(tot / (float)k + 1e-6f);
    }
    const float cnorm = 0.08838834764831845f;   // 2^-3.5
    for (int b = wave; b < k / 128; b += 4) {
        const int i0 = b * 128 + lane, i1 = i0 + 64;
        float a = load_elem(x, in_dt, base + i0);
        float c = load_elem(x, in_dt, base + i1);
        if (flags & PG_FLAG_RMSNORM) {
            a = h2f(f2h(a * inv));
            c = h2f(f2h(c * inv));
        }
        if ((sign_bits[i0 >> 3] >> (i0 & 7)) & 1) a = -a;
        if ((sign_bits[i1 >> 3] >> (i1 & 7)) & 1) c = -c;
        float t0 = a + c, t1 = a - c;
        a = t0;
        c = t1;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {
            const float pa = __shfl_xor(a, h), pc = __shfl_xor(c, h);
            const bool upper = (lane & h) != 0;
            a = upper ? pa - a : a + pa;
            c = upper ? pc - c : c + pc;
        }
        store_elem(y, out_dt, base + i0, a * cnorm);
        store_elem(y, out_dt, base + i1, c * cnorm);
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
    if (rows > 0x7fffffff) return fail(PG_ERR_UNSUPPORTED, "rows too large");
    hipLaunchKernelGGL(k_fwht, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)s, x, in_dt, y, out_dt,
                       sign_bits, (int)k, flags);
    return hip_check(hipGetLastError(), "pg_fwht_rotate launch");
}

int launch_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                 int x_dt, int batch, float* y, pg_stream_t s) {
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

int launch_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x,
                 int64_t m, float* y, pg_stream_t s) {
    const dim3 grid((unsigned)((n + QG_BN - 1) / QG_BN), (unsigned)((m + QG_BM - 1) / QG_BM));
    if (grid.y > 65535) return fail(PG_ERR_UNSUPPORTED, "m too large");
    hipLaunchKernelGGL(k_qgemm_v1, grid, dim3(256), 0, (hipStream_t)s, codes, scales, (int)n, (int)k, x, (int)m, y);
    return hip_check(hipGetLastError(), "pg_qgemm launch");
}

}  // namespace pg
