// HIP kernels of libpingala for gfx950 (MI355X, wave64): trellis decode,
// the run-time Hadamard rotation and the batch-1..8 product (qgemv).  The
// fused stage is in pg_fused.h, the prompt product in pg_qgemm.hip.
//
// Method: "Pingala-8" landing page, section "How it works" -- an 8-state
// Ungerboeck trellis over groups of 4 weights, the state carried from group
// to group choosing the value set of the next group, plus a random Hadamard
// rotation.  Bit layout: format P8F v1 as stated in include/pingala.h.
#include "pg_device.h"

namespace pg {
namespace {

// ------------------------------------------------------------------ decode
// One thread per code byte; the state comes from the bit 0 of the previous
// (at most three) bytes of the same 128-block, or of the same row for codes
// of the carried-state variant.  w = fp32(scale) * level is exact, so the
// output is bit-identical to any exact decoder.
__global__ void k_decode(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                         int64_t total_groups, int kg, int carry, float* __restrict__ w) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total_groups) return;
    const int64_t row = g / kg;
    const int t = (int)(g - row * kg);
    const int tb = carry ? t : (t & 31);          // groups of this trellis path before group t
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

// Decode through a codebook table T[s][byte] (four int8 levels per entry):
// the workgroup stages the 8 KB table in LDS, then each thread decodes
// groups as k_decode does, one table lookup per group; the state follows
// P8F v1's trellis or the rate-2/3 one.
constexpr int DT_GROUPS = 16;                 // groups per thread

__global__ __launch_bounds__(256) void k_decode_table(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales, int64_t total_groups,
                                                      int kg, int carry, int rate23,
                                                      const uint4* __restrict__ table, float* __restrict__ w) {
    __shared__ uint4 tab[512];
    tab[threadIdx.x] = table[threadIdx.x];
    tab[threadIdx.x + 256] = table[threadIdx.x + 256];
    __syncthreads();
    const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tab);
    const int64_t g0 = (int64_t)blockIdx.x * (256 * DT_GROUPS) + threadIdx.x;
    for (int i = 0; i < DT_GROUPS; ++i) {
        const int64_t g = g0 + 256 * i;
        if (g >= total_groups) return;
        const int64_t row = g / kg;
        const int t = (int)(g - row * kg);
        const int tb = carry ? t : (t & 31);
        const uint8_t* rp = codes + row * kg;
        const uint32_t c = rp[t];
        uint32_t st;
        if (rate23) {                             // previous byte's two branch bits, u0 of the one before
            st = (tb >= 1 ? (rp[t - 1] & 3u) : 0u) | (tb >= 2 ? (rp[t - 2] & 1u) << 2 : 0u);
        } else {                                  // the three previous branch bits
            st = (tb >= 1 ? (rp[t - 1] & 1u) : 0u) | (tb >= 2 ? (rp[t - 2] & 1u) << 1 : 0u) |
                 (tb >= 3 ? (rp[t - 3] & 1u) << 2 : 0u);
        }
        const uint32_t pt = t32[(st << 8) | c];
        const float s = h2f(scales[row * (kg / 32) + (t >> 5)]);
        float4 o;
        o.x = s * (float)(int8_t)(pt & 0xffu);
        o.y = s * (float)(int8_t)((pt >> 8) & 0xffu);
        o.z = s * (float)(int8_t)((pt >> 16) & 0xffu);
        o.w = s * (float)(int8_t)(pt >> 24);
        reinterpret_cast<float4*>(w)[g] = o;
    }
}

// ---------------------------------------------------------------- rotation
// Grid (ceil(nblocks/4), rows): each of the 4 waves of a workgroup transforms
// one 128-block; lane l holds elements l and l+64, the first butterfly stage
// (distance 64) is inside the lane, the other six exchange across lanes.
// With PG_FLAG_RMSNORM every workgroup first sums the squares of its whole
// row (fixed order: strided per thread, then waves 0..3) and rounds the
// normalised values to fp16.  PG_Q16 output writes the 16-bit fixed-point
// activation format that pg_qgemv reads (layout in include/pingala.h).

__device__ __forceinline__ void q16_store(uint8_t* row, int k, int blk, int i, int q) {
    // element i of block blk: chunk c' = i/16, group g = (i/4)%4, position j = i%4
    const int hi = (q + 128) >> 8;
    const int lo = q - (hi << 8);
    const int off = (blk * 8 + (i >> 4)) * 32 + 4 * (i & 3) + ((i >> 2) & 3);
    row[off] = (uint8_t)(int8_t)hi;
    row[off + 16] = (uint8_t)(int8_t)lo;
}

// squares of the 4 (fp32) or 8 (fp16, bf16) values of a 16-byte vector, in order
template <int IDT>
__device__ __forceinline__ float sq16(const uint4 w) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if constexpr (IDT == PG_F32) {
            const float f = __builtin_bit_cast(float, v[t]);
            s += f * f;
        } else {
            const float f0 = IDT == PG_F16 ? h2f((uint16_t)(v[t] & 0xffffu)) : bf2f((uint16_t)(v[t] & 0xffffu));
            const float f1 = IDT == PG_F16 ? h2f((uint16_t)(v[t] >> 16)) : bf2f((uint16_t)(v[t] >> 16));
            s += f0 * f0;
            s += f1 * f1;
        }
    }
    return s;
}

// (arguments in 14 dwords, the 8-byte ones first: the hardware preloads all
// of them into scalar registers, so no wave waits for a scalar load)
template <int IDT>
__global__ __launch_bounds__(256) void k_fwht(const void* __restrict__ x, void* __restrict__ y,
                                              const uint8_t* __restrict__ sign_bits, int64_t ldx,
                                              int64_t q16_stride, int out_dt, int k, uint32_t flags, int vec) {
    constexpr int in_dt = IDT;
    const int64_t row = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nblk = k >> 7;
    const int blk = blockIdx.x * 4 + wave;
    const int64_t xbase = row * ldx;                          // row of x (ldx elements apart)
    const int64_t base = row * (int64_t)k;                    // row of an fp output
    __shared__ float red[4];
    const float rk = 1.0f / (float)k;
    // this wave's block first (its loads overlap the normalisation pass)
    const bool active = blk < nblk;
    const int i0 = (active ? blk : 0) * 128 + lane, i1 = i0 + 64;
    float a = load_elem(x, in_dt, xbase + i0);
    float c = load_elem(x, in_dt, xbase + i1);
    const uint32_t sg0 = sign_bits[i0 >> 3], sg1 = sign_bits[i1 >> 3];
    float inv = 1.0f;
    if ((flags & PG_FLAG_RMSNORM) && vec) {
        // the whole row's squares, rows 16-byte aligned: 16-byte vectors
        // t + 256 u, up to 16 per thread in flight at once (one round trip
        // for k <= 16384 at fp32; the sum runs over u in the same order)
        constexpr int per = IDT == PG_F32 ? 4 : 8;
        const int nv = k / per;
        const uint4* xv = reinterpret_cast<const uint4*>((const uint8_t*)x + xbase * (IDT == PG_F32 ? 4 : 2));
        float ss = 0.0f;
        for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * 16) {
            uint4 w[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int v = v0 + 256 * u;
                w[u] = v < nv ? xv[v] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) ss += sq16<IDT>(w[u]);
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        inv = rms_inv(tot, rk);
    } else if (flags & PG_FLAG_RMSNORM) {
        // the whole row's squares: up to 64 loads per thread in flight at once
        float ss = 0.0f;
        for (int i0r = threadIdx.x; i0r < k; i0r += 256 * 64) {
            float v[64];
#pragma unroll
            for (int u = 0; u < 64; ++u) {
                const int i = i0r + 256 * u;
                v[u] = i < k ? load_elem(x, in_dt, xbase + i) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 64; ++u) ss += v[u] * v[u];
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        inv = rms_inv(tot, rk);
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
                                                   float* __restrict__ y, int nthr) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // the block size as an argument (13 dwords, all preloaded into scalar
    // registers) rather than from the dispatch's hidden arguments, which
    // would cost a scalar load at entry
    const int tid = threadIdx.x;
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

// ----------------------------------------------------------- streaming read
// The HBM ceiling a plain streaming kernel reaches: every thread reads 16-byte
// words in a grid-stride sweep with four requests in flight and XORs them;
// each workgroup folds its XOR into *out with one atomic (XOR does not depend
// on the order, so the result is exact and checkable).
__global__ __launch_bounds__(256) void k_hbm_read(const uint4* __restrict__ p, int64_t n16, uint32_t* out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    acc = (uint32_t)wave_xor(acc);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicXor(out, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

}  // namespace

int launch_hbm_read(const void* p, int64_t bytes, uint32_t* out, pg_stream_t s) {
    const int64_t n16 = bytes / 16;
    int64_t grid = (int64_t)compute_units() * 32;
    if (grid > (n16 + 255) / 256) grid = (n16 + 255) / 256;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_hbm_read, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)s, (const uint4*)p, n16, out);
    return hip_check(hipGetLastError(), "pg_hbm_read launch");
}

int launch_decode(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, float* w,
                  bool carry, pg_stream_t s) {
    const int64_t total = n * (k / 4);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_decode, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)s, codes, scales, total,
                       (int)(k / 4), carry ? 1 : 0, w);
    return hip_check(hipGetLastError(), "pg_decode launch");
}

int launch_decode_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const int8_t* table,
                        bool carry, bool rate23, float* w, pg_stream_t s) {
    const int64_t total = n * (k / 4);
    const int64_t blocks = (total + 256 * DT_GROUPS - 1) / (256 * DT_GROUPS);
    if (blocks > 0x7fffffff) return fail(PG_ERR_UNSUPPORTED, "pg_decode_table: too many groups");
    hipLaunchKernelGGL(k_decode_table, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)s, codes, scales, total,
                       (int)(k / 4), carry ? 1 : 0, rate23 ? 1 : 0, reinterpret_cast<const uint4*>(table), w);
    return hip_check(hipGetLastError(), "pg_decode_table launch");
}

int launch_fwht(const void* x, int in_dt, int64_t ldx, void* y, int out_dt, const uint8_t* sign_bits,
                int64_t rows, int64_t k, uint32_t flags, pg_stream_t s) {
    if (rows > 65535) return fail(PG_ERR_UNSUPPORTED, "rows > 65535");
    const dim3 grid((unsigned)((k / 128 + 3) / 4), (unsigned)rows);
    // 16-byte loads for the RMS pass where every row starts 16-byte aligned
    const int vec = (ldx * (in_dt == PG_F32 ? 4 : 2)) % 16 == 0 && (uintptr_t)x % 16 == 0;
    const int64_t qs = (int64_t)q16_row_bytes(k);
    hipStream_t st = (hipStream_t)s;
    if (in_dt == PG_F32)
        hipLaunchKernelGGL(k_fwht<PG_F32>, grid, dim3(256), 0, st, x, y, sign_bits, ldx, qs, out_dt, (int)k, flags, vec);
    else if (in_dt == PG_F16)
        hipLaunchKernelGGL(k_fwht<PG_F16>, grid, dim3(256), 0, st, x, y, sign_bits, ldx, qs, out_dt, (int)k, flags, vec);
    else
        hipLaunchKernelGGL(k_fwht<PG_BF16>, grid, dim3(256), 0, st, x, y, sign_bits, ldx, qs, out_dt, (int)k, flags, vec);
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
                           stride, batch, y, 64 * W);
    else
        hipLaunchKernelGGL((k_qgemv_q16<BS, 1>), grid, dim3(64 * W), lds, st, codes, scales, (int)n, (int)k, xq,
                           stride, batch, y, 64 * W);
    return hip_check(hipGetLastError(), "pg_qgemv launch");
}

}  // namespace

int launch_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                 int x_dt, int batch, uint32_t kflags, float* y, pg_stream_t s) {
    if (x_dt == PG_Q16) {
        // batch 2..8: the matrix-core kernel, whose vector work per weight
        // does not grow with the batch (PG_FLAG_KERNEL_VDOT keeps the v_dot4
        // kernel, PG_FLAG_KERNEL_MMA takes the matrix cores at any batch)
        const bool force_q16 = (kflags & PG_FLAG_KERNEL_VDOT) != 0, force_mma = (kflags & PG_FLAG_KERNEL_MMA) != 0;
        if (force_mma || (!force_q16 && batch >= 2))
            return launch_qgemv_mma(codes, scales, n, k, (const uint8_t*)x, batch, y, s);
        const int stride = (int)q16_row_bytes(k);
        // rows per workgroup 8*R; waves per workgroup W split each row's
        // 64-weight chunks, chosen so that the launch has about 2048+ waves
        // while every lane still gets at least one chunk
        int R = 1;
        const int64_t wgs = (n + 7) / 8;
        int W = 1;
        while (W < 8 && wgs * W < 2048 && (k / 64) >= 16 * W) W *= 2;
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

}  // namespace pg
