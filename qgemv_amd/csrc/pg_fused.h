// Fused stage of a stack for gfx950 (MI355X, wave64): rotation, RMS
// normalisation and the product y = W~ . R . n(x) in one launch, for P8F v1
// codes and for codes of the carried-state variant (a compile-time switch,
// so each format's instances carry no code of the other).
//
// Method: "Pingala-8" landing page, section "How it works" (trellis decode
// and random Hadamard rotation); the carried-state variant is the
// small-state coset-trellis design of the landing page's section "Paper".
// Bit layout: include/pingala.h.
#pragma once
#include "pg_device.h"

namespace pg {

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

// launch shape for n rows of k columns at the given batch (pg_fused.hip)
int fused_shape(int64_t n, int64_t k, int batch, FusedShape* out);

namespace {

constexpr int FS_PITCH = 144;      // LDS bytes per 64-value chunk of digits (128 + 16 against bank conflicts)
constexpr int FS_CPREV = 64 * 16 * 4;   // carried state: one dword per (team, row slot)
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
           (size_t)((k / 8 + 15) & ~15) + (size_t)S.BT * S.R * S.CG * 4 + (size_t)S.BT * S.W * 4 + FS_CPREV;
}

// Element of a 128-block held by accumulator row M = 8 i + 4 h + r of row
// tile mt: quarter mt, part i / 2 of the quarter, group r, position
// 2 (i % 2) + h.
__device__ __forceinline__ int fs_elem(int mt, int M) {
    const int i = M >> 3, h = (M >> 2) & 1, r = M & 3;
    return 32 * mt + 16 * (i >> 1) + 4 * r + 2 * (i & 1) + h;
}

typedef _Float16 fs_f16x8 __attribute__((ext_vector_type(8)));

// A operand patterns of the Hadamard product (see fs_elem): lane l holds
// row M = l % 32 and inputs 8 (l / 32) + t of a 16-wide step; the entry is
//   (-1)^popcount(e & 7 & t) (-1)^(bit 3 of e & l / 32)   (fixed per lane)
//   (-1)^(bit 4 of e & step % 2)                            (odd steps)
//   (-1)^popcount(mt & step / 2)                            (uniform)
__device__ __forceinline__ void fs_apat(int lane, uint32_t (&apat)[2][4]) {
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

// One 32 x 32 rotation tile: the rows of quarter mt of H_128 (ordered as
// fs_elem) times 32 staged fp16 blocks, one per lane column (lane % 32);
// xr is this lane's block plus 16 (lane / 32) bytes, bok whether the block
// exists (else zeros).  The B operands are read first, for one LDS wait.
__device__ __forceinline__ f32x16 fs_rot_tile(const uint8_t* xr, bool bok, int mt, const uint32_t (&apat)[2][4]) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    uint4 bv[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) bv[st] = *reinterpret_cast<const uint4*>(xr + 32 * st);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const uint4 bw = bok ? bv[st] : make_uint4(0, 0, 0, 0);
        const uint32_t fl = (__builtin_popcount(mt & (st >> 1)) & 1) ? 0x80008000u : 0u;
        const uint32_t* av = apat[st & 1];
        const uint4 aw = make_uint4(av[0] ^ fl, av[1] ^ fl, av[2] ^ fl, av[3] ^ fl);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(fs_f16x8, aw), __builtin_bit_cast(fs_f16x8, bw),
                                                     acc, 0, 0, 0);
    }
    return acc;
}

// Instances that loop over batch tiles themselves (the codes stay in
// registers); the others get one launch per tile.  The loop keeps more
// values live, so only instances with registers to spare have it.
__host__ __device__ constexpr bool fused_loops(int RS, int BTM) {
    return BTM > 1 && RS * BTM <= 16 && !(RS == 2 && BTM == 8);
}

template <int XDT, int XG, int RS, int BTM, bool CARRY>
__global__ __launch_bounds__(512) void k_rot_qgemv(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales,
                                                    const void* __restrict__ x,
                                                    const uint8_t* __restrict__ sign_bits,
                                                    float* __restrict__ y, int n, uint32_t kword, int ldx32,
                                                    uint32_t shape) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // 14 argument dwords, all preloaded into scalar registers (fused_arg_words)
    const int k = (int)(kword & 0xffffu), batch = (int)((kword >> 16) & 0xfu), BT = (int)((kword >> 20) & 0xfu);
    const uint32_t flags = ((kword >> 24) & 1u) ? (uint32_t)PG_FLAG_RMSNORM : 0u;
    const int64_t ldx = ldx32;
    const int R = (int)(shape & 0x7ffu), CG = (int)((shape >> 11) & 0x7fu), RP = (int)((shape >> 18) & 0x7fu);
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
    uint32_t* cprev = reinterpret_cast<uint32_t*>(wsum + (size_t)BT * W);  // [64 teams][16 row slots]: last
                                                                           // code dword of each team's chunks
    const bool norm = (flags & PG_FLAG_RMSNORM) != 0;
    float rk = 1.0f / (float)k;
    asm volatile("" : "+v"(rk));                      // computed here, before any wait (the
                                                      // compiler would sink it past the barrier)
    constexpr bool carry = CARRY;                      // codes of the carried-state variant

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
    int rowj[RS];
    bool rok[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
        const int r = rp + j * RP;
        rok[j] = col_ok && r < R && row0 + r < n;
        rowj[j] = rok[j] ? row0 + r : (row0 < n ? row0 : n - 1);
    }
    asm volatile("" ::: "memory");
    // The scale of a chunk: a 16-bit load into a whole register (converted
    // only where it is used).
    uint4 q[RS];
    uint32_t wsr[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
        const int row = rowj[j];
        q[j] = *reinterpret_cast<const uint4*>(codes + (int64_t)row * kg + 16 * cc);
        wsr[j] = scales[(int64_t)row * nbk + (cc >> 1)];
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * RS));      // x copies and sign loads done
    if (sg_on) reinterpret_cast<uint32_t*>(sbuf)[tid] = sg;
    __syncthreads();

    uint32_t apat[2][4];                                     // A operand patterns of the Hadamard product
    fs_apat(lane, apat);
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
                inv = rms_inv(tot, rk);
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
            const f32x16 acc = fs_rot_tile(xr, bok, mt, apat);
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
            // Carried-state codes: a team's first chunk (tl = 0) starts a block
            // whose state comes from the chunk before it, the last chunk of the
            // team before (T - 1: the same rows, column group cg - 1), which can
            // sit in another wave: every team's last lane leaves its chunks'
            // last dwords in LDS.
            if (carry) {
                if (tl == 7)
#pragma unroll
                    for (int j = 0; j < RS; ++j) cprev[16 * T + j] = qb[j].w;
                __syncthreads();
            }
            // the neighbour dword ahead of this lane's chunk: the left lane's (odd
            // chunk, or an even one of carried-state codes), from LDS (a team's
            // first chunk of carried-state codes), or none (a block start)
            const uint32_t left_mask = ((c & 1) || (carry && c > 0)) ? ~0u : 0u;
            const bool cp_lane = carry && tl == 0 && c > 0;
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
                        // last dword of the left neighbour's chunk (same row, chunk c - 1):
                        // within the block, or across a block start for carried-state codes
                        const uint32_t left = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb[j].w, 0x111, 0xf, 0xf, true);
                        if (carry) {                                 // uniform
                            // cp_lane implies cg > 0, so T > 0 there; team 0 reads slot 0, unused
                            const uint32_t cpj = cprev[16 * (T > 0 ? T - 1 : 0) + j];
                            prev = cp_lane ? cpj : (left & left_mask);
                        } else {
                            prev = left & left_mask;
                        }
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
                const float wsc = h2f((uint16_t)wb[j]);
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


// The arguments of k_rot_qgemv in 14 dwords, so that the hardware preloads
// all of them into scalar registers (the build asks for preloading; the
// argument-segment pointer takes 2 of the 16 user registers) and no wave
// waits for a scalar load before its first requests: k (16 bits), the
// launch's batch rows and BT (4 bits each) and the RMS flag in one word; R,
// CG and RP (11, 7 and 7 bits) in another; ldx in 32 bits.  False when a
// value does not fit.
__host__ inline bool fused_arg_words(const FusedShape& S, int64_t k, int bt, int64_t ldx, uint32_t flags,
                                     uint32_t* kword, uint32_t* shape) {
    if (k >= 65536 || bt < 0 || bt >= 16 || S.BT >= 16 || ldx < 0 || ldx > 0x7fffffff || S.R >= 2048 ||
        S.CG >= 128 || S.RP >= 128)
        return false;
    *kword = (uint32_t)k | ((uint32_t)bt << 16) | ((uint32_t)S.BT << 20) | ((flags & PG_FLAG_RMSNORM) ? 1u << 24 : 0u);
    *shape = (uint32_t)S.R | ((uint32_t)S.CG << 11) | ((uint32_t)S.RP << 18);
    return true;
}

template <int XDT, int XG, int RS, int BTM, bool CARRY>
int launch_fused_t(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                   const void* x, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                   hipStream_t st) {
    const dim3 grid((unsigned)((n + S.R - 1) / S.R));
    const int esz = XDT == PG_F32 ? 4 : 2;
    const int tile = fused_loops(RS, BTM) ? batch : S.BT;  // rows handed to one launch
    for (int b0 = 0; b0 < batch; b0 += tile) {
        const int bt = batch - b0 < tile ? batch - b0 : tile;
        const void* xb = (const uint8_t*)x + (int64_t)b0 * ldx * esz;
        uint32_t kword, shape;
        if (!fused_arg_words(S, k, bt, ldx, flags, &kword, &shape))
            return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv: shape n=%lld k=%lld ldx=%lld out of the kernel's range",
                        (long long)n, (long long)k, (long long)ldx);
        hipLaunchKernelGGL((k_rot_qgemv<XDT, XG, RS, BTM, CARRY>), grid, dim3(64 * S.W), fused_lds_bytes((int)k, esz, S),
                           st, codes, scales, xb, sign_bits, y + (int64_t)b0 * n, (int)n, kword, (int)ldx, shape);
        const int rc = hip_check(hipGetLastError(), "pg_rot_qgemv launch");
        if (rc != PG_OK) return rc;
    }
    return PG_OK;
}

// (rows per lane, batch rows per launch) combinations that fit the register
// budget (RS * BTM <= 32, and RS <= 2 for 8 rows)
template <int XDT, int XG, bool CARRY>
int launch_fused_rs(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                    const void* x, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                    hipStream_t st) {
#define PG_FUSED(RS_, BTM_) return launch_fused_t<XDT, XG, RS_, BTM_, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st)
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

// every (x dtype, x groups per thread) instance set, for one of the two formats
template <bool CARRY>
int launch_fused_all(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                     const void* x, int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch,
                     float* y, hipStream_t st) {
    if (x_dt == PG_F32) {
        if (S.XG <= 1) return launch_fused_rs<PG_F32, 1, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
        if (S.XG <= 2) return launch_fused_rs<PG_F32, 2, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
        return launch_fused_rs<PG_F32, 4, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    }
    if (S.XG <= 1) return launch_fused_rs<PG_F16, 1, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    if (S.XG <= 2) return launch_fused_rs<PG_F16, 2, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
    return launch_fused_rs<PG_F16, 4, CARRY>(S, codes, scales, n, k, x, ldx, sign_bits, flags, batch, y, st);
}

}  // namespace

// batch 4..8 on the int8 matrix cores (pg_fused_mma.hip): the same stage
// with activations quantised per 128-block; PG_ERR_UNSUPPORTED (message not
// set) when the shape does not fit it
int launch_rot_qmma(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dt,
                    int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y, hipStream_t st);

// batch 1 on P8F v1 codes (pg_fused1.hip): the stage with the rotation in
// registers; PG_ERR_UNSUPPORTED (message set) when the shape does not fit it
int launch_rot_qgemv1(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dt,
                      const uint8_t* sign_bits, uint32_t flags, float* y, hipStream_t st);

// batch 1 through a codebook table (pg_fused1.hip): the same stage with the
// table-driven decode, k <= 16384; PG_ERR_UNSUPPORTED (message set) when the
// shape does not fit it
int launch_rot_qgemv1_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                            int x_dt, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                            hipStream_t st);

// the carried-state instances (pg_fused_carry.hip, compiled on their own)
int launch_fused_carry(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const void* x, int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch,
                       float* y, hipStream_t st);

}  // namespace pg
