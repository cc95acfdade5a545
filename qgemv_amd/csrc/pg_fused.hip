// Launch side of the fused stage (pg_fused.h): the launch shape and the
// P8F v1 instances; the carried-state ones are in pg_fused_carry.hip.
#include "pg_fused.h"

namespace pg {

// Launch shape of the fused stage: about one workgroup per CU, each with
// all of its rows' codes in registers (at most 16 rows per lane).
int fused_shape(int64_t n, int64_t k, int batch, FusedShape* out) {
    FusedShape S;
    S.W = 8;                                           // the kernel assumes 512 threads
    const int nchunk = (int)(k / 64), nbk = (int)(k / 128);
    S.CG = (nchunk + 7) / 8;
    if (S.CG > 8 * S.W) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    S.RP = 8 * S.W / S.CG;
    S.XG = (int)((k / 8 + 64 * S.W - 1) / (64 * S.W));   // 8-value groups of x per thread
    if (k / 32 > 64 * S.W || S.XG > 4)
        return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    (void)nbk;
    const int64_t cus = compute_units();
    int64_t R = (n + cus - 1) / cus;
    if (R > 16 * S.RP) R = 16 * S.RP;                      // at most 16 rows per lane
    if (R > n) R = n;
    S.R = (int)R;
    S.RS = (S.R + S.RP - 1) / S.RP;
    // batch rows per tile: as many as the LDS holds, up to the template's bound
    // BTM (registers: RS * BTM <= 32, RS <= 2 for 8 rows); with fewer rows
    // per tile than the batch, the kernel loops over tiles itself where its
    // registers allow (fused_loops), else one launch per tile
    const size_t budget = 150 * 1024;
    int bt_lds = 1;                                    // rows of x the LDS holds at once
    for (;;) {
        FusedShape T = S;
        T.BTM = T.BT = bt_lds + 1;
        if (bt_lds >= 8 || fused_lds_bytes((int)k, 4, T) > budget) break;
        ++bt_lds;
    }
    const int t = batch < bt_lds ? batch : bt_lds;
    S.BTM = batch <= 1 ? 1 : S.RS <= 2 ? (t > 4 ? 8 : 4) : S.RS <= 4 ? 4 : S.RS <= 8 ? (t <= 2 ? 2 : 4) : 2;
    S.BT = t < S.BTM ? t : S.BTM;
    if (fused_lds_bytes((int)k, 4, S) > budget) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    *out = S;
    return PG_OK;
}

int launch_rot_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                     int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                     pg_stream_t s) {
    FusedShape S;
    const int rc = fused_shape(n, k, batch, &S);
    if (rc != PG_OK) return rc;
    if (x_dt == PG_F32 && !(flags & PG_FLAG_RMSNORM))
        return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv: fp32 input needs PG_FLAG_RMSNORM (its rotation runs in fp16)");
    hipStream_t st = (hipStream_t)s;
    // batch 2..8 on the matrix cores where the shape fits (PG_FLAG_KERNEL_VDOT
    // keeps the v_dot4 stage, PG_FLAG_KERNEL_MMA takes the matrix cores at
    // any batch)
    const bool carry = (flags & PG_FLAG_CARRY_STATE) != 0;
    const bool force_v = (flags & PG_FLAG_KERNEL_VDOT) != 0, force_m = (flags & PG_FLAG_KERNEL_MMA) != 0;
    if (!carry && !force_v && (force_m || batch >= 2)) {
        const int r = launch_rot_qmma(codes, scales, n, k, x, x_dt, ldx, sign_bits, flags, batch, y, st);
        if (r != PG_ERR_UNSUPPORTED) return r;
    }
    // batch 1 on P8F v1 codes: the register-rotation stage where the
    // rotation is at most one round per wave (k <= 4096); larger k keeps the
    // matrix-core rotation below, which is faster there (k = 9728: 8.5 against
    // 9.1 us per launch)
    if (batch == 1 && !carry && !force_v && k <= 4096)
        return launch_rot_qgemv1(codes, scales, n, k, x, x_dt, sign_bits, flags, y, st);
    if (flags & PG_FLAG_CARRY_STATE)
        return launch_fused_carry(S, codes, scales, n, k, x, x_dt, ldx, sign_bits, flags, batch, y, st);
    return launch_fused_all<false>(S, codes, scales, n, k, x, x_dt, ldx, sign_bits, flags, batch, y, st);
}

int launch_rot_qgemv_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                           int x_dt, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                           pg_stream_t s) {
    if (x_dt == PG_F32 && !(flags & PG_FLAG_RMSNORM))
        return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv_table: fp32 input needs PG_FLAG_RMSNORM (its rotation runs in fp16)");
    return launch_rot_qgemv1_table(codes, scales, n, k, x, x_dt, sign_bits, table, flags, y, (hipStream_t)s);
}

}  // namespace pg
