// Launch side of the batch-1 fused stage (pg_fused1.h): P8F v1 codes with the
// closed-form decode, and codes read through a codebook table.
#include "pg_fused1.h"

namespace pg {

// Launch shape of the batch-1 stage (pg_fused1.h): about one workgroup per
// CU, each with all of its rows' codes in registers (at most 16 rows per
// lane), four 128-blocks per wave and rotation round, at most umax rounds.
int fused1_shape(int64_t n, int64_t k, int umax, bool table, Fused1Shape* out) {
    Fused1Shape S;
    S.W = 8;                                           // the kernel assumes 512 threads
    const int nchunk = (int)(k / 64), nbk = (int)(k / 128);
    S.CG = (nchunk + 7) / 8;
    S.U = (nbk + 4 * S.W - 1) / (4 * S.W);
    if (S.CG > 8 * S.W || S.U > umax) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for the batch-1 stage", (long long)k);
    S.RP = 8 * S.W / S.CG;
    const int64_t cus = compute_units();
    int64_t R = (n + cus - 1) / cus;
    // at most 16 rows per lane; 10 through a table, whose lookups in flight
    // hold more registers per row (12 rows spill)
    const int rs_max = table ? 10 : 16;
    if (R > rs_max * S.RP) R = rs_max * S.RP;
    if (R > n) R = n;
    S.R = (int)R;
    S.RS = (S.R + S.RP - 1) / S.RP;
    if (fused1_lds_bytes((int)k, S, table) > 160 * 1024)
        return fail(PG_ERR_UNSUPPORTED, "shape n=%lld k=%lld does not fit the batch-1 stage", (long long)n, (long long)k);
    // the fields of fused1_shape_word (R <= 16 RP <= 1024, CG and RP <= 64, U <= 4 here)
    if (S.R >= 2048 || S.CG >= 128 || S.RP >= 128 || S.U >= 128)
        return fail(PG_ERR_UNSUPPORTED, "shape n=%lld k=%lld does not fit the batch-1 stage", (long long)n, (long long)k);
    *out = S;
    return PG_OK;
}

int launch_rot_qgemv1(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dt,
                      const uint8_t* sign_bits, uint32_t flags, float* y, hipStream_t st) {
    Fused1Shape S;
    const int rc = fused1_shape(n, k, F1_UMAX, false, &S);
    if (rc != PG_OK) return rc;
    if (x_dt == PG_F32) return launch_fused1_rs<PG_F32, 0, F1_UMAX>(S, codes, scales, n, k, x, sign_bits, nullptr, flags, y, st);
    return launch_fused1_rs<PG_F16, 0, F1_UMAX>(S, codes, scales, n, k, x, sign_bits, nullptr, flags, y, st);
}

// the table stage: one rotation round where k <= 4096 (fewer registers
// held), up to four beyond
int launch_rot_qgemv1_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                            int x_dt, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                            hipStream_t st) {
    Fused1Shape S;
    const int rc = fused1_shape(n, k, F1T_UMAX, true, &S);
    if (rc != PG_OK) return rc;
    const uint32_t* t = reinterpret_cast<const uint32_t*>(table);
    if (flags & PG_FLAG_RATE23) return launch_table_r23(S, codes, scales, n, k, x, x_dt, sign_bits, t, flags, y, st);
    if (S.U <= 1) {
        if (x_dt == PG_F32) return launch_fused1_rs<PG_F32, 1, 1>(S, codes, scales, n, k, x, sign_bits, t, flags, y, st);
        return launch_fused1_rs<PG_F16, 1, 1>(S, codes, scales, n, k, x, sign_bits, t, flags, y, st);
    }
    if (x_dt == PG_F32) return launch_fused1_rs<PG_F32, 1, F1T_UMAX>(S, codes, scales, n, k, x, sign_bits, t, flags, y, st);
    return launch_fused1_rs<PG_F16, 1, F1T_UMAX>(S, codes, scales, n, k, x, sign_bits, t, flags, y, st);
}

}  // namespace pg
