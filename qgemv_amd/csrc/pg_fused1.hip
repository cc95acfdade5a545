// Launch side of the batch-1 fused stage (pg_fused1.h), P8F v1 codes.
#include "pg_fused1.h"

namespace pg {

// Launch shape of the batch-1 stage (pg_fused1.h): about one workgroup per
// CU, each with all of its rows' codes in registers (at most 16 rows per
// lane), four 128-blocks per wave and rotation round.
int fused1_shape(int64_t n, int64_t k, Fused1Shape* out) {
    Fused1Shape S;
    S.W = 8;                                           // the kernel assumes 512 threads
    const int nchunk = (int)(k / 64), nbk = (int)(k / 128);
    S.CG = (nchunk + 7) / 8;
    S.U = (nbk + 4 * S.W - 1) / (4 * S.W);
    if (S.CG > 8 * S.W || S.U > F1_UMAX) return fail(PG_ERR_UNSUPPORTED, "k=%lld too large for pg_rot_qgemv", (long long)k);
    S.RP = 8 * S.W / S.CG;
    const int64_t cus = compute_units();
    int64_t R = (n + cus - 1) / cus;
    if (R > 16 * S.RP) R = 16 * S.RP;                  // at most 16 rows per lane
    if (R > n) R = n;
    S.R = (int)R;
    S.RS = (S.R + S.RP - 1) / S.RP;
    if (fused1_lds_bytes((int)k, S) > 160 * 1024)
        return fail(PG_ERR_UNSUPPORTED, "pg_rot_qgemv: shape n=%lld k=%lld does not fit the batch-1 stage", (long long)n,
                    (long long)k);
    *out = S;
    return PG_OK;
}

int launch_rot_qgemv1(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dt,
                      const uint8_t* sign_bits, uint32_t flags, float* y, hipStream_t st) {
    Fused1Shape S;
    const int rc = fused1_shape(n, k, &S);
    if (rc != PG_OK) return rc;
    if (x_dt == PG_F32) return launch_fused1_rs<PG_F32>(S, codes, scales, n, k, x, sign_bits, flags, y, st);
    return launch_fused1_rs<PG_F16>(S, codes, scales, n, k, x, sign_bits, flags, y, st);
}

}  // namespace pg
