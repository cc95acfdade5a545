// The batch-1 stage through a codebook table on the rate-2/3 trellis
// (pg_fused1.h, TAB = 2), compiled apart from the other instances.
#include "pg_fused1.h"

namespace pg {

int launch_table_r23(const Fused1Shape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                     const void* x, int x_dt, const uint8_t* sign_bits, const uint32_t* table, uint32_t flags,
                     float* y, hipStream_t st) {
    if (S.U <= 1) {
        if (x_dt == PG_F32) return launch_fused1_rs<PG_F32, 2, 1>(S, codes, scales, n, k, x, sign_bits, table, flags, y, st);
        return launch_fused1_rs<PG_F16, 2, 1>(S, codes, scales, n, k, x, sign_bits, table, flags, y, st);
    }
    if (x_dt == PG_F32)
        return launch_fused1_rs<PG_F32, 2, F1T_UMAX>(S, codes, scales, n, k, x, sign_bits, table, flags, y, st);
    return launch_fused1_rs<PG_F16, 2, F1T_UMAX>(S, codes, scales, n, k, x, sign_bits, table, flags, y, st);
}

}  // namespace pg
