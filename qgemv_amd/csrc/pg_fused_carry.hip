// Fused-stage instances for codes of the carried-state variant (trellis
// state running on from block to block along a row; "Pingala-8" landing
// page, section "Paper", small-state coset trellises), in a translation unit
// of their own so they compile beside the P8F v1 ones.
#include "pg_fused.h"

namespace pg {

int launch_fused_carry(const FusedShape& S, const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const void* x, int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch,
                       float* y, hipStream_t st) {
    return launch_fused_all<true>(S, codes, scales, n, k, x, x_dt, ldx, sign_bits, flags, batch, y, st);
}

}  // namespace pg
