"""qgemv_amd: Python binding of libpingala (Pingala-8 P8F v1 kernels for
MI355X).  The library is loaded on first use; importing the package does not
touch the GPU."""
from ._lib import (EXPORTS, PG_BF16, PG_F16, PG_F32, PG_FLAG_CARRY_STATE, PG_FLAG_RMSNORM, PG_Q16,  # noqa: F401
                   PgError, lib, pg_codebook_table, pg_q16_row_bytes, pg_decode, pg_decode_ex, pg_encode,
                   pg_encode_ex, pg_encode_ref, pg_footprint_bytes, pg_fwht_rotate,
                   pg_fwht_rotate_ex,
                   pg_last_error, pg_qgemm, pg_qgemm_ex, pg_qgemm_workspace_bytes, pg_qgemv, pg_rot_qgemv, pg_version)
