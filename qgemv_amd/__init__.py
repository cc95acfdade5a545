"""qgemv_amd: Python binding of libpingala (Pingala-8 P8F v1 kernels for
MI355X).  The library is loaded on first use; importing the package does not
touch the GPU."""
from ._lib import (EXPORTS, PG_BF16, PG_F16, PG_F32, PG_FLAG_CARRY_STATE, PG_FLAG_KERNEL_MMA, PG_FLAG_KERNEL_VDOT, PG_FLAG_RATE23, PG_FLAG_RMSNORM, PG_Q16,  # noqa: F401
                   PgError, lib, pg_codebook_table, pg_codebook_table_ex, pg_q16_row_bytes, pg_decode, pg_decode_ex, pg_decode_table, pg_encode,
                   pg_encode_ex, pg_encode_ldlq, pg_encode_ref, pg_encode_ref_ldlq, pg_encode_ref_table, pg_encode_table, pg_footprint_bytes, pg_fwht_rotate,
                   pg_fwht_rotate_ex, pg_hbm_read,
                   pg_last_error, pg_qgemm, pg_qgemm_ex, pg_qgemm_noalloc, pg_qgemm_tune, pg_qgemm_workspace_bytes, pg_qgemv, pg_qgemv_ex, pg_rot_qgemv, pg_rot_qgemv_table, pg_version)
