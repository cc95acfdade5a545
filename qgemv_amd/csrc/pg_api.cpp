// The C ABI of libpingala (declared in include/pingala.h): argument
// validation on the host, then dispatch to the HIP launchers.  No call
// launches anything when an argument is invalid.
#include <cstdint>

#include <vector>

#include "pg_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_nk(int64_t n, int64_t k) {
    if (n < 1) return pg::fail(PG_ERR_INVALID_ARG, "n must be >= 1 (got %lld)", (long long)n);
    if (k < 128 || k % 128 != 0)
        return pg::fail(PG_ERR_INVALID_ARG, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    // device kernels index rows and columns with 32-bit offsets per row
    if (k > (int64_t)1 << 24 || n > (int64_t)1 << 30)
        return pg::fail(PG_ERR_UNSUPPORTED, "n or k too large (n=%lld k=%lld)", (long long)n, (long long)k);
    return PG_OK;
}

int check_ptr(const void* p, uintptr_t align, const char* name) {
    if (!p) return pg::fail(PG_ERR_INVALID_ARG, "%s is null", name);
    if (!aligned(p, align)) return pg::fail(PG_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, (unsigned)align);
    return PG_OK;
}

int check_dtype(int dt, const char* name, bool allow_bf16, bool allow_q16) {
    if (dt == PG_F32 || dt == PG_F16 || (allow_bf16 && dt == PG_BF16) || (allow_q16 && dt == PG_Q16)) return PG_OK;
    return pg::fail(PG_ERR_INVALID_ARG, "%s: unsupported dtype %d", name, dt);
}

}  // namespace

#define PG_TRY(expr)                 \
    do {                             \
        int _rc = (expr);            \
        if (_rc != PG_OK) return _rc; \
    } while (0)

extern "C" {

int pg_version(void) { return (PG_FORMAT_VERSION << 16) | PG_LIB_VERSION; }

size_t pg_q16_row_bytes(int64_t k) {
    if (k < 128 || k % 128 != 0) return 0;
    return pg::q16_row_bytes(k);
}

size_t pg_footprint_bytes(int64_t n, int64_t k) {
    if (n < 1 || k < 128 || k % 128 != 0) return 0;
    return (size_t)(n * (k / 4) + n * (k / 128) * 2);
}

const char* pg_last_error(void) { return pg::last_error(); }

int pg_codebook_table(int8_t* out) {
    pg::clear_error();
    PG_TRY(check_ptr(out, 1, "out"));
    pg::build_codebook(out);
    return PG_OK;
}

int pg_codebook_table_ex(uint32_t flags, int8_t* out) {
    pg::clear_error();
    if (flags & ~PG_FLAG_RATE23) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_ptr(out, 1, "out"));
    if (flags & PG_FLAG_RATE23) pg::build_codebook_r23(out);
    else pg::build_codebook(out);
    return PG_OK;
}

int pg_encode_ref(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
                  uint16_t* scales, int n_threads) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(codes, 1, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::encode_ref(w, n, k, sign_bits, codes, scales, n_threads);
}

int pg_encode(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes, uint16_t* scales,
              pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::launch_encode(w, n, k, sign_bits, codes, scales, stream);
}

int pg_encode_ref_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                       uint8_t* codes, uint16_t* scales, int n_threads) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (k > 16384) return pg::fail(PG_ERR_UNSUPPORTED, "pg_encode_ref_ldlq: k <= 16384 (the feedback matrix is k^2 fp64)");
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(hessian, 8, "hessian"));
    PG_TRY(check_ptr(codes, 1, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    std::vector<double> fb((size_t)(k * k));
    PG_TRY(pg::ldlq_feedback(hessian, k, sign_bits, n_threads, fb.data()));
    return pg::encode_ref_ldlq(w, n, k, sign_bits, fb.data(), codes, scales, n_threads);
}

int pg_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                   uint8_t* codes, uint16_t* scales, pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (k > 16384) return pg::fail(PG_ERR_UNSUPPORTED, "pg_encode_ldlq: k <= 16384 (the feedback matrix is k^2 fp64)");
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(hessian, 8, "hessian"));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::run_encode_ldlq(w, n, k, sign_bits, hessian, codes, scales, stream);
}

int pg_encode_ref_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                        uint32_t flags, uint8_t* codes, uint16_t* scales, int n_threads) {
    pg::clear_error();
    if (flags & ~PG_FLAG_RATE23) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(table, 1, "table"));
    PG_TRY(check_ptr(codes, 1, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::encode_ref_table(w, n, k, sign_bits, table, (flags & PG_FLAG_RATE23) != 0, codes, scales, n_threads);
}

int pg_encode_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                    uint32_t flags, uint8_t* codes, uint16_t* scales, pg_stream_t stream) {
    pg::clear_error();
    if (flags & ~PG_FLAG_RATE23) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(table, 16, "table"));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::launch_encode_table(w, n, k, sign_bits, table, (flags & PG_FLAG_RATE23) != 0, codes, scales, stream);
}

int pg_encode_ex(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint32_t flags, uint8_t* codes,
                 uint16_t* scales, pg_stream_t stream) {
    pg::clear_error();
    if (flags & ~PG_FLAG_CARRY_STATE) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    if (!(flags & PG_FLAG_CARRY_STATE)) return pg_encode(w, n, k, sign_bits, codes, scales, stream);
    PG_TRY(check_nk(n, k));
    if (k > 16384) return pg::fail(PG_ERR_UNSUPPORTED, "pg_encode_ex: carried state needs k <= 16384");
    PG_TRY(check_ptr(w, 4, "w"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    return pg::launch_encode_carry(w, n, k, sign_bits, codes, scales, stream);
}

int pg_decode_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, uint32_t flags, float* w_rot,
                 pg_stream_t stream) {
    pg::clear_error();
    if (flags & ~PG_FLAG_CARRY_STATE) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(w_rot, 16, "w_rot"));
    return pg::launch_decode(codes, scales, n, k, w_rot, (flags & PG_FLAG_CARRY_STATE) != 0, stream);
}

int pg_decode_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const int8_t* table,
                    uint32_t flags, float* w_rot, pg_stream_t stream) {
    pg::clear_error();
    if (flags & ~(uint32_t)(PG_FLAG_CARRY_STATE | PG_FLAG_RATE23))
        return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(table, 16, "table"));
    PG_TRY(check_ptr(w_rot, 16, "w_rot"));
    return pg::launch_decode_table(codes, scales, n, k, table, (flags & PG_FLAG_CARRY_STATE) != 0,
                                   (flags & PG_FLAG_RATE23) != 0, w_rot, stream);
}

int pg_decode(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, float* w_rot,
              pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(w_rot, 16, "w_rot"));
    return pg::launch_decode(codes, scales, n, k, w_rot, false, stream);
}

int pg_fwht_rotate_ex(const void* x, int in_dtype, int64_t ldx, void* y, int out_dtype, const uint8_t* sign_bits,
                      int64_t rows, int64_t k, uint32_t flags, pg_stream_t stream) {
    pg::clear_error();
    if (rows < 1) return pg::fail(PG_ERR_INVALID_ARG, "rows must be >= 1 (got %lld)", (long long)rows);
    PG_TRY(check_nk(rows, k));
    if (ldx < k) return pg::fail(PG_ERR_INVALID_ARG, "ldx (%lld) < k (%lld)", (long long)ldx, (long long)k);
    PG_TRY(check_dtype(in_dtype, "in_dtype", true, false));
    PG_TRY(check_dtype(out_dtype, "out_dtype", true, true));
    PG_TRY(check_ptr(x, 16, "x"));
    PG_TRY(check_ptr(y, 16, "y"));
    PG_TRY(check_ptr(sign_bits, 1, "sign_bits"));
    if (flags & ~PG_FLAG_RMSNORM) return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    const size_t in_b = ((size_t)(rows - 1) * ldx + k) * (in_dtype == PG_F32 ? 4 : 2);
    const size_t out_b = out_dtype == PG_Q16 ? (size_t)rows * pg::q16_row_bytes(k)
                                             : (size_t)rows * k * (out_dtype == PG_F32 ? 4 : 2);
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    if (xa < ya + out_b && ya < xa + in_b) return pg::fail(PG_ERR_INVALID_ARG, "x and y overlap");
    return pg::launch_fwht(x, in_dtype, ldx, y, out_dtype, sign_bits, rows, k, flags, stream);
}

int pg_fwht_rotate(const void* x, int in_dtype, void* y, int out_dtype, const uint8_t* sign_bits,
                   int64_t rows, int64_t k, uint32_t flags, pg_stream_t stream) {
    return pg_fwht_rotate_ex(x, in_dtype, k, y, out_dtype, sign_bits, rows, k, flags, stream);
}

int pg_qgemv_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x_rot,
                int x_dtype, int batch, uint32_t flags, float* y, pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (batch < 1 || batch > 8) return pg::fail(PG_ERR_INVALID_ARG, "batch must be 1..8 (got %d)", batch);
    PG_TRY(check_dtype(x_dtype, "x_dtype", false, true));
    if (flags & ~(uint32_t)(PG_FLAG_KERNEL_VDOT | PG_FLAG_KERNEL_MMA))
        return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    if ((flags & PG_FLAG_KERNEL_VDOT) && (flags & PG_FLAG_KERNEL_MMA))
        return pg::fail(PG_ERR_INVALID_ARG, "PG_FLAG_KERNEL_VDOT and PG_FLAG_KERNEL_MMA exclude each other");
    if (flags && x_dtype != PG_Q16) return pg::fail(PG_ERR_INVALID_ARG, "kernel choice needs PG_Q16 input");
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(x_rot, 16, "x_rot"));
    PG_TRY(check_ptr(y, 16, "y"));
    return pg::launch_qgemv(codes, scales, n, k, x_rot, x_dtype, batch, flags, y, stream);
}

int pg_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x_rot,
             int x_dtype, int batch, float* y, pg_stream_t stream) {
    return pg_qgemv_ex(codes, scales, n, k, x_rot, x_dtype, batch, 0, y, stream);
}

int pg_rot_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x, int x_dtype,
                 int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y, pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (batch < 1 || batch > 8) return pg::fail(PG_ERR_INVALID_ARG, "batch must be 1..8 (got %d)", batch);
    PG_TRY(check_dtype(x_dtype, "x_dtype", false, false));
    if (ldx < k) return pg::fail(PG_ERR_INVALID_ARG, "ldx (%lld) < k (%lld)", (long long)ldx, (long long)k);
    if (ldx > 0x7fffffffLL)   // the stage kernels take it in 32 bits (all of their arguments are preloaded)
        return pg::fail(PG_ERR_UNSUPPORTED, "ldx (%lld) above 2^31 - 1", (long long)ldx);
    if (flags & ~(uint32_t)(PG_FLAG_RMSNORM | PG_FLAG_CARRY_STATE | PG_FLAG_KERNEL_VDOT | PG_FLAG_KERNEL_MMA))
        return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    if ((flags & PG_FLAG_KERNEL_VDOT) && (flags & PG_FLAG_KERNEL_MMA))
        return pg::fail(PG_ERR_INVALID_ARG, "PG_FLAG_KERNEL_VDOT and PG_FLAG_KERNEL_MMA exclude each other");
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 4, "scales"));
    PG_TRY(check_ptr(x, 16, "x"));
    if ((ldx * (x_dtype == PG_F32 ? 4 : 2)) % 16 != 0)
        return pg::fail(PG_ERR_INVALID_ARG, "rows of x (ldx = %lld) are not 16-byte multiples", (long long)ldx);
    PG_TRY(check_ptr(sign_bits, 4, "sign_bits"));
    PG_TRY(check_ptr(y, 4, "y"));
    const uintptr_t ya = (uintptr_t)y, xa = (uintptr_t)x;
    const size_t yb = (size_t)batch * n * 4, xb = (size_t)batch * ldx * (x_dtype == PG_F32 ? 4 : 2);
    if (xa < ya + yb && ya < xa + xb) return pg::fail(PG_ERR_INVALID_ARG, "x and y overlap");
    return pg::launch_rot_qgemv(codes, scales, n, k, x, x_dtype, ldx, sign_bits, flags, batch, y, stream);
}

int pg_rot_qgemv_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                       int x_dtype, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                       pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    PG_TRY(check_dtype(x_dtype, "x_dtype", false, false));
    if (flags & ~(uint32_t)(PG_FLAG_RMSNORM | PG_FLAG_CARRY_STATE | PG_FLAG_RATE23))
        return pg::fail(PG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 4, "scales"));
    PG_TRY(check_ptr(x, 16, "x"));
    PG_TRY(check_ptr(sign_bits, 4, "sign_bits"));
    PG_TRY(check_ptr(table, 16, "table"));
    PG_TRY(check_ptr(y, 4, "y"));
    const uintptr_t ya = (uintptr_t)y, xa = (uintptr_t)x;
    const size_t yb = (size_t)n * 4, xb = (size_t)k * (x_dtype == PG_F32 ? 4 : 2);
    if (xa < ya + yb && ya < xa + xb) return pg::fail(PG_ERR_INVALID_ARG, "x and y overlap");
    return pg::launch_rot_qgemv_table(codes, scales, n, k, x, x_dtype, sign_bits, table, flags, y, stream);
}

int pg_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x_rot_bf16,
             int64_t m, float* y, pg_stream_t stream) {
    return pg_qgemm_ex(codes, scales, n, k, x_rot_bf16, m, y, nullptr, 0, stream);
}

size_t pg_qgemm_workspace_bytes(int64_t n, int64_t k, int64_t m) {
    if (n < 1 || k < 128 || k % 128 != 0 || k > (int64_t)1 << 24 || n > (int64_t)1 << 30 || m < 1 ||
        m > ((int64_t)1 << 30))
        return 0;
    return pg::qgemm_workspace_bytes(n, k, m);
}

int pg_qgemm_tune(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x_rot_bf16,
                  int64_t m, float* y, void* workspace, size_t workspace_bytes, int kernel, int splits,
                  int64_t first_split, pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (m < 1 || m > ((int64_t)1 << 30)) return pg::fail(PG_ERR_INVALID_ARG, "m must be >= 1 (got %lld)", (long long)m);
    if (kernel < 0 || kernel > 8) return pg::fail(PG_ERR_INVALID_ARG, "kernel must be 0..8 (got %d)", kernel);
    if (splits < 0 || first_split < 0)
        return pg::fail(PG_ERR_INVALID_ARG, "splits and first_split must be >= 0 (got %d, %lld)", splits,
                        (long long)first_split);
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(x_rot_bf16, 16, "x_rot_bf16"));
    PG_TRY(check_ptr(y, 16, "y"));
    if (!workspace && workspace_bytes) return pg::fail(PG_ERR_INVALID_ARG, "workspace is null but workspace_bytes > 0");
    if (workspace) {
        PG_TRY(check_ptr(workspace, 16, "workspace"));
        // the workspace may not overlap any operand
        const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + workspace_bytes;
        const struct { const void* p; size_t bytes; const char* name; } ops[] = {
            {codes, (size_t)n * (size_t)(k / 4), "codes"},
            {scales, (size_t)n * (size_t)(k / 128) * 2, "scales"},
            {x_rot_bf16, (size_t)m * (size_t)k * 2, "x_rot_bf16"},
            {y, (size_t)m * (size_t)n * 4, "y"}};
        for (const auto& o : ops) {
            const uintptr_t a = (uintptr_t)o.p;
            if (w0 < a + o.bytes && a < w1) return pg::fail(PG_ERR_INVALID_ARG, "workspace overlaps %s", o.name);
        }
    }
    return pg::launch_qgemm(codes, scales, n, k, x_rot_bf16, m, y, workspace, workspace_bytes, stream, kernel, splits,
                            first_split);
}

int pg_qgemm_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x_rot_bf16,
                int64_t m, float* y, void* workspace, size_t workspace_bytes, pg_stream_t stream) {
    return pg_qgemm_tune(codes, scales, n, k, x_rot_bf16, m, y, workspace, workspace_bytes, 0, 0, 0, stream);
}

int pg_qgemm_noalloc(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint16_t* x_rot_bf16,
                     int64_t m, float* y, pg_stream_t stream) {
    pg::clear_error();
    PG_TRY(check_nk(n, k));
    if (m < 1 || m > ((int64_t)1 << 30)) return pg::fail(PG_ERR_INVALID_ARG, "m must be >= 1 (got %lld)", (long long)m);
    PG_TRY(check_ptr(codes, 16, "codes"));
    PG_TRY(check_ptr(scales, 2, "scales"));
    PG_TRY(check_ptr(x_rot_bf16, 16, "x_rot_bf16"));
    PG_TRY(check_ptr(y, 16, "y"));
    const size_t need = pg::qgemm_workspace_bytes(n, k, m);
    if (need > pg::QGEMM_SCRATCH_BYTES)
        return pg::fail(PG_ERR_UNSUPPORTED,
                        "pg_qgemm_noalloc: n=%lld k=%lld m=%lld needs %zu bytes of split workspace, the library's "
                        "scratch holds %zu; use pg_qgemm_ex with a caller workspace",
                        (long long)n, (long long)k, (long long)m, need, pg::QGEMM_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) PG_TRY(pg::qgemm_scratch(&ws));
    return pg::launch_qgemm(codes, scales, n, k, x_rot_bf16, m, y, ws, need, stream);
}

int pg_hbm_read(const void* p, size_t bytes, uint32_t* xor_out, pg_stream_t stream) {
    pg::clear_error();
    if (bytes == 0 || bytes % 16 != 0)
        return pg::fail(PG_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 (got %zu)", bytes);
    PG_TRY(check_ptr(p, 16, "p"));
    PG_TRY(check_ptr(xor_out, 4, "xor_out"));
    const uintptr_t a = (uintptr_t)p, o = (uintptr_t)xor_out;
    if (o < a + bytes && a < o + 4) return pg::fail(PG_ERR_INVALID_ARG, "xor_out overlaps p");
    return pg::launch_hbm_read(p, (int64_t)bytes, xor_out, stream);
}

}  // extern "C"
