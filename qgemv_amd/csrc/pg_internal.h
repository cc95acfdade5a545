// Internal declarations shared by the host C++ and the HIP launchers of
// libpingala.  Not part of the public C ABI (include/pingala.h).
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/pingala.h"

namespace pg {

// error plumbing (pg_host.cpp)
int fail(int code, const char* fmt, ...);
void clear_error();
const char* last_error();

// bytes of one PG_Q16 activation row (digits, block scales, half-block sums,
// padded to 64 B)
inline size_t q16_row_bytes(int64_t k) {
    const size_t raw = (size_t)(2 * k + k / 32 + k / 16);
    return (raw + 63) & ~(size_t)63;
}

// format helpers (pg_host.cpp)
void group_levels(int s, int c, int out[4]);
void build_codebook(int8_t* out /* [8][256][4] */);
void build_codebook_r23(int8_t* out /* [8][256][4] */);
uint16_t double_to_half_rne(double v);
double half_to_double(uint16_t h);
int encode_ref(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
               uint16_t* scales, int n_threads);
// the encoder through a codebook table (pg_host.cpp), P8F v1's or the rate-2/3 trellis
int encode_ref_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                     bool r23, uint8_t* codes, uint16_t* scales, int n_threads);
// LDLQ (pg_host.cpp): the feedback matrix U - I of the rotated Hessian
// (k x k fp64, host), and the reference encoder that uses it
int ldlq_feedback(const double* hessian, int64_t k, const uint8_t* sign_bits, int n_threads, double* fb);
int encode_ref_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* fb,
                    uint8_t* codes, uint16_t* scales, int n_threads);

// HIP launchers (pg_kernels.hip, pg_fused.hip, pg_qgemm.hip); arguments are
// already validated.
// Each returns PG_OK or PG_ERR_HIP (message set).
int launch_decode(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, float* w,
                  bool carry, pg_stream_t s);
int launch_decode_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const int8_t* table,
                        bool carry, bool rate23, float* w, pg_stream_t s);
int launch_fwht(const void* x, int in_dt, int64_t ldx, void* y, int out_dt, const uint8_t* sign_bits,
                int64_t rows, int64_t k, uint32_t flags, pg_stream_t s);
int launch_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                 const void* x, int x_dt, int batch, uint32_t kflags, float* y, pg_stream_t s);
int launch_rot_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                     int x_dt, int64_t ldx, const uint8_t* sign_bits, uint32_t flags, int batch, float* y,
                     pg_stream_t s);
int launch_rot_qgemv_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                           int x_dt, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                           pg_stream_t s);
// (pg_qgemv_mma.hip) batched product on PG_Q16 activations, matrix cores
int launch_qgemv_mma(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const uint8_t* xq,
                     int batch, float* y, pg_stream_t s);
// (pg_qgemm.hip) the prompt product; with a workspace it may split K:
// the first t_full output tiles whole, the others `splits` ways
// (qgemm_plan picks the plan, qgemm_workspace_bytes the bytes that allow the
// plan it picks with no workspace limit)
struct QgPlan {
    int64_t t_full;
    int splits;
};
int launch_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                 const uint16_t* x, int64_t m, float* y, void* workspace, size_t ws_bytes, pg_stream_t s,
                 int kernel = 0, int splits = 0, int64_t first_split = 0);
QgPlan qgemm_plan(int64_t n, int64_t k, int64_t m, size_t ws_bytes);
QgPlan qgemm_forced(int64_t n, int64_t k, int64_t m, size_t ws_bytes, int splits, int64_t t_full);
// the library's own split-K workspace on the current device (pg_qgemm_noalloc)
constexpr size_t QGEMM_SCRATCH_BYTES = (size_t)32 << 20;
int qgemm_scratch(void** out);
size_t qgemm_workspace_bytes(int64_t n, int64_t k, int64_t m);
// (pg_kernels.hip) streaming read of `bytes` (a multiple of 16) at p
int launch_hbm_read(const void* p, int64_t bytes, uint32_t* out, pg_stream_t s);
// (pg_encode.hip)
int launch_encode(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
                  uint16_t* scales, pg_stream_t s);
int launch_encode_carry(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
                        uint16_t* scales, pg_stream_t s);
// LDLQ on the GPU: fb device fp64 [k][k] (ldlq_feedback's output), err device
// fp64 [n][k] scratch; one launch per block in order
int launch_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* fb,
                       double* err, uint8_t* codes, uint16_t* scales, pg_stream_t s);
int launch_encode_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                        bool r23, uint8_t* codes, uint16_t* scales, pg_stream_t s);
// pg_encode_ldlq's device side: factor on the host, allocate, launch, free
int run_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                    uint8_t* codes, uint16_t* scales, pg_stream_t s);

}  // namespace pg
