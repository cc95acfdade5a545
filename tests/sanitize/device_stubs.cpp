// Stand-ins for the device side of libpingala in the host-only sanitizer
// build: every launcher refuses (nothing runs on a GPU here), so the C ABI's
// argument validation and the host encoder can be run under AddressSanitizer
// and UndefinedBehaviorSanitizer on the CPU.
#include "../../qgemv_amd/csrc/pg_internal.h"

namespace pg {
namespace {
int no_device(const char* what) { return fail(PG_ERR_UNSUPPORTED, "%s: no device in the host-only build", what); }
}  // namespace

int launch_decode(const uint8_t*, const uint16_t*, int64_t, int64_t, float*, bool, pg_stream_t) {
    return no_device("pg_decode");
}
int launch_decode_table(const uint8_t*, const uint16_t*, int64_t, int64_t, const int8_t*, bool, bool, float*,
                        pg_stream_t) {
    return no_device("pg_decode_table");
}
int launch_rot_qgemv_table(const uint8_t*, const uint16_t*, int64_t, int64_t, const void*, int, const uint8_t*,
                           const int8_t*, uint32_t, float*, pg_stream_t) {
    return no_device("pg_rot_qgemv_table");
}
int launch_fwht(const void*, int, int64_t, void*, int, const uint8_t*, int64_t, int64_t, uint32_t, pg_stream_t) {
    return no_device("pg_fwht_rotate");
}
int launch_qgemv(const uint8_t*, const uint16_t*, int64_t, int64_t, const void*, int, int, uint32_t, float*,
                 pg_stream_t) {
    return no_device("pg_qgemv");
}
int launch_rot_qgemv(const uint8_t*, const uint16_t*, int64_t, int64_t, const void*, int, int64_t, const uint8_t*,
                     uint32_t, int, float*, pg_stream_t) {
    return no_device("pg_rot_qgemv");
}
int launch_qgemm(const uint8_t*, const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, float*, void*, size_t,
                 pg_stream_t, int, int, int64_t) {
    return no_device("pg_qgemm");
}
int qgemm_scratch(void**) { return no_device("pg_qgemm_noalloc"); }
size_t qgemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
int launch_hbm_read(const void*, int64_t, uint32_t*, pg_stream_t) { return no_device("pg_hbm_read"); }
int launch_encode(const float*, int64_t, int64_t, const uint8_t*, uint8_t*, uint16_t*, pg_stream_t) {
    return no_device("pg_encode");
}
int launch_encode_carry(const float*, int64_t, int64_t, const uint8_t*, uint8_t*, uint16_t*, pg_stream_t) {
    return no_device("pg_encode_ex");
}
int run_encode_ldlq(const float*, int64_t, int64_t, const uint8_t*, const double*, uint8_t*, uint16_t*, pg_stream_t) {
    return no_device("pg_encode_ldlq");
}
int launch_encode_table(const float*, int64_t, int64_t, const uint8_t*, const int8_t*, bool, uint8_t*, uint16_t*,
                        pg_stream_t) {
    return no_device("pg_encode_table");
}
}  // namespace pg
