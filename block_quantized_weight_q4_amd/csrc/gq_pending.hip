#include "gq_internal.h"
size_t gqk_matvec_id_ws_bytes(int, int, int, int64_t) { return 256; }
hipError_t gqk_matvec_id(int, const void*, int, int64_t, int64_t, const int32_t*, int, int, const void*, int, int, const float*, float*, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t gqk_matvec_id_bad_count(const void*, hipStream_t, int32_t*) { return hipErrorNotSupported; }
hipError_t gqk_matmul(int, const void*, int64_t, int64_t, const void*, int, int64_t, int64_t, float*, int64_t, hipStream_t) { return hipErrorNotSupported; }
