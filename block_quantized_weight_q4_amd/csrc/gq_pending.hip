// Placeholder for the prefill product until its kernel lands: reports
// "not supported" through the ABI.
#include "gq_internal.h"

hipError_t gqk_matmul(int, const void*, int64_t, int64_t, const void*, int, int64_t, int64_t, float*, int64_t,
                      hipStream_t) {
    return hipErrorNotSupported;
}
