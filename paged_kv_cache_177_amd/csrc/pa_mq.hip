// Multi-query paged attention (n_q > 1) on the matrix cores -- not built yet.
#include "pa_internal.h"

namespace pa {

hipError_t launch_decode_mq(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
