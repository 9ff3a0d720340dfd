// kda_bwd.hip -- chunked KDA backward for gfx950 (placeholder launcher).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

hipError_t launch_bwd(const BwdParams& p, int in_dtype, int out_dtype, int dk, hipStream_t s) {
    (void)p; (void)in_dtype; (void)out_dtype; (void)dk; (void)s;
    return hipErrorNotSupported;
}

}  // namespace kda
