// gdn_prefill.hip -- chunked prefill (not yet built: the call reports that it
// is not supported until the chunked kernels land).
#include "gdn_launch.hpp"

namespace gdn {

size_t prefill_workspace_bytes(const Geo&, int) { return 0; }

hipError_t launch_prefill(const Geo&, float*, void*, const void*, int, const void*, const float*, const float*,
                          float*, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
