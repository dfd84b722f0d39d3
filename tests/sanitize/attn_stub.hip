// Host-sanitizer build of the C ABI (tests/test_sanitized_host.py): the two
// launchers of the attention kernel's translation unit, replaced by stubs so
// that the build skips the slow kernel compile.  The sanitized library never
// reaches a launch (it runs on a host without a GPU).
#include "kernels.hpp"

namespace lamp {

hipError_t launch_attention(const Shape&, const AttnParams&, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_debug_fp8_dot(const uint8_t*, const uint8_t*, float*, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace lamp
