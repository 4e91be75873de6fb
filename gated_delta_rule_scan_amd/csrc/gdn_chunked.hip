// Chunked matrix-core replay kernel (bf16 inputs, float32 state).
#include "gdn_launch.h"

namespace gdn {

bool chunked_supported(int, int, Elem) { return false; }

hipError_t launch_chunked(const LaunchDesc &, int, int, Elem, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
