// pa_decode_mfma.hip -- matrix-core decode kernel for grouped-query attention.
#include "pa_internal.h"

namespace pa {

bool mfma_path_supported(int, int, int) { return false; }

hipError_t launch_decode_mfma(int, int, const DecodeParams &, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace pa
