// decode_mfma.hip -- paged decode attention on the matrix cores (gfx950).
#include "pa_device.h"

namespace pa {

bool mfma_supported(int, int, int, int, int) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs &, int, int, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace pa
