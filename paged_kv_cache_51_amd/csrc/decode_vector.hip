// decode_vector.hip — vector-ALU variant of the partition kernel (same math
// and layout as decode.hip, no matrix cores); kept for the MFMA comparison.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

hipError_t launch_decode_vector(const DecodeArgs&, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace pkv
