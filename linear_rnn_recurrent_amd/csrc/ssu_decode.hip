// Decode entry: dispatch on the state dtype to the per-dtype kernel files.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream)
{
    if (p.batch == 0)
        return hipSuccess;
    switch (p.state_dtype) {
    case kF32: return launch_decode_f32(p, stream);
    case kF16: return launch_decode_f16(p, stream);
    case kBF16: return launch_decode_bf16(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
