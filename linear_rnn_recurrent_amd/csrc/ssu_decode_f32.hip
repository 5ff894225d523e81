// Decode kernels for float state (template in ssu_decode_impl.h).
#include "ssu_decode_impl.h"

namespace ssu {

hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream)
{
    return launch_decode_state<float>(p, stream);
}

}  // namespace ssu
