// Decode kernels for bf16_t state (template in ssu_decode_impl.h).
#include "ssu_decode_impl.h"

namespace ssu {

hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t stream)
{
    return launch_decode_state<bf16_t>(p, stream);
}

}  // namespace ssu
