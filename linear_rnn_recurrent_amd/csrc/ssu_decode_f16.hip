// Decode kernels for _Float16 state (template in ssu_decode_impl.h).
#include "ssu_decode_impl.h"

namespace ssu {

hipError_t launch_decode_f16(const DecodeParams &p, hipStream_t stream)
{
    return launch_decode_state<_Float16>(p, stream);
}

}  // namespace ssu
