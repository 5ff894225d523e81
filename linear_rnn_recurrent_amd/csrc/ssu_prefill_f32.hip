// Prefill kernels for float state (template in ssu_prefill_impl.h).
#include "ssu_prefill_impl.h"

namespace ssu {

hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream)
{
    return launch_prefill_state<float>(p, stream);
}

}  // namespace ssu
