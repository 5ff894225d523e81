// Prefill kernels for bf16_t state (template in ssu_prefill_impl.h).
#include "ssu_prefill_impl.h"

namespace ssu {

hipError_t launch_prefill_bf16(const PrefillParams &p, hipStream_t stream)
{
    return launch_prefill_state<bf16_t>(p, stream);
}

}  // namespace ssu
