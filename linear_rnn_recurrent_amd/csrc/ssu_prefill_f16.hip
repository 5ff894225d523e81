// Prefill kernels for _Float16 state (template in ssu_prefill_impl.h).
#include "ssu_prefill_impl.h"

namespace ssu {

hipError_t launch_prefill_f16(const PrefillParams &p, hipStream_t stream)
{
    return launch_prefill_state<_Float16>(p, stream);
}

}  // namespace ssu
