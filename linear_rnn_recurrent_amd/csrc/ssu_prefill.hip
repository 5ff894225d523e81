// Prefill entry: dispatch on the state dtype to the per-dtype kernel files.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream)
{
    if (p.d.batch == 0 || p.seq_len == 0)
        return hipSuccess;
    switch (p.d.state_dtype) {
    case kF32: return launch_prefill_f32(p, stream);
    case kF16: return launch_prefill_f16(p, stream);
    case kBF16: return launch_prefill_bf16(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
