// Tree-verify kernels for _Float16 state (template in ssu_tree_impl.h).
#include "ssu_tree_impl.h"

namespace ssu {

hipError_t launch_tree_f16(const TreeParams &p, hipStream_t stream)
{
    return launch_tree_state<_Float16>(p, stream);
}

}  // namespace ssu
