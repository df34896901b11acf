// Kernel instantiations for one element type (f16).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f16, DT_F16)
}  // namespace spt
