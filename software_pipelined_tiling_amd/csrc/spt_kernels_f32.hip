// Kernel instantiations for one element type (f32).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f32, DT_F32)
}  // namespace spt
