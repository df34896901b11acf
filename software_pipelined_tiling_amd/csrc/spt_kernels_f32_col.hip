// Kernel instantiations for one element type (f32) and B layout (col-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f32_col, DT_F32, 1)
}  // namespace spt
