// Kernel instantiations for one element type (f32) and B layout (row-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f32_row, DT_F32, 0)
}  // namespace spt
