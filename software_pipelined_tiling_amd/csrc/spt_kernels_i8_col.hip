// Kernel instantiations for one element type (i8) and B layout (col-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(i8_col, DT_I8, 1)
}  // namespace spt
