// Kernel instantiations for one element type (i8) and B layout (row-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(i8_row, DT_I8, 0)
}  // namespace spt
