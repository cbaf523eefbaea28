// The Q4_0 instantiations of the block-format kernels and launchers
// (qmv_blocks_impl.h), compiled on their own and exported as a FormatOps
// table.
#include "qmv_blocks_impl.h"

namespace qmv {
const FormatOps& ops_q4_0() { return format_ops_for<Q4_0>(); }
}  // namespace qmv
