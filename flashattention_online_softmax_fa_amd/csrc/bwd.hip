// bwd.hip -- placeholder until the matrix-core backward lands.
#include "fa_internal.h"
namespace fa {
hipError_t launch_bwd_bf16(const BwdArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
