// Multi-row (speculative verify) split kernel: placeholder until the MFMA
// kernel lands; every multi-row shape is reported unsupported.
#include "pkv_common.h"

namespace pkv {

bool verify_supported(int, int, int) { return false; }

hipError_t launch_verify_split(const DecodeArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pkv
