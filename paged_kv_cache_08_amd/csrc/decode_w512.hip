// Split kernels with a 512-token window (16 strided blocks of 32 tokens), bf16
// caches, for grids of at most one workgroup per CU: the partials are written
// through to memory, since the whole grid ends at once and the merge reads
// them next.
#include "decode_split.h"

namespace pkv {

hipError_t launch_decode_split_w512(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                    hipEvent_t e0, hipEvent_t e1) {
  return launch_decode_window<16, kRingOne, true>(a, head_dim, group, st, e0, e1);
}

}  // namespace pkv
