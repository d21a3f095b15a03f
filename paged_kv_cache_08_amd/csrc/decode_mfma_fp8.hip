// MFMA split kernels for FP8 E4M3 caches, every window (64 .. 512 tokens).
#include "decode_mfma.h"

namespace pkv {

namespace {
constexpr int kW = 4;   // waves per workgroup
constexpr int kR = 2;   // register ring depth: one step in flight
}  // namespace

hipError_t launch_decode_mfma_fp8(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                                  hipEvent_t e1) {
  switch (decode_window(a.chunk)) {
    case 64: return launch_decode_mfma_window<2, true, kW, kR>(a, head_dim, group, st, e0, e1);
    case 128: return launch_decode_mfma_window<4, true, kW, kR>(a, head_dim, group, st, e0, e1);
    case 256: return launch_decode_mfma_window<8, true, kW, kR>(a, head_dim, group, st, e0, e1);
    default: return launch_decode_mfma_window<16, true, kW, kR>(a, head_dim, group, st, e0, e1);
  }
}

}  // namespace pkv
