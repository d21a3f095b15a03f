// MFMA split kernels for calls with several query rows per sequence (uniform
// q_len or varlen rows) and at most 32 rows per KV head: the single-query
// MFMA kernel with two 16-row tiles and per-row causal bounds, bf16 and FP8
// caches, head_dim 256.
#include "decode_mfma.h"

namespace pkv {

namespace {
constexpr int kW = 4;   // waves per workgroup
constexpr int kR = 2;   // register ring depth: one step in flight

template <int NBLK>
hipError_t rows_window(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return a.kv_fp8 ? launch_decode_mfma_window<NBLK, true, kW, kR, true>(a, head_dim, group, st, e0, e1)
                  : launch_decode_mfma_window<NBLK, false, kW, kR, true>(a, head_dim, group, st, e0, e1);
}
}  // namespace

bool rows_mfma_supported(int head_dim, int group, int q_len) {
  return head_dim == 256 && group >= 1 && q_len >= 1 && int64_t(group) * q_len <= 32;
}

hipError_t launch_decode_mfma_rows(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                                   hipEvent_t e1) {
  if (!rows_mfma_supported(head_dim, group, a.q_len)) return hipErrorInvalidValue;
  switch (decode_window(a.chunk)) {
    case 64: return rows_window<2>(a, head_dim, group, st, e0, e1);
    case 128: return rows_window<4>(a, head_dim, group, st, e0, e1);
    case 256: return rows_window<8>(a, head_dim, group, st, e0, e1);
    default: return rows_window<16>(a, head_dim, group, st, e0, e1);
  }
}

}  // namespace pkv
