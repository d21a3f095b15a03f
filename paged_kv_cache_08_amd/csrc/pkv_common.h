// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Split planner constants (the plan itself is documented in include/pkv.h).
constexpr int kTile = 64;        // split boundaries are multiples of this many tokens
constexpr int kWgPerCu = 1;      // planner target: this many split workgroups per CU
constexpr int kMinTiles = 1;     // a split covers at least this many tiles when planned
constexpr int kMaxTiles = 8;     // a split covers at most this many tiles (one kernel window)
constexpr int kMaxChunk = kMaxTiles * kTile;

constexpr int kWsHeaderBytes = 256;   // workspace: error word, then partials

// Division of a non-negative 32-bit n by an invariant divisor d >= 1 with one
// multiply-high, after Granlund & Montgomery, "Division by Invariant Integers
// using Multiplication" (PLDI 1994), unsigned case: with l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, sh1 = min(l, 1), sh2 = max(l - 1, 0),
// q = (t1 + ((n - t1) >> sh1)) >> sh2 where t1 = mulhi(m, n).
struct MagicDiv {
  uint32_t m;
  uint32_t sh1;
  uint32_t sh2;
  uint32_t d;
};

inline MagicDiv make_magic(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  MagicDiv r;
  r.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  r.sh1 = l < 1 ? l : 1;
  r.sh2 = l > 0 ? l - 1 : 0;
  r.d = d;
  return r;
}

__host__ __device__ inline uint32_t magic_div(uint32_t n, const MagicDiv& md) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t t1 = __umulhi(md.m, n);
#else
  uint32_t t1 = uint32_t((uint64_t(md.m) * n) >> 32);
#endif
  return (t1 + ((n - t1) >> md.sh1)) >> md.sh2;
}

// Everything a split / merge kernel needs, passed by value.
struct DecodeArgs {
  const uint16_t* q;        // bf16 [num_seqs, q_len, hq, D]
  const uint16_t* k;        // paged K: bf16, or FP8 codes addressed bytewise (kv_fp8)
  const uint16_t* v;        // paged V, the same
  const int32_t* table;     // [num_seqs, max_pages]
  const int32_t* seq_lens;  // [num_seqs]
  void* out;                // [num_seqs, q_len, hq, D] f32 or bf16
  float* part_ml;           // [(b*q_len+i)*hq+h][S][2]  (reference max in log2 units, sum)
  float* part_acc;          // [(b*q_len+i)*hq+h][S][D]  un-normalised weighted V
  uint32_t* err;            // workspace error word
  int64_t k_sp, k_st, k_sh;
  int64_t v_sp, v_st, v_sh;
  int32_t num_seqs, q_len, hq, hkv, max_pages, num_pages;
  int32_t chunk;            // tokens per split
  int32_t num_splits;       // S (grid x)
  MagicDiv bdiv;            // division by block_size
  float scale_log2;         // scale * log2(e): scores kept in log2 units
  int32_t out_bf16;
  // Varlen multi-row calls: cu_q[b] .. cu_q[b + 1] are sequence b's rows of the
  // packed q / out ([total_q, Hq, D]); q_len is then the largest row count.
  // nullptr for uniform calls (sequence b owns rows b * q_len .. + q_len).
  const int32_t* cu_q;
  int32_t window;           // sliding window in positions (0 = whole context)
  int32_t kv_fp8;           // K/V caches hold FP8 E4M3 codes (else bf16)
  float out_scale;          // applied to every stored output (the FP8 V scale, else 1)
  int32_t pf_rows;          // prefill calls: query positions per workgroup block (else 0)
  float* lse;               // optional [rows, hq] natural-log log-sum-exp of each row's scores (nullptr: none)
  int32_t many_wg;          // the split grid holds more workgroups than the device has CUs
};

// Launchers (decode_kernels.hip, decode_w*.hip, decode_mfma_fp8.hip,
// verify_kernels.hip). Return
// hipError_t. The split launchers take optional start/stop events, stamped at
// the start and end of the kernel's execution (hipExtLaunchKernel) when both
// are non-null. launch_decode_split picks the smallest window (64, 128, 256 or
// 512 tokens, decode_window()) that holds a split of a.chunk tokens.
int decode_window(int chunk);
hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                               hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode_split_w512_many(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                         hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode_split_w64(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                   hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode_split_w128(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                    hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode_split_w256(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                    hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode_split_w512(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                    hipEvent_t ev_start, hipEvent_t ev_stop);
// The single-query split kernel on MFMA for FP8 caches (decode_mfma_fp8.hip).
hipError_t launch_decode_mfma_fp8(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                  hipEvent_t ev_start, hipEvent_t ev_stop);
// Several query rows, at most 32 per KV head, on the single-query MFMA
// kernel's structure (decode_mfma_rows.hip).
hipError_t launch_decode_mfma_rows(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                   hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_verify_split(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                               hipEvent_t ev_start, hipEvent_t ev_stop);
// Prefill: blocks of a.pf_rows query positions per workgroup, each over its
// whole visible range in one pass (no split, no merge; output written directly).
hipError_t launch_prefill(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                          hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_lse_merge(const DecodeArgs& a, int head_dim, hipStream_t st);
hipError_t launch_debug_offsets(const DecodeArgs& a, int kv_head, int max_seq_len,
                                int64_t* k_off, int64_t* v_off, hipStream_t st);
hipError_t launch_debug_ranges(const DecodeArgs& a, int32_t* ranges, hipStream_t st);
hipError_t launch_debug_token_splits(const DecodeArgs& a, int max_seq_len, int32_t* slots, hipStream_t st);
bool decode_supported(int head_dim, int group);
bool verify_supported(int head_dim, int group, int q_len);
bool rows_mfma_supported(int head_dim, int group, int q_len);

}  // namespace pkv
