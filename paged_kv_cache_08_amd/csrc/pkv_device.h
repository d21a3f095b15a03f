// Device-side helpers shared by the gfx950 kernels: bf16 arithmetic, DPP
// moves, the split range of a workgroup, block-table staging in LDS and the
// element offset of a token row.
#pragma once

#include <math.h>

#include <type_traits>

#include "pkv_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
// The same move for controls where every lane has a source lane (broadcasts
// within a row): no old value, so no register is zeroed first.
template <int CTRL>
__device__ __forceinline__ float dpp_move_full(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950 lane swaps. swap32(a, b) returns {[a_lo, b_lo], [a_hi, b_hi]} (wave
// halves of 32 lanes); swap16(a, b) returns {[a0, b0, a2, b2], [a1, b1, a3, b3]}
// (16-lane rows). With a == b they pair lane l with l ^ 32, or l ^ 16.
struct Pair {
  float lo, hi;
};
__device__ __forceinline__ Pair swap32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ Pair swap16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Max and sum over the 4 rows of a wave (same lane column); every lane gets
// the result, in a fixed order.
__device__ __forceinline__ float rows_max(float x) {
  const Pair p = swap32(x, x);
  const float y = fmaxf(p.lo, p.hi);
  const Pair q = swap16(y, y);
  return fmaxf(q.lo, q.hi);
}
__device__ __forceinline__ float rows_sum(float x) {
  const Pair p = swap32(x, x);
  const float y = p.lo + p.hi;
  const Pair q = swap16(y, y);
  return q.lo + q.hi;
}

// Two OCP FP8 E4M3 codes of a 32-bit word (bytes 0, 1, or 2, 3 when hi) as an
// exact bf16 pair, or as two floats (low byte first); one instruction each.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ float2 fp8x2_to_f32x2(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
  return make_float2(f[0], f[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float x) {
  x *= a.out_scale;
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(x);
  else
    static_cast<float*>(a.out)[idx] = x;
}

// Four consecutive outputs from element idx (a multiple of 4): one 16-byte
// store, or 8 bytes of bf16.
__device__ __forceinline__ void store_out4(const DecodeArgs& a, int64_t idx, float4 x) {
  x.x *= a.out_scale;
  x.y *= a.out_scale;
  x.z *= a.out_scale;
  x.w *= a.out_scale;
  if (a.out_bf16) {
    const uint2 v = make_uint2(uint32_t(f32_to_bf16_rne(x.x)) | (uint32_t(f32_to_bf16_rne(x.y)) << 16),
                               uint32_t(f32_to_bf16_rne(x.z)) | (uint32_t(f32_to_bf16_rne(x.w)) << 16));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + idx) = v;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + idx) = x;
  }
}

// Optional log-sum-exp output of output row `row` (= query row * hq + head):
// ln sum_j e^(score_j) from the row's (m, l) in log2 units, l = sum_j
// 2^(score_j * log2(e) - m): (m + log2 l) * ln 2; -inf for a row that saw no
// token (l = 0). Not scaled by the V scale.
__device__ __forceinline__ void store_lse(const DecodeArgs& a, int64_t row, float m, float l) {
  if (a.lse) a.lse[row] = l > 0.0f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
}

struct SplitSpan {
  int L;        // live tokens of the sequence (clamped to what the table and the plan can map)
  int lo;       // first token the sequence's query rows can see
  int begin;    // first token of the split
  int end;      // one past the last token
  int nsplit;   // splits this sequence uses
  bool clamped; // the sequence length was cut to what the table or the plan can map
};

// Bit 2 of the workspace error word: a sequence longer than the launch can
// map (seq_lens[b] above what max_pages_per_seq * block_size, or the splits
// planned for max_seq_len, cover) was cut to that range. Reported once per
// sequence, by the thread passed as `lead`.
__device__ __forceinline__ void flag_clamped(const DecodeArgs& a, const SplitSpan& sp, bool lead) {
  if (a.err && sp.clamped && lead) atomicOr(a.err, 4u);
}

// Longest token range the launch can map without a sliding window: what the
// block table can address and what the planned splits cover. (The host keeps
// max_seq_len <= 2^30, so the planned range fits an int.)
__device__ __forceinline__ int planned_cap(const DecodeArgs& a) {
  const int64_t cap = int64_t(a.max_pages) * int64_t(a.bdiv.d);
  const int64_t planned = int64_t(a.num_splits) * a.chunk;
  return int(cap < planned ? cap : planned);
}

// Tokens that sequence b's `rows` query rows can see: [lo, L), lo = 0, or with
// a sliding window max(0, L - rows + 1 - window) (the union of the rows'
// windows). Split s covers [lo + s * chunk, min(lo + (s + 1) * chunk, L)). L
// is clamped to what the block table can map and [lo, L) to what the planned
// splits cover, so a length above the host's max_seq_len can never index past
// the table, the grid or the workspace. split_span_len() takes the sequence
// length already read from seq_lens.
__device__ __forceinline__ SplitSpan split_span_len(const DecodeArgs& a, int64_t L, int s, int rows) {
  const int64_t table_cap = int64_t(a.max_pages) * int64_t(a.bdiv.d);
  const int64_t planned = int64_t(a.num_splits) * a.chunk;
  bool clamped = L > table_cap;
  L = L < 0 ? 0 : (L > table_cap ? table_cap : L);
  int64_t lo = 0;
  if (a.window > 0) {
    lo = L - rows + 1 - a.window;
    lo = lo < 0 ? 0 : lo;
  }
  if (L - lo > planned) {
    L = lo + planned;
    clamped = true;
  }
  SplitSpan r;
  r.clamped = clamped;
  r.L = int(L);
  r.lo = int(lo);
  r.begin = r.lo + s * a.chunk;
  r.end = min(r.begin + a.chunk, r.L);
  r.nsplit = (r.L - r.lo + a.chunk - 1) / a.chunk;
  return r;
}

__device__ __forceinline__ SplitSpan split_span(const DecodeArgs& a, int b, int s, int rows) {
  return split_span_len(a, a.seq_lens[b], s, rows);
}

// The single-query split kernel deals its splits out strided: [lo, L) is cut
// into blocks of kBlockTokens tokens and split s of the sequence's n = nsplit
// splits takes blocks s, s + n, s + 2n, ... (the same number of splits as the
// contiguous plan, and at most chunk / kBlockTokens blocks each, since the
// plan gives n * chunk >= L - lo). Slot i of the split's window holds token
// lo + kBlockTokens * (s + (i / kBlockTokens) * n) + i % kBlockTokens; the
// slot is live while that token is below L. At any moment the splits of one
// sequence then stream one band of the context together instead of n bands
// far apart.
constexpr int kBlockTokens = 32;

__device__ __forceinline__ int strided_token(int lo, int nsplit, int s, int i) {
  return lo + kBlockTokens * (s + (i / kBlockTokens) * nsplit) + i % kBlockTokens;
}

// Sub-steps of kBlockTokens tokens that split s (< sp.nsplit) reads.
__device__ __forceinline__ int strided_blocks(const SplitSpan& sp, int s) {
  const int nb = (sp.L - sp.lo + kBlockTokens - 1) / kBlockTokens;
  return (nb - s + sp.nsplit - 1) / sp.nsplit;
}

// Query rows of sequence b: rows [base, base + n) of the packed q and out.
// Uniform calls: base = b * q_len, n = q_len. Varlen calls take them from
// cu_q and check 0 <= cu_q[b] <= cu_q[b + 1] <= cu_q[num_seqs],
// cu_q[b + 1] <= num_seqs * q_len (the workspace's rows) and n <= q_len; a
// sequence that fails is skipped (n = 0, ok = false), so no row index leaves
// the packed buffers or the workspace.
struct QRows {
  int base;
  int n;
  bool ok;
};

__device__ __forceinline__ QRows seq_q_rows(const DecodeArgs& a, int b) {
  if (!a.cu_q) return {b * a.q_len, a.q_len, true};
  const int lo = a.cu_q[b], hi = a.cu_q[b + 1], total = a.cu_q[a.num_seqs];
  const bool ok = lo >= 0 && hi >= lo && hi - lo <= a.q_len && hi <= total &&
                  int64_t(hi) <= int64_t(a.num_seqs) * a.q_len;
  return {ok ? lo : 0, ok ? hi - lo : 0, ok};
}

// Element offsets of one physical page's first row for KV head g, for K and
// for V; k < 0 marks a table entry that is skipped.
struct PageOffs {
  int64_t k;
  int64_t v;
};

// Block-table slots split s may touch, from the launch plan alone: the pages
// of [s * chunk, min((s + 1) * chunk, planned_cap())). They contain the pages
// of the split's real range (which also depends on seq_lens) and start at the
// same page, so the table can be fetched while seq_lens is still in flight.
struct SplitPages {
  int p_first;
  int n;   // 0: the split is empty for every sequence length
};

// Without a sliding window: the pages split s may touch follow from the plan
// alone (the split starts at s * chunk for every sequence length).
__device__ __forceinline__ SplitPages split_pages(const DecodeArgs& a, int s) {
  const int begin = s * a.chunk;
  const int end = min(begin + a.chunk, planned_cap(a));
  SplitPages r;
  r.p_first = int(magic_div(uint32_t(begin), a.bdiv));
  r.n = end > begin ? int(magic_div(uint32_t(end - 1), a.bdiv)) - r.p_first + 1 : 0;
  return r;
}

// The pages of a split's real range [begin, end) (end > begin).
__device__ __forceinline__ SplitPages span_pages(const DecodeArgs& a, const SplitSpan& sp) {
  SplitPages r;
  r.p_first = int(magic_div(uint32_t(sp.begin), a.bdiv));
  r.n = int(magic_div(uint32_t(sp.end - 1), a.bdiv)) - r.p_first + 1;
  return r;
}

// Stage block-table entries [p_first, p_first + n) of sequence b in LDS as
// page offsets of KV head g. Entries outside [0, num_pages) are marked invalid
// (k = v = -1); only those the split really reads are reported, by
// flag_invalid_entries() once the sequence length is known. Entries past the
// sequence's last page are never dereferenced.
__device__ __forceinline__ void stage_table(const DecodeArgs& a, int b, int g, int p_first, int n,
                                            PageOffs* tbl) {
  const int32_t* row = a.table + int64_t(b) * a.max_pages + p_first;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = row[i];
    PageOffs po;
    if (uint32_t(e) >= uint32_t(a.num_pages)) {
      po.k = -1;
      po.v = -1;
    } else {
      po.k = int64_t(e) * a.k_sp + int64_t(g) * a.k_sh;
      po.v = int64_t(e) * a.v_sp + int64_t(g) * a.v_sh;
    }
    tbl[i] = po;
  }
}

// Set bit 0 of the workspace error word if one of the first n staged entries
// (the pages of the split's real range) is invalid. Call after the barrier
// that publishes the staged table.
__device__ __forceinline__ void flag_invalid_entries(const DecodeArgs& a, const PageOffs* tbl, int n) {
  if (!a.err) return;
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (tbl[i].k < 0) atomicOr(a.err, 1u);
}

// Prefill block: query positions [p0, p0 + rows) of a sequence with n new
// rows (of L tokens) see tokens up to L - n + p0 + rows - 1; the block is one
// span [lo, that + 1) (lo from the window), in a single split.
__device__ __forceinline__ SplitSpan prefill_span(const DecodeArgs& a, int b, int n, int p0, int rows) {
  const int64_t table_cap = int64_t(a.max_pages) * int64_t(a.bdiv.d);
  int64_t L = a.seq_lens[b];
  const bool clamped = L > table_cap;
  L = L < 0 ? 0 : (L > table_cap ? table_cap : L);
  int64_t end = L - n + p0 + rows;
  end = end < 0 ? 0 : end;
  int64_t lo = 0;
  if (a.window > 0) {
    lo = end - rows + 1 - a.window;
    lo = lo < 0 ? 0 : lo;
  }
  SplitSpan r;
  r.L = int(end);
  r.lo = int(lo);
  r.begin = r.lo;
  r.end = r.L;
  r.nsplit = 1;
  r.clamped = clamped;
  return r;
}

// Element offsets of token t's K and V rows; false if its page entry is
// invalid. The in-page part off * stride_tok fits 32 bits (checked on the host).
__device__ __forceinline__ bool token_row(const DecodeArgs& a, const PageOffs* tbl, int p_first, int t,
                                          int64_t& ko, int64_t& vo) {
  const uint32_t pg = magic_div(uint32_t(t), a.bdiv);
  const int off = t - int(pg * a.bdiv.d);
  const PageOffs po = tbl[int(pg) - p_first];
  ko = po.k + int64_t(off * int32_t(a.k_st));
  vo = po.v + int64_t(off * int32_t(a.v_st));
  return po.k >= 0;
}

// The same element offsets from page entry e (already read from the block
// table) and the token index; false if e is outside [0, num_pages).
__device__ __forceinline__ bool token_row_entry(const DecodeArgs& a, int e, int g, int t, int64_t& ko,
                                                int64_t& vo) {
  if (uint32_t(e) >= uint32_t(a.num_pages)) return false;
  const uint32_t pg = magic_div(uint32_t(t), a.bdiv);
  const int off = t - int(pg * a.bdiv.d);
  ko = (int64_t(e) * a.k_sp + int64_t(g) * a.k_sh) + int64_t(off * int32_t(a.k_st));
  vo = (int64_t(e) * a.v_sp + int64_t(g) * a.v_sh) + int64_t(off * int32_t(a.v_st));
  return true;
}

// Block-table entry of token t of sequence b (t below max_pages * B).
__device__ __forceinline__ int table_entry(const DecodeArgs& a, int b, int t) {
  return a.table[int64_t(b) * a.max_pages + magic_div(uint32_t(t), a.bdiv)];
}

// Element offsets of token t's rows with the entry read straight from
// sequence b's block-table row (no staged table). Same arithmetic as
// token_row(), so both give the same bits.
__device__ __forceinline__ bool token_row_direct(const DecodeArgs& a, int b, int g, int t, int64_t& ko,
                                                 int64_t& vo) {
  return token_row_entry(a, table_entry(a, b, t), g, t, ko, vo);
}

// Calls f(std::integral_constant<int, J>) for J = I .. N-1, so every index the
// body uses is a compile-time constant (no dynamic register indexing).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace
}  // namespace pkv
