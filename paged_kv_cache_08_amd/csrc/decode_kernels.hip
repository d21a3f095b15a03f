// The log-sum-exp merge kernel, the index-debug kernels and the dispatch of
// the single-query split kernel (decode_split.h) by window size.
//
// The merge combines the splits of one (sequence, query row, head) as the
// split-KV paragraph of "vLLM 下双卡 Radeon 上的混合 SSM 解码速率" describes:
// partial results of pieces of the KV range, reduced afterwards.
#include "decode_split.h"

namespace pkv {
namespace {

constexpr int kMergeSplitsLds = 1024;          // splits whose weights the merge keeps in LDS

// Wave-wide reductions (every lane gets the result; fixed butterfly order).
__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// out[b,i,h,:] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the
// sequence's splits with l_s > 0, M = max of their m_s; a row with no such
// split gets zeros. Workgroup = (64-column block, query head, query row x
// sequence), MW waves; wave w sums splits w, w + MW, .... The first
// accumulator loads are issued as early as possible (see kAhead). Every wave
// finds M and the denominator over all splits by itself (wave-wide
// reductions, the (m, l) pairs are a few hundred bytes) and keeps its
// weights 2^(m_s - M) in its own LDS row, so the only barrier is the one
// before the MW wave sums are added. All sums run in a
// fixed order. MW = 8 (8 splits per wave) for small grids (a batch-1 decode
// step has 24 (row, head) pairs), MW = 4 (16 splits per wave) otherwise:
// measured, small grids want more waves with fewer loads each, large grids
// the opposite. AHEAD: the first pass is loaded before the sequence length
// is known, for small grids (32K decode step -0.4 us) and for a single
// sequence, whose plan was made for its own length; in large grids of mostly
// short sequences those loads of unused splits cost more than they save.
template <int D, int MW, bool AHEAD>
__global__ __launch_bounds__(64 * MW) void lse_merge_kernel(DecodeArgs a) {
  constexpr int kPerWave = 64 / MW;   // accumulator loads in flight per thread per pass
  constexpr int kPass = MW * kPerWave;
  constexpr bool kAhead = AHEAD;
  static_assert(MW == 4 || MW == 8, "the final sum over the waves is written out for 4 or 8 waves");
  __shared__ float sm_w[MW][kMergeSplitsLds];
  __shared__ float part[MW][64];
  const int cb = blockIdx.z, h = blockIdx.y;
  const int i = blockIdx.x % a.q_len, b = blockIdx.x / a.q_len;
  const QRows qr = seq_q_rows(a, b);
  if (i >= qr.n) return;          // no such row in a varlen batch
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int d = cb * 64 + lane;
  const int64_t prow = (int64_t(qr.base) + i) * a.hq + h;
  const float* ml = a.part_ml + prow * a.num_splits * 2;
  const float* ac = a.part_acc + prow * a.num_splits * D;
  // The first pass of accumulators and the first 64 (m, l) pairs. With
  // kAhead they are loaded for every planned split before the sequence
  // length arrives (the row is known without a load unless the call is
  // varlen): one memory round trip instead of two, values of splits the
  // sequence does not use dropped, and no branch between these loads and
  // their first use, so they stay ahead of the wait for the length.
  // Otherwise only the splits the sequence uses are loaded, once the length
  // is known.
  float vals[kPerWave];
  float2 ml0;
  auto load_first = [&](int n) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = wave + MW * j;
      vals[j] = sidx < n ? ac[int64_t(sidx) * D + d] : 0.0f;
    }
    ml0 = lane < n ? reinterpret_cast<const float2*>(ml)[lane] : make_float2(0.0f, 0.0f);
  };
  if constexpr (kAhead) load_first(a.num_splits);
  const SplitSpan sp = split_span(a, b, 0, qr.n);
  const int ns = sp.nsplit;      // <= 1: the split kernel wrote the output
  if constexpr (!kAhead) {
    if (ns <= 1) return;
    load_first(ns);
  }
  // (m, l) of every split; a split with l = 0 (no visible token) gets m = -inf.
  float mloc = lane < ns && ml0.y > 0.0f ? ml0.x : -INFINITY;
  for (int t = lane + 64; t < ns; t += 64) {
    const float2 v = reinterpret_cast<const float2*>(ml)[t];
    mloc = fmaxf(mloc, v.y > 0.0f ? v.x : -INFINITY);
  }
  const float M = wave_max64(mloc);   // the same in every wave; -inf: no split has a visible token
  float dloc = 0.0f;
  for (int t = lane; t < ns; t += 64) {
    const float2 v = t < 64 ? ml0 : reinterpret_cast<const float2*>(ml)[t];
    const float f = v.y > 0.0f ? fast_exp2(v.x - M) : 0.0f;   // 0 for empty splits
    dloc += f * v.y;
    if (t < kMergeSplitsLds) sm_w[wave][t] = f;
  }
  const float den = wave_sum64(dloc);
  const float inv_den = 1.0f / den;
  // The wave reads back the weights it wrote (LDS operations of one wave run
  // in order; this keeps the compiler from moving the reads above the writes).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // First pass from the registers loaded up front; an unused split adds 0.
  float num = 0.0f;
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int sidx = wave + MW * j;   // < 64 <= kMergeSplitsLds
    const float f = sidx < ns ? sm_w[wave][sidx] : 0.0f;
    num += f * (sidx < ns ? vals[j] : 0.0f);
  }
  for (int s0 = kPass; s0 < ns; s0 += kPass) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = s0 + wave + MW * j;
      vals[j] = sidx < ns ? ac[int64_t(sidx) * D + d] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = s0 + wave + MW * j;
      if (sidx < ns) {
        float f;
        if (sidx < kMergeSplitsLds) {
          f = sm_w[wave][sidx];
        } else {
          const float2 v = reinterpret_cast<const float2*>(ml)[sidx];
          f = v.y > 0.0f ? fast_exp2(v.x - M) : 0.0f;
        }
        num += f * vals[j];
      }
    }
  }
  part[wave][lane] = num;
  __syncthreads();
  if (wave == 0 && ns > 1) {
    float t = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    if constexpr (MW == 8) t += (part[4][lane] + part[5][lane]) + (part[6][lane] + part[7][lane]);
    store_out(a, prow * D + d, M == -INFINITY ? 0.0f : t * inv_den);
    if (cb == 0 && lane == 0) store_lse(a, prow, M, M == -INFINITY ? 0.0f : den);
  }
}

// The same merge for head_dim 256 with whole rows per workgroup: workgroup =
// (query head, query row x sequence), MW waves, lane l holds columns
// 4l .. 4l + 3 and loads them with one 16-byte load per split, wave w sums
// splits w, w + MW, .... A quarter of the workgroups and of the load
// instructions of lse_merge_kernel for the same bytes (the grids of
// multi-row calls read tens of MB of partials). Same rule and order of
// additions per column as lse_merge_kernel.
template <int MW, bool AHEAD>
__global__ __launch_bounds__(64 * MW) void lse_merge_row_kernel(DecodeArgs a) {
  constexpr int D = 256;
  static_assert(MW == 4, "the final sum over the waves is written out for 4 waves");
  constexpr int kPerWave = 64 / MW;   // accumulator loads in flight per thread per pass
  constexpr int kPass = MW * kPerWave;
  __shared__ float sm_w[MW][kMergeSplitsLds];
  __shared__ __attribute__((aligned(16))) float4 part[MW][64];
  const int h = blockIdx.y;
  const int i = blockIdx.x % a.q_len, b = blockIdx.x / a.q_len;
  const QRows qr = seq_q_rows(a, b);
  if (i >= qr.n) return;          // no such row in a varlen batch
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t prow = (int64_t(qr.base) + i) * a.hq + h;
  const float* ml = a.part_ml + prow * a.num_splits * 2;
  const float* ac = a.part_acc + prow * a.num_splits * D + 4 * lane;
  float4 vals[kPerWave];
  float2 ml0;
  auto load_first = [&](int n) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = wave + MW * j;
      vals[j] = sidx < n ? *reinterpret_cast<const float4*>(ac + int64_t(sidx) * D) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ml0 = lane < n ? reinterpret_cast<const float2*>(ml)[lane] : make_float2(0.0f, 0.0f);
  };
  if constexpr (AHEAD) load_first(a.num_splits);
  const SplitSpan sp = split_span(a, b, 0, qr.n);
  const int ns = sp.nsplit;      // <= 1: the split kernel wrote the output
  if constexpr (!AHEAD) {
    if (ns <= 1) return;
    load_first(ns);
  } else {
    if (ns <= 1) return;
  }
  float mloc = lane < ns && ml0.y > 0.0f ? ml0.x : -INFINITY;
  for (int t = lane + 64; t < ns; t += 64) {
    const float2 v = reinterpret_cast<const float2*>(ml)[t];
    mloc = fmaxf(mloc, v.y > 0.0f ? v.x : -INFINITY);
  }
  const float M = wave_max64(mloc);
  float dloc = 0.0f;
  for (int t = lane; t < ns; t += 64) {
    const float2 v = t < 64 ? ml0 : reinterpret_cast<const float2*>(ml)[t];
    const float f = v.y > 0.0f ? fast_exp2(v.x - M) : 0.0f;
    dloc += f * v.y;
    if (t < kMergeSplitsLds) sm_w[wave][t] = f;
  }
  const float den = wave_sum64(dloc);
  const float inv_den = 1.0f / den;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto add = [&](float f, const float4& v) {
    num.x += f * v.x;
    num.y += f * v.y;
    num.z += f * v.z;
    num.w += f * v.w;
  };
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int sidx = wave + MW * j;
    const float f = sidx < ns ? sm_w[wave][sidx] : 0.0f;
    add(f, sidx < ns ? vals[j] : make_float4(0.f, 0.f, 0.f, 0.f));
  }
  for (int s0 = kPass; s0 < ns; s0 += kPass) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = s0 + wave + MW * j;
      vals[j] = sidx < ns ? *reinterpret_cast<const float4*>(ac + int64_t(sidx) * D) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int sidx = s0 + wave + MW * j;
      if (sidx < ns) {
        float f;
        if (sidx < kMergeSplitsLds) {
          f = sm_w[wave][sidx];
        } else {
          const float2 v = reinterpret_cast<const float2*>(ml)[sidx];
          f = v.y > 0.0f ? fast_exp2(v.x - M) : 0.0f;
        }
        add(f, vals[j]);
      }
    }
  }
  part[wave][lane] = num;
  __syncthreads();
  if (wave == 0) {
    // Pairwise over the 4 waves, as lse_merge_kernel<D, 4> adds them.
    const float4 u0 = part[0][lane], u1 = part[1][lane], u2 = part[2][lane], u3 = part[3][lane];
    const float4 t = make_float4((u0.x + u1.x) + (u2.x + u3.x), (u0.y + u1.y) + (u2.y + u3.y),
                                 (u0.z + u1.z) + (u2.z + u3.z), (u0.w + u1.w) + (u2.w + u3.w));
    const float4 o = M == -INFINITY ? make_float4(0.f, 0.f, 0.f, 0.f)
                                    : make_float4(t.x * inv_den, t.y * inv_den, t.z * inv_den, t.w * inv_den);
    store_out4(a, prow * D + 4 * lane, o);
    if (lane == 0) store_lse(a, prow, M, M == -INFINITY ? 0.0f : den);
  }
}

// The merge for plans of at most kFewSplits splits (short contexts, batched
// verify): workgroup = (query row slot, 4 query heads), one wave per head, each
// lane D / 64 columns, so the grid is not 64-column blocks times heads times
// rows of tiny workgroups. Every lane reads its head's (m, l) pairs (the same
// addresses across the wave), so the weights need no cross-lane step; the
// accumulator loads are all issued first. Same rule as lse_merge_kernel:
// M over the splits with l > 0, weights 2^(m_s - M), sums in split order.
constexpr int kFewSplits = 8;

template <int D>
__global__ __launch_bounds__(256) void lse_merge_few_kernel(DecodeArgs a) {
  constexpr int kCols = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  const int i = blockIdx.x % a.q_len, b = blockIdx.x / a.q_len;
  if (h >= a.hq) return;
  const QRows qr = seq_q_rows(a, b);
  if (i >= qr.n) return;          // no such row in a varlen batch
  const SplitSpan sp = split_span(a, b, 0, qr.n);
  if (sp.nsplit <= 1) return;    // written by the split kernel
  const int ns = sp.nsplit;      // <= num_splits <= kFewSplits
  const int64_t prow = (int64_t(qr.base) + i) * a.hq + h;
  const float* ml = a.part_ml + prow * a.num_splits * 2;
  const float* ac = a.part_acc + prow * a.num_splits * D;

  float acc[kFewSplits][kCols];
  float m[kFewSplits], l[kFewSplits];
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[s][c] = s < ns ? ac[int64_t(s) * D + c * 64 + lane] : 0.0f;
    const float2 v = s < ns ? reinterpret_cast<const float2*>(ml)[s] : make_float2(0.0f, 0.0f);
    m[s] = v.y > 0.0f ? v.x : -INFINITY;   // a split with no visible token weighs 0
    l[s] = v.y;
  }
  float M = m[0];
#pragma unroll
  for (int s = 1; s < kFewSplits; ++s) M = fmaxf(M, m[s]);
  if (M == -INFINITY) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) store_out(a, prow * D + c * 64 + lane, 0.0f);
    if (lane == 0) store_lse(a, prow, 0.0f, 0.0f);
    return;
  }
  float den = 0.0f, num[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) num[c] = 0.0f;
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s) {
    const float f = fast_exp2(m[s] - M);   // 0 for empty and unused splits
    den = fmaf(f, l[s], den);
#pragma unroll
    for (int c = 0; c < kCols; ++c) num[c] = fmaf(f, acc[s][c], num[c]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int c = 0; c < kCols; ++c) store_out(a, prow * D + c * 64 + lane, num[c] * inv);
  if (lane == 0) store_lse(a, prow, M, den);
}

// Debug: offsets of every live token row of the split ranges, found both
// ways the kernels find them: token_row() on the staged table (the MFMA
// kernel) and token_row_direct() on the table row in global memory (the
// single-query split kernel). A token on which they disagree gets -3, an
// invalid page entry -2.
constexpr int kDebugThreads = 512;

__global__ __launch_bounds__(kDebugThreads) void debug_offsets_kernel(DecodeArgs a, int g, int max_seq_len,
                                                                 int64_t* k_off, int64_t* v_off) {
  __shared__ PageOffs tbl[kMaxChunk + 2];
  const int s = blockIdx.x, b = blockIdx.y;
  const SplitSpan sp = split_span(a, b, s, a.q_len);
  if (sp.begin >= sp.L) return;
  const SplitPages pages = a.window == 0 ? split_pages(a, s) : span_pages(a, sp);
  const int p_first = pages.p_first;
  stage_table(a, b, g, p_first, pages.n, tbl);
  __syncthreads();
  const int t_end = min(sp.end, max_seq_len);
  for (int t = sp.begin + threadIdx.x; t < t_end; t += kDebugThreads) {
    int64_t ko = 0, vo = 0, kd = 0, vd = 0;
    const bool ok = token_row(a, tbl, p_first, t, ko, vo);     // staged table (MFMA kernel)
    const bool okd = token_row_direct(a, b, g, t, kd, vd);     // table row in global memory (split kernel)
    const bool same = ok == okd && (!ok || (ko == kd && vo == vd));
    k_off[int64_t(b) * max_seq_len + t] = !same ? -3 : ok ? ko : -2;
    v_off[int64_t(b) * max_seq_len + t] = !same ? -3 : ok ? vo : -2;
  }
}

__global__ void debug_ranges_kernel(DecodeArgs a, int32_t* ranges) {
  const int b = blockIdx.x;
  for (int s = threadIdx.x; s < a.num_splits; s += blockDim.x) {
    const SplitSpan sp = split_span(a, b, s, a.q_len);
    const int lo = min(sp.begin, sp.L);
    const int hi = max(lo, sp.end);
    ranges[(int64_t(b) * a.num_splits + s) * 2] = lo;
    ranges[(int64_t(b) * a.num_splits + s) * 2 + 1] = hi;
  }
}

// Debug: the split and window slot the single-query split kernel reads each
// token with, written forward from strided_token() and strided_blocks() the
// way the kernel derives them: slots[(b * max_seq_len + t) * 2] = split,
// [... + 1] = slot. Tokens that no slot reads keep what the host wrote.
__global__ __launch_bounds__(kMaxChunk) void debug_token_splits_kernel(DecodeArgs a, int max_seq_len, int win,
                                                                       int32_t* slots) {
  const int s = blockIdx.x, b = blockIdx.y;
  const SplitSpan sp = split_span(a, b, s, 1);
  if (sp.begin >= sp.L) return;
  const int n_sub = strided_blocks(sp, s);
  for (int i = threadIdx.x; i < win; i += blockDim.x) {
    const int t = strided_token(sp.lo, sp.nsplit, s, i);
    if (i / kBlockTokens < n_sub && t < sp.L && t < max_seq_len) {
      slots[(int64_t(b) * max_seq_len + t) * 2] = s;
      slots[(int64_t(b) * max_seq_len + t) * 2 + 1] = i;
    }
  }
}

}  // namespace

bool decode_supported(int head_dim, int group) {
  return (head_dim == 128 || head_dim == 256) && group >= 1 && group <= 8;
}

int decode_window(int chunk) {
  return chunk <= 64 ? 64 : chunk <= 128 ? 128 : chunk <= 256 ? 256 : 512;
}

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
  // FP8 caches: q.k and p.v on MFMA (the VALU kernel would be bound by
  // widening the codes). Measured per step on one MI355X against the VALU
  // kernel: 32K 20.5 vs 23.0 us, 16K 14.4 vs 16.3 us, 4K 10.3 vs 11.0 us,
  // 16-sequence mixed batch 48.3 vs 61.4 us.
  if (a.kv_fp8) return launch_decode_mfma_fp8(a, head_dim, group, st, e0, e1);
  switch (decode_window(a.chunk)) {
    case 64: return launch_decode_split_w64(a, head_dim, group, st, e0, e1);
    case 128: return launch_decode_split_w128(a, head_dim, group, st, e0, e1);
    case 256: return launch_decode_split_w256(a, head_dim, group, st, e0, e1);
    default:
      // Grids of several workgroups per CU run the shallower ring.
      return (a.many_wg ? launch_decode_split_w512_many : launch_decode_split_w512)(a, head_dim, group, st, e0, e1);
  }
}

hipError_t launch_lse_merge(const DecodeArgs& a, int head_dim, hipStream_t st) {
  if (a.num_splits <= kFewSplits) {
    dim3 grid(a.q_len * a.num_seqs, (a.hq + 3) / 4);
    if (head_dim == 256)
      hipLaunchKernelGGL(lse_merge_few_kernel<256>, grid, dim3(256), 0, st, a);
    else if (head_dim == 128)
      hipLaunchKernelGGL(lse_merge_few_kernel<128>, grid, dim3(256), 0, st, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  dim3 grid(a.q_len * a.num_seqs, a.hq, head_dim / 64);
  const bool small = int64_t(a.q_len) * a.num_seqs * a.hq < 128;
  const bool one_seq = a.num_seqs == 1 && a.cu_q == nullptr;
  if (head_dim == 256 && !small && a.q_len > 1) {
    dim3 rgrid(a.q_len * a.num_seqs, a.hq);
    if (one_seq)
      hipLaunchKernelGGL((lse_merge_row_kernel<4, true>), rgrid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((lse_merge_row_kernel<4, false>), rgrid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (head_dim == 256) {
    if (small)
      hipLaunchKernelGGL((lse_merge_kernel<256, 8, true>), grid, dim3(512), 0, st, a);
    else if (one_seq)
      hipLaunchKernelGGL((lse_merge_kernel<256, 4, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((lse_merge_kernel<256, 4, false>), grid, dim3(256), 0, st, a);
  } else if (head_dim == 128) {
    if (small)
      hipLaunchKernelGGL((lse_merge_kernel<128, 8, true>), grid, dim3(512), 0, st, a);
    else if (one_seq)
      hipLaunchKernelGGL((lse_merge_kernel<128, 4, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((lse_merge_kernel<128, 4, false>), grid, dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_debug_offsets(const DecodeArgs& a, int kv_head, int max_seq_len, int64_t* k_off,
                                int64_t* v_off, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_seqs);
  hipLaunchKernelGGL(debug_offsets_kernel, grid, dim3(kDebugThreads), 0, st, a, kv_head, max_seq_len, k_off, v_off);
  return hipGetLastError();
}

hipError_t launch_debug_token_splits(const DecodeArgs& a, int max_seq_len, int32_t* slots, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_seqs);
  hipLaunchKernelGGL(debug_token_splits_kernel, grid, dim3(kMaxChunk), 0, st, a, max_seq_len,
                     decode_window(a.chunk), slots);
  return hipGetLastError();
}

hipError_t launch_debug_ranges(const DecodeArgs& a, int32_t* ranges, hipStream_t st) {
  hipLaunchKernelGGL(debug_ranges_kernel, dim3(a.num_seqs), dim3(64), 0, st, a, ranges);
  return hipGetLastError();
}

}  // namespace pkv
