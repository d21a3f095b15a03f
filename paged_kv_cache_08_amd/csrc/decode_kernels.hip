// Single-query paged decode attention for gfx950 (wave64, CDNA4): the split
// kernel, the log-sum-exp merge kernel and the index-debug kernels.
//
// What is computed follows "DCU page832 attention" (luanjiahao.me): §1 and §5
// for the address of a token row (logical page = t / B, offset = t % B,
// physical page from the block table, then page / token / head strides), §5
// for score = dot(q, k) * scale with an online softmax over V, and §7 for the
// fact that decode walks every logical page. The split of one (sequence, KV
// head) context over many workgroups followed by a merge is the split-KV
// paragraph of "vLLM 下双卡 Radeon 上的混合 SSM 解码速率".
//
// Work mapping (one workgroup = one split of one (sequence, KV head)):
//   * 4 waves x 4 token rows per wave: 16 consecutive logical tokens per
//     sub-step, one token row per 16-lane DPP row.
//   * Each lane owns D/16 head-dim elements of its token row and loads them
//     with 16-byte global loads (a 512-byte K row of D=256 is read by 16 lanes
//     in two fully used 256-byte segments).
//   * The G query heads of the GQA group all use the row held in registers, so
//     K and V are fetched once per group.
//   * q.k partial sums are reduced across the 16 lanes of a row with four DPP
//     butterfly adds (quad_perm, row_half_mirror, row_mirror); all lanes end up
//     with the same bits.
//   * Online softmax in log2 units, per token row, with a lazy reference max:
//     the accumulators are rescaled only when a score exceeds the reference by
//     more than 2^8, so probabilities stay <= 256 and rescales are rare.
//   * Token rows, then waves, are merged in a fixed order; the split's
//     (reference max, sum, accumulator) go to the workspace, or the normalised
//     output directly when the sequence has a single split.
// Every reduction order depends only on logical token indices and the split
// plan, never on block_size or physical page ids, so the same logical K/V gives
// bitwise-identical output for any page size or page placement.
#include <math.h>

#include "pkv_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerWave = 64 / kLanesPerRow;
constexpr int kStep = kWaves * kRowsPerWave;   // tokens per workgroup sub-step
constexpr int kSub = 2;                        // sub-steps per pipeline stage
constexpr float kLazy = 8.0f;                  // log2 headroom before a rescale

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

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_move<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_move<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_move<0x141>(x);   // row_half_mirror
  x += dpp_move<0x140>(x);   // row_mirror
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float x) {
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(x);
  else
    static_cast<float*>(a.out)[idx] = x;
}

struct SplitSpan {
  int L;        // live tokens of the sequence (clamped to what the table can map)
  int begin;    // first token of the split
  int end;      // one past the last token
  int nsplit;   // splits this sequence uses
};

// Split s of sequence b: [s * chunk, min((s + 1) * chunk, L)). L is clamped to
// what the block table can map and to what the planned splits cover, so a
// length above the host's max_seq_len can never index past the table, the
// grid or the workspace.
__device__ __forceinline__ SplitSpan split_span(const DecodeArgs& a, int b, int s) {
  int64_t cap = int64_t(a.max_pages) * int64_t(a.bdiv.d);
  const int64_t planned = int64_t(a.num_splits) * a.chunk;
  cap = cap < planned ? cap : planned;
  int64_t L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  SplitSpan r;
  r.L = int(L);
  r.begin = s * a.chunk;
  r.end = min(r.begin + a.chunk, r.L);
  r.nsplit = (r.L + a.chunk - 1) / a.chunk;
  return r;
}

// Stage block-table entries [p_first, p_first + n) of sequence b in LDS.
// Entries outside [0, num_pages) become -1 (their tokens are skipped) and set
// bit 0 of the workspace error word.
__device__ __forceinline__ void stage_table(const DecodeArgs& a, int b, int p_first, int n, int* tbl) {
  const int32_t* row = a.table + int64_t(b) * a.max_pages + p_first;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int e = row[i];
    if (uint32_t(e) >= uint32_t(a.num_pages)) {
      if (a.err) atomicOr(a.err, 1u);
      e = -1;
    }
    tbl[i] = e;
  }
}

// Element offsets of token t's K and V rows of KV head g; false if its page
// entry is invalid.
__device__ __forceinline__ bool token_row(const DecodeArgs& a, const int* tbl, int p_first, int t,
                                          int g, int64_t& ko, int64_t& vo) {
  const uint32_t pg = magic_div(uint32_t(t), a.bdiv);
  const int off = t - int(pg * a.bdiv.d);
  const int phys = tbl[int(pg) - p_first];
  ko = int64_t(phys) * a.k_sp + int64_t(off) * a.k_st + int64_t(g) * a.k_sh;
  vo = int64_t(phys) * a.v_sp + int64_t(off) * a.v_st + int64_t(g) * a.v_sh;
  return phys >= 0;
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeArgs a) {
  constexpr int kEpl = D / kLanesPerRow;   // head-dim elements per lane: 16 or 8
  constexpr int kCpl = kEpl / 8;           // 16-byte chunks per lane: 2 or 1
  static_assert(kCpl >= 1 && kEpl % 8 == 0, "head_dim must be a multiple of 128");

  __shared__ int tbl[kTblCap];
  __shared__ float mrg_acc[kWaves][G][D];
  __shared__ float mrg_ml[kWaves][G][2];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const SplitSpan sp = split_span(a, b, s);
  const int64_t out_row0 = (int64_t(b) * a.hq + int64_t(g) * G) * D;   // q_len == 1

  if (sp.begin >= sp.L) {
    if (s == 0)   // empty sequence: zeros
      for (int i = tid; i < G * D; i += kThreads) store_out(a, out_row0 + i, 0.0f);
    return;
  }
  const int p_first = int(magic_div(uint32_t(sp.begin), a.bdiv));
  const int p_last = int(magic_div(uint32_t(sp.end - 1), a.bdiv));
  stage_table(a, b, p_first, p_last - p_first + 1, tbl);

  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane >> 4, col = lane & 15;

  // q of the group's G heads: lane col holds elements [k*128 + col*8, +8) of each head.
  uint4 qv[G][kCpl];
  {
    const uint16_t* qp = a.q + out_row0 + col * 8;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < kCpl; ++k)
        qv[h][k] = *reinterpret_cast<const uint4*>(qp + h * D + k * 128);
  }
  __syncthreads();

  float m[G], l[G], acc[G][kEpl];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[h][e] = 0.0f;
  }

  const int my = wave * kRowsPerWave + row;   // token of this row within a sub-step

  auto fetch = [&](int base, uint4 (&kk)[kSub][kCpl], uint4 (&vv)[kSub][kCpl], bool (&ok)[kSub]) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const int t = base + u * kStep + my;
      int64_t ko = 0, vo = 0;
      bool valid = t < sp.end;
      if (valid) valid = token_row(a, tbl, p_first, t, g, ko, vo);
      ok[u] = valid;
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        kk[u][k] = make_uint4(0, 0, 0, 0);
        vv[u][k] = make_uint4(0, 0, 0, 0);
      }
      if (valid) {
        const uint16_t* kp = a.k + ko + col * 8;
        const uint16_t* vp = a.v + vo + col * 8;
#pragma unroll
        for (int k = 0; k < kCpl; ++k) {
          kk[u][k] = *reinterpret_cast<const uint4*>(kp + k * 128);
          vv[u][k] = *reinterpret_cast<const uint4*>(vp + k * 128);
        }
      }
    }
  };

  auto consume = [&](const uint4 (&kk)[kSub][kCpl], const uint4 (&vv)[kSub][kCpl], const bool (&ok)[kSub]) {
    float sc[kSub][G];
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = 0.0f;
#pragma unroll
        for (int k = 0; k < kCpl; ++k) {
          d0 = dot2_bf16(qv[h][k].x, kk[u][k].x, d0);
          d0 = dot2_bf16(qv[h][k].y, kk[u][k].y, d0);
          d0 = dot2_bf16(qv[h][k].z, kk[u][k].z, d0);
          d0 = dot2_bf16(qv[h][k].w, kk[u][k].w, d0);
        }
        const float r = row16_sum(d0) * a.scale_log2;
        sc[u][h] = ok[u] ? r : -INFINITY;
      }
    float p[kSub][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < kSub; ++u) mx = fmaxf(mx, sc[u][h]);
      if (mx > m[h] + kLazy) {
        const float al = fast_exp2(m[h] - mx);
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[h][e] *= al;
        m[h] = mx;
      }
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        p[u][h] = ok[u] ? fast_exp2(sc[u][h] - m[h]) : 0.0f;
        l[h] += p[u][h];
      }
    }
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        const uint32_t w4[4] = {vv[u][k].x, vv[u][k].y, vv[u][k].z, vv[u][k].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float v0 = bf16_lo(w4[w]), v1 = bf16_hi(w4[w]);
          const int e = k * 8 + w * 2;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][e] = fmaf(p[u][h], v0, acc[h][e]);
            acc[h][e + 1] = fmaf(p[u][h], v1, acc[h][e + 1]);
          }
        }
      }
  };

  uint4 kA[kSub][kCpl], vA[kSub][kCpl], kB[kSub][kCpl], vB[kSub][kCpl];
  bool okA[kSub], okB[kSub];
  int base = sp.begin;
  fetch(base, kA, vA, okA);
  while (true) {
    fetch(base + kSub * kStep, kB, vB, okB);
    consume(kA, vA, okA);
    base += kSub * kStep;
    if (base >= sp.end) break;
    fetch(base + kSub * kStep, kA, vA, okA);
    consume(kB, vB, okB);
    base += kSub * kStep;
    if (base >= sp.end) break;
  }

  // Merge the 4 token rows of each wave (fixed butterfly order).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = fmaxf(m[h], __shfl_xor(m[h], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float w = (m[h] == -INFINITY) ? 0.0f : fast_exp2(m[h] - M);
    float lw = l[h] * w;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      float x = acc[h][e] * w;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[h][e] = x;
    }
    m[h] = M;
    l[h] = lw;
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < kCpl; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) mrg_acc[wave][h][k * 128 + col * 8 + j] = acc[h][k * 8 + j];
    if (col == 0)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mrg_ml[wave][h][0] = m[h];
        mrg_ml[wave][h][1] = l[h];
      }
  }
  __syncthreads();

  // Merge the waves (fixed order) and write the split's result.
  const int64_t prow0 = int64_t(b) * a.q_len * a.hq + int64_t(g) * G;   // partial row of head 0, query row 0
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i - h * D;
    float M = mrg_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg_ml[w][h][0]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mrg_ml[w][h][0];
      const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
      num += f * mrg_acc[w][h][d];
      den += f * mrg_ml[w][h][1];
    }
    if (sp.nsplit == 1) {
      store_out(a, out_row0 + i, den > 0.0f ? num / den : 0.0f);
    } else {
      const int64_t pr = (prow0 + h) * a.num_splits + s;
      a.part_acc[pr * D + d] = num;
      if (d == 0) {
        a.part_ml[pr * 2] = M;
        a.part_ml[pr * 2 + 1] = den;
      }
    }
  }
}

// out[b,i,h,:] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the
// sequence's splits, M = max_s m_s; splits with no visible token carry
// m = -inf and weigh nothing. One workgroup per (query head, query row, seq).
template <int D>
__global__ __launch_bounds__(D) void lse_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int d = threadIdx.x;
  const SplitSpan sp = split_span(a, b, 0);
  if (sp.nsplit <= 1) return;    // written by the split kernel
  const int64_t prow = (int64_t(b) * a.q_len + i) * a.hq + h;
  const float* ml = a.part_ml + prow * a.num_splits * 2;
  const float* ac = a.part_acc + prow * a.num_splits * D;
  const int64_t oidx = prow * D + d;
  float M = -INFINITY;
  for (int s = 0; s < sp.nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  if (M == -INFINITY) {
    store_out(a, oidx, 0.0f);
    return;
  }
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < sp.nsplit; ++s) {
    const float ms = ml[2 * s];
    const float f = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - M);
    den += f * ml[2 * s + 1];
    num += f * ac[int64_t(s) * D + d];
  }
  store_out(a, oidx, den > 0.0f ? num / den : 0.0f);
}

// Debug: offsets of every live token row, through the same split range,
// table staging and token_row() the split kernel uses.
__global__ __launch_bounds__(kThreads) void debug_offsets_kernel(DecodeArgs a, int g, int max_seq_len,
                                                                 int64_t* k_off, int64_t* v_off) {
  __shared__ int tbl[kTblCap];
  const int s = blockIdx.x, b = blockIdx.y;
  const SplitSpan sp = split_span(a, b, s);
  if (sp.begin >= sp.L) return;
  const int p_first = int(magic_div(uint32_t(sp.begin), a.bdiv));
  const int p_last = int(magic_div(uint32_t(sp.end - 1), a.bdiv));
  stage_table(a, b, p_first, p_last - p_first + 1, tbl);
  __syncthreads();
  const int t_end = min(sp.end, max_seq_len);
  for (int t = sp.begin + threadIdx.x; t < t_end; t += kThreads) {
    int64_t ko, vo;
    const bool ok = token_row(a, tbl, p_first, t, g, ko, vo);
    k_off[int64_t(b) * max_seq_len + t] = ok ? ko : -2;
    v_off[int64_t(b) * max_seq_len + t] = ok ? vo : -2;
  }
}

__global__ void debug_ranges_kernel(DecodeArgs a, int32_t* ranges) {
  const int b = blockIdx.x;
  for (int s = threadIdx.x; s < a.num_splits; s += blockDim.x) {
    const SplitSpan sp = split_span(a, b, s);
    const int lo = min(sp.begin, sp.L);
    const int hi = max(lo, sp.end);
    ranges[(int64_t(b) * a.num_splits + s) * 2] = lo;
    ranges[(int64_t(b) * a.num_splits + s) * 2 + 1] = hi;
  }
}

template <int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.num_splits, a.hkv, a.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<D, G>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_decode_t<D, 1>(a, st);
    case 2: return launch_decode_t<D, 2>(a, st);
    case 3: return launch_decode_t<D, 3>(a, st);
    case 4: return launch_decode_t<D, 4>(a, st);
    case 5: return launch_decode_t<D, 5>(a, st);
    case 6: return launch_decode_t<D, 6>(a, st);
    case 7: return launch_decode_t<D, 7>(a, st);
    case 8: return launch_decode_t<D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int head_dim, int group) {
  return (head_dim == 128 || head_dim == 256) && group >= 1 && group <= 8;
}

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int group, hipStream_t st) {
  if (head_dim == 256) return launch_decode_d<256>(a, group, st);
  if (head_dim == 128) return launch_decode_d<128>(a, group, st);
  return hipErrorInvalidValue;
}

hipError_t launch_lse_merge(const DecodeArgs& a, int head_dim, hipStream_t st) {
  dim3 grid(a.hq, a.q_len, a.num_seqs);
  if (head_dim == 256)
    hipLaunchKernelGGL(lse_merge_kernel<256>, grid, dim3(256), 0, st, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(128), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_debug_offsets(const DecodeArgs& a, int kv_head, int max_seq_len, int64_t* k_off,
                                int64_t* v_off, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_seqs);
  hipLaunchKernelGGL(debug_offsets_kernel, grid, dim3(kThreads), 0, st, a, kv_head, max_seq_len, k_off, v_off);
  return hipGetLastError();
}

hipError_t launch_debug_ranges(const DecodeArgs& a, int32_t* ranges, hipStream_t st) {
  hipLaunchKernelGGL(debug_ranges_kernel, dim3(a.num_seqs), dim3(64), 0, st, a, ranges);
  return hipGetLastError();
}

}  // namespace pkv
