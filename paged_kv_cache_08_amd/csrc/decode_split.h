// The single-query split kernel for bf16 caches on gfx950 (wave64, CDNA4),
// templated on head_dim D, group size G (query heads per KV head), window
// NBLK (strided blocks of 32 tokens; a split holds at most NBLK * 32 tokens)
// and its register ring depth. Each window size is instantiated in its own
// source file (decode_w64.hip .. decode_w512.hip, and decode_w512_many.hip
// with a shallower ring for grids of several workgroups per CU) so the fully
// unrolled kernels compile in parallel. FP8 caches run the MFMA kernel of
// decode_mfma.h, which the code widening would otherwise make VALU-bound.
//
// What is computed follows "DCU page832 attention" (luanjiahao.me): §1 and §5
// for the address of a token row (logical page = t / B, offset = t % B,
// physical page from the block table, then page / token / head strides), §5
// for score = dot(q, k) * scale with a softmax-weighted sum of V, and §7 for
// the fact that decode walks every logical page. The split of one (sequence,
// KV head) context over many workgroups, merged afterwards, is the split-KV
// paragraph of "vLLM 下双卡 Radeon 上的混合 SSM 解码速率".
//
// Work mapping (one workgroup = one split of one (sequence, KV head)):
//   * Splits are strided: the sequence's context is dealt out in blocks of
//     32 tokens, block k to split k mod n (n = the sequence's split count),
//     so the n workgroups of a (sequence, KV head) stream neighbouring blocks
//     at the same time. (Bare reads of the same bytes finish about 3% sooner
//     when the whole chip streams one band than with n bands far apart.)
//   * 4 waves (one per SIMD) x 4 token rows per wave: 16 consecutive logical
//     tokens of one strided block per sub-step, one token row per 16-lane DPP
//     row. Each lane owns D/16 head-dim elements of its row and loads them
//     with 16-byte global loads (a 512-byte K row of D = 256 is read by 16
//     lanes in two fully used 256-byte segments). The G query heads of the group all use the row held
//     in registers, so K and V are fetched once per group. The K/V loads are
//     non-temporal: each byte is read once per call.
//   * The split is one window, fully unrolled: a K pass over its NS sub-steps,
//     then a V pass over the same tokens. Loads run through a ring of register
//     buffers that spans both passes, so the first V loads are in flight while
//     the last scores are computed. Loads are branch-free: a masked row (past
//     the split end, or an invalid page entry) reads the q row instead.
//   * K pass: q.k partial sums are reduced across the 16 lanes of a row with a
//     DPP reduce-scatter (row_mirror, row_half_mirror, quad_perm); lanes 2h and
//     2h + 1 keep head h's score, in log2 units.
//   * V pass: with the exact maximum of the lane's own window scores, each
//     probability is computed once per (token, head), broadcast to the row with
//     DPP row_newbcast, and accumulated with fp32 FMAs.
//   * Token offsets: one thread per window slot (two slots per thread in
//     4-wave workgroups) divides its token index by
//     the page size (multiply-high), reads the block-table entry and stores
//     the token's K and V row offsets in LDS, once per split (without a
//     sliding window, while seq_lens is still in flight, for the stride of a
//     sequence that uses every split); a masked slot gets the offset of the
//     q row. A lane then costs one LDS read and one address add per K or V
//     row, instead of every lane of a row repeating the division and the
//     table lookup.
//   * Epilogue: the 4 token rows of a wave are merged by a reduce-scatter over
//     lane swaps (v_permlane32_swap, v_permlane16_swap); the W waves publish
//     their sums with their reference max in LDS and, after one barrier, are
//     rescaled to the workgroup max and added in a fixed order; the split's
//     (max, sum, accumulator) go to the workspace, or the normalised output
//     directly when the sequence has a single split.
// Every reduction order depends only on logical token indices and the split
// plan, never on block_size or physical page ids, so the same logical K/V gives
// bitwise-identical output for any page size or page placement.
#pragma once

#include <math.h>

#include <hip/hip_ext.h>

#include "pkv_device.h"

namespace pkv {
namespace {


// Workgroup shape: 4 waves of 4 token rows (16 lanes per row), one wave per
// SIMD; a sub-step reads 16 consecutive tokens of one strided block. Against
// 8-wave workgroups (two waves per SIMD, rings of 6), measured per step: the
// batch-1 32K call 28.9 -> 27.3 us, the 16-sequence mixed batch 81.6 -> 74.4
// us, the 32 / 8-head dense control 29.1 -> 27.0 us, 1K 10.04 -> 9.68 us, 4K
// 11.35 -> 10.98 us, a 2048-token sliding window 10.38 -> 10.1 us.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerWave = 64 / kLanesPerRow;
static_assert(kBlockTokens % (kWaves * kRowsPerWave) == 0, "sub-steps tile a strided block");
// Register ring depth (steps in flight + 1), a template argument of the
// kernel. Measured with 4-wave workgroups, depths 2 / 3 / 4 / 5: the 32K step
// 33.4 / 27.6 / 27.3 / 28.5 us (page 16: 33.8 / 28.1 / 27.5 / 28.5), the
// mixed batch 81.8 / 74.1 / 74.4 / 75.3 us, the dense control 31.8 / 27.0 /
// 27.3 / 27.9 us, 4K 11.5 / 11.0 / 10.9 / 11.2 us. Depth 4, and 3 for the
// 512-token kernels launched on grids of more workgroups than the device
// has CUs.
constexpr int kRingOne = 4;    // grids of at most one workgroup per CU, and shorter windows
constexpr int kRingMany = 3;   // 512-token windows on grids of several workgroups per CU
constexpr float kMinit = -1.0e30f;             // floor of a row's max (finite: no inf - inf)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16 bytes read with a non-temporal load (global_load_dwordx4 ... nt).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp_move_full<0x150 + N>(x);
}

// out[h] = value held by lane 2h of the row (the lanes that own head h after
// the reduce-scatter below).
template <int G>
__device__ __forceinline__ void head_bcast(float x, float (&out)[G]) {
  if constexpr (G > 0) out[0] = row_bcast<0>(x);
  if constexpr (G > 1) out[1] = row_bcast<2>(x);
  if constexpr (G > 2) out[2] = row_bcast<4>(x);
  if constexpr (G > 3) out[3] = row_bcast<6>(x);
  if constexpr (G > 4) out[4] = row_bcast<8>(x);
  if constexpr (G > 5) out[5] = row_bcast<10>(x);
  if constexpr (G > 6) out[6] = row_bcast<12>(x);
  if constexpr (G > 7) out[7] = row_bcast<14>(x);
}

// Reduce-scatter of up to 8 per-lane partial sums over the 16 lanes of a row.
// Partners are lane ^ 15 (row_mirror), ^ 7 (row_half_mirror), ^ 2 and ^ 1
// (quad_perm); at each step a lane keeps the half of the heads selected by one
// bit of its lane index and receives its partner's copy of that half. Lanes 2h
// and 2h + 1 end with the full sum of head h (bitwise equal); the order of the
// additions depends only on the lane index.
template <int G>
__device__ __forceinline__ float reduce_scatter16(const float (&x)[G], int col) {
  float y[4], z[2];
  const bool b3 = col >= 8, b2 = (col & 4) != 0, b1 = (col & 2) != 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = j < G ? x[j] : 0.0f;
    const float hi = j + 4 < G ? x[j + 4] : 0.0f;
    const float keep = b3 ? hi : lo;
    const float send = b3 ? lo : hi;
    y[j] = keep + dpp_move<0x140>(send);   // row_mirror
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b2 ? y[j + 2] : y[j];
    const float send = b2 ? y[j] : y[j + 2];
    z[j] = keep + dpp_move<0x141>(send);   // row_half_mirror
  }
  float w;
  {
    const float keep = b1 ? z[1] : z[0];
    const float send = b1 ? z[0] : z[1];
    w = keep + dpp_move<0x4E>(send);       // quad_perm [2,3,0,1]
  }
  return w + dpp_move<0xB1>(w);            // quad_perm [1,0,3,2]
}

// Head-dim element of lane column col's e-th element: two 16-byte pieces per
// 512-byte row (D = 256), lane col holds [k * 128 + col * 8, +8) of piece k.
__device__ __forceinline__ int elem_d(int col, int e) { return (e / 8) * 128 + col * 8 + (e % 8); }

template <int D, int G, int NBLK, int RING, bool WT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int kStep = kWaves * kRowsPerWave;          // tokens per workgroup sub-step
  constexpr int kSubSteps = NBLK * (kBlockTokens / kStep);
  constexpr int kEpl = D / kLanesPerRow;   // head-dim elements per lane: 16 or 8
  constexpr int kCq = kEpl / 8;            // 16-byte pieces of q per lane: 2 or 1
  constexpr int kCpl = kCq;                // 16-byte K/V loads per lane and row
  constexpr int kSteps = 2 * kSubSteps;    // K pass, then V pass
  constexpr int kRing = RING;
  constexpr int kWin = kSubSteps * kStep;  // tokens of the window
  constexpr int kEsz = 2;                  // bytes per cache element
  static_assert(kCpl >= 1 && kEpl % 8 == 0, "head_dim must be a multiple of 128");
  static_assert(G <= 8, "at most 8 query heads per KV head");
  static_assert(RING >= 2, "at least one step in flight");
  static_assert(kSubSteps >= 1 && kWin <= kMaxChunk, "window of at most kMaxChunk tokens");

  __shared__ int64_t tok_k[kWin];   // element offset of each window token's K row (a masked token: the q row)
  __shared__ int64_t tok_v[kWin];
  __shared__ __attribute__((aligned(16))) float mrg_acc[kWaves][G][D];
  __shared__ __attribute__((aligned(16))) float mrg_m[G][kWaves];
  __shared__ __attribute__((aligned(16))) float mrg_l[G][kWaves];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t out_row0 = (int64_t(b) * a.hq + int64_t(g) * G) * D;   // q_len == 1
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane >> 4, col = lane & 15;

  // A masked token (past the split end, or behind an invalid page entry)
  // reads the group's first q row instead: finite and in bounds. Its offset
  // from each cache base, in cache elements (every base is 16-byte aligned).
  const int64_t qrow_addr = int64_t(reinterpret_cast<uintptr_t>(a.q + out_row0));
  const int64_t kmask = (qrow_addr - int64_t(reinterpret_cast<uintptr_t>(a.k))) / kEsz;
  const int64_t vmask = (qrow_addr - int64_t(reinterpret_cast<uintptr_t>(a.v))) / kEsz;
  // The lane's first element of any row, as a byte address relative to a row start.
  const uint8_t* const kbase = reinterpret_cast<const uint8_t*>(a.k) + elem_d(col, 0) * kEsz;
  const uint8_t* const vbase = reinterpret_cast<const uint8_t*>(a.v) + elem_d(col, 0) * kEsz;

  // One thread per window slot finds its token's K and V rows. The loads the
  // start-up waits on are issued together: the sequence length and the
  // block-table entry of the slot's token. Without a sliding window the
  // entry is fetched before the length is known, for the stride of a
  // sequence that uses every planned split (the token index is clamped into
  // the mapped range, so the load needs no branch); a sequence with fewer
  // splits, or a window, fetches it again once the length is known.
  const int L_in = a.seq_lens[b];
  constexpr int kPer = (kWin + kThreads - 1) / kThreads;   // window slots per thread
  int e_tok[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    e_tok[r] = -1;
    if (a.window == 0) {
      const int t = min(strided_token(0, a.num_splits, s, min(tid + r * kThreads, kWin - 1)), planned_cap(a) - 1);
      e_tok[r] = table_entry(a, b, t);
    }
  }

  const SplitSpan sp = split_span_len(a, L_in, s, 1);
  flag_clamped(a, sp, s == 0 && g == 0 && tid == 0);
  if (sp.begin >= sp.L) {
    if (s == 0) {   // empty sequence: zeros (log-sum-exp -inf)
      for (int i = tid; i < G * D; i += kThreads) store_out(a, out_row0 + i, 0.0f);
      if (tid < G) store_lse(a, out_row0 / D + tid, 0.0f, 0.0f);
    }
    return;
  }
  bool bad_entry = false;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int slot = tid + r * kThreads;
    const int t_tok = strided_token(sp.lo, sp.nsplit, s, min(slot, kWin - 1));
    const bool live = slot < kWin && t_tok < sp.L;
    if ((a.window > 0 || sp.nsplit != a.num_splits) && live) e_tok[r] = table_entry(a, b, t_tok);
    int64_t ko = kmask, vo = vmask;
    const bool entry_ok = token_row_entry(a, e_tok[r], g, t_tok, ko, vo);
    if (slot < kWin) {
      const bool ok = live && entry_ok;
      tok_k[slot] = ok ? ko : kmask;
      tok_v[slot] = ok ? vo : vmask;
    }
    bad_entry |= live && !entry_ok;
  }
  if (a.err && __any(bad_entry) && lane == 0) atomicOr(a.err, 1u);
  __syncthreads();
  // q is loaded only now, with the first K rows (it is needed no earlier),
  // so the start-up above waits for nothing but the sequence length and the
  // block-table entries.
  // q of the group's G heads, in the lane's element order (elem_d).
  uint4 qv[G][kCq];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < kCq; ++k)
      qv[h][k] = *reinterpret_cast<const uint4*>(a.q + out_row0 + h * D + elem_d(col, 8 * k));

  // The split is one window of at most kSubSteps sub-steps of kStep tokens
  // (one strided block each); row `row` of wave `wave` owns window slots
  // j * kStep + my.
  const int my = wave * kRowsPerWave + row;
  const int n_sub = strided_blocks(sp, s) * (kBlockTokens / kStep);   // uniform, <= kSubSteps

  float acc[G][kEpl];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[h][e] = 0.0f;
  // Score of head (col / 2) for each sub-step's token (log2 units); the K
  // fetch sets it to +inf for a live token and -inf for a masked one.
  float sc[kSubSteps];
  float m_row = kMinit, l_row = 0.0f;

  uint4 ring[kRing][kCpl];
  // One lane's piece of a K or V row: kCpl 16-byte loads. Every K/V byte is
  // read once per call, so the loads are non-temporal (streaming cache policy).
  auto load_row = [&](const uint8_t* p, uint4 (&buf)[kCpl]) {
#pragma unroll
    for (int k = 0; k < kCpl; ++k) buf[k] = load_stream16(p + k * 256);
  };
  // K step j: the token's K row (branch-free: a masked token reads the q row).
  auto fetch_k = [&](int j, uint4 (&buf)[kCpl]) {
    const int64_t off = tok_k[j * kStep + my];
    sc[j] = off != kmask ? INFINITY : -INFINITY;
    load_row(kbase + off * kEsz, buf);
  };
  // V step j: the same token's V row.
  auto fetch_v = [&](int j, uint4 (&buf)[kCpl]) { load_row(vbase + tok_v[j * kStep + my] * kEsz, buf); };
  // q.k of the G heads; lanes 2h, 2h+1 keep head h's score.
  auto consume_k = [&](int j, const uint4 (&kk)[kCpl]) {
    float dq[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d0 = 0.0f;
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        d0 = dot2_bf16(qv[h][k].x, kk[k].x, d0);
        d0 = dot2_bf16(qv[h][k].y, kk[k].y, d0);
        d0 = dot2_bf16(qv[h][k].z, kk[k].z, d0);
        d0 = dot2_bf16(qv[h][k].w, kk[k].w, d0);
      }
      dq[h] = d0;
    }
    // sc[j] is +inf (live) or -inf (masked): the minimum keeps the score of a
    // live token and gives -inf for a masked one whatever its q-row score is.
    sc[j] = fminf(sc[j], reduce_scatter16<G>(dq, col) * a.scale_log2);
  };
  // p of head (col / 2), broadcast to the row, V accumulation.
  auto consume_v = [&](int j, const uint4 (&vv)[kCpl]) {
    const float pl = fast_exp2(sc[j] - m_row);
    l_row += pl;
    float p[G];
    head_bcast<G>(pl, p);
#pragma unroll
    for (int k = 0; k < kCpl; ++k) {
      const uint32_t w4[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float v0 = bf16_lo(w4[w]), v1 = bf16_hi(w4[w]);
        const int e = k * 8 + w * 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][e] = fmaf(p[h], v0, acc[h][e]);
          acc[h][e + 1] = fmaf(p[h], v1, acc[h][e + 1]);
        }
      }
    }
  };
  // One stream of 2 * kSubSteps steps (K pass, then V pass) through a ring of
  // kRing register buffers: kRing - 1 steps of loads stay in flight. Fully
  // unrolled, so every buffer lives in fixed registers. Loads are issued for
  // every step (a dead step only reads the q row); the arithmetic of steps
  // past n_sub is skipped with uniform branches.
  static_for<0, (kRing - 1 < kSteps ? kRing - 1 : kSteps)>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < kSubSteps) fetch_k(j, ring[j % kRing]);
    else fetch_v(j - kSubSteps, ring[j % kRing]);
  });
  static_for<0, kSteps>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int jn = j + kRing - 1;
    if constexpr (jn < kSteps) {
      if constexpr (jn < kSubSteps) fetch_k(jn, ring[jn % kRing]);
      else fetch_v(jn - kSubSteps, ring[jn % kRing]);
    }
    if ((j < kSubSteps ? j : j - kSubSteps) < n_sub) {
      if constexpr (j < kSubSteps) consume_k(j, ring[j % kRing]);
      else consume_v(j - kSubSteps, ring[j % kRing]);
    }
    if constexpr (j == kSubSteps - 1) {
      // Reference for the V pass: the max over the window scores of the
      // wave's 4 rows (same lane column, so the same head).
#pragma unroll
      for (int i = 0; i < kSubSteps; ++i) m_row = fmaxf(m_row, sc[i]);
      m_row = rows_max(m_row);
    }
  });

  // Every row already shares the wave's reference m_row: sum l over the
  // rows, and reduce-scatter the accumulators over the rows with lane swaps
  // (wave halves, then row pairs). Row r of lane column col ends with the
  // sums of elements e in [r * kEpl / 4, (r + 1) * kEpl / 4) of each head.
  // All of this runs before the barrier, while slower waves stream.
  constexpr int kE2 = kEpl / 2, kE4 = kEpl / 4;
  float m[G], l[G];
  head_bcast<G>(m_row, m);
  head_bcast<G>(rows_sum(l_row), l);
  float part[G][kE4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float half[kE2];
#pragma unroll
    for (int e = 0; e < kE2; ++e) {
      const Pair p = swap32(acc[h][e], acc[h][e + kE2]);
      half[e] = p.lo + p.hi;
    }
#pragma unroll
    for (int e = 0; e < kE4; ++e) {
      const Pair p = swap16(half[e], half[e + kE4]);
      part[h][e] = p.lo + p.hi;
    }
  }
  // Every wave publishes its sums with its reference max and its sum of
  // probabilities; one barrier; the final pass rescales each wave to the
  // workgroup max while it adds the waves (fixed order).
  {
    const int d0 = elem_d(col, row * kE4);     // kE4 contiguous elements
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = &mrg_acc[wave][h][d0];
      if constexpr (kE4 == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(part[h][0], part[h][1], part[h][2], part[h][3]);
      } else {
        *reinterpret_cast<float2*>(dst) = make_float2(part[h][0], part[h][1]);
      }
    }
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mrg_m[h][wave] = m[h];
        mrg_l[h][wave] = l[h];
      }
  }
  __syncthreads();

  // One thread per 4 consecutive outputs: vector LDS reads and one 16-byte
  // store each, every load issued up front.
  const int64_t prow0 = int64_t(b) * a.q_len * a.hq + int64_t(g) * G;   // partial row of head 0, query row 0
  for (int i4 = tid; i4 < G * D / 4; i4 += kThreads) {
    const int h = (4 * i4) / D, d = 4 * i4 - h * D;
    float mw[kWaves], lw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; w += 4) {
      const float4 x = *reinterpret_cast<const float4*>(&mrg_m[h][w]);
      const float4 y = *reinterpret_cast<const float4*>(&mrg_l[h][w]);
      mw[w] = x.x;
      mw[w + 1] = x.y;
      mw[w + 2] = x.z;
      mw[w + 3] = x.w;
      lw[w] = y.x;
      lw[w + 1] = y.y;
      lw[w + 2] = y.z;
      lw[w + 3] = y.w;
    }
    float4 acc4[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc4[w] = *reinterpret_cast<const float4*>(&mrg_acc[w][h][d]);
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
    float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(mw[w] - M);
      num.x = fmaf(f, acc4[w].x, num.x);
      num.y = fmaf(f, acc4[w].y, num.y);
      num.z = fmaf(f, acc4[w].z, num.z);
      num.w = fmaf(f, acc4[w].w, num.w);
      den = fmaf(f, lw[w], den);
    }
    if (sp.nsplit == 1) {
      const float4 o = den > 0.0f ? make_float4(num.x / den, num.y / den, num.z / den, num.w / den)
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      store_out4(a, out_row0 + 4 * i4, o);
    } else {
      const int64_t pr = (prow0 + h) * a.num_splits + s;
      if constexpr (WT) {
        // Written through to memory (agent-scope relaxed stores): the merge
        // kernel reads them from another XCD, and the kernel's end has no
        // dirty partial lines left to write back.
        uint64_t* const pa = reinterpret_cast<uint64_t*>(a.part_acc + pr * D + d);
        __hip_atomic_store(pa, __builtin_bit_cast(uint64_t, make_float2(num.x, num.y)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pa + 1, __builtin_bit_cast(uint64_t, make_float2(num.z, num.w)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(reinterpret_cast<uint64_t*>(a.part_ml + pr * 2),
                             __builtin_bit_cast(uint64_t, make_float2(M, den)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      } else {
        *reinterpret_cast<float4*>(a.part_acc + pr * D + d) = num;
        if (d == 0) *reinterpret_cast<float2*>(a.part_ml + pr * 2) = make_float2(M, den);
      }
    }
  }
  // A single-split sequence's optional log-sum-exp, one thread per head, from
  // the same (max, sum) pairs and in the same order as the loop above (kept
  // out of that loop, which every split runs).
  if (sp.nsplit == 1 && a.lse != nullptr && tid < G) {
    float M = mrg_m[tid][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg_m[tid][w]);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) den = fmaf(fast_exp2(mrg_m[tid][w] - M), mrg_l[tid][w], den);
    store_lse(a, out_row0 / D + tid, M, den);
  }
}

template <int D, int G, int NS, int RING, bool WT>
hipError_t launch_decode_k(const DecodeArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  dim3 grid(a.num_splits, a.hkv, a.num_seqs);
  if (e0 && e1)
    hipExtLaunchKernelGGL((decode_split_kernel<D, G, NS, RING, WT>), grid, dim3(kThreads), 0, st, e0, e1, 0,
                          a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, G, NS, RING, WT>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, int NS, int RING, bool WT>
hipError_t launch_decode_d(const DecodeArgs& a, int group, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (group) {
    case 1: return launch_decode_k<D, 1, NS, RING, WT>(a, st, e0, e1);
    case 2: return launch_decode_k<D, 2, NS, RING, WT>(a, st, e0, e1);
    case 3: return launch_decode_k<D, 3, NS, RING, WT>(a, st, e0, e1);
    case 4: return launch_decode_k<D, 4, NS, RING, WT>(a, st, e0, e1);
    case 5: return launch_decode_k<D, 5, NS, RING, WT>(a, st, e0, e1);
    case 6: return launch_decode_k<D, 6, NS, RING, WT>(a, st, e0, e1);
    case 7: return launch_decode_k<D, 7, NS, RING, WT>(a, st, e0, e1);
    case 8: return launch_decode_k<D, 8, NS, RING, WT>(a, st, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

// Launch the split kernel with a window of NS strided blocks of 32 tokens
// (a.chunk <= NS * 32) for bf16 caches, with a register ring of RING steps;
// WT: partials written through to memory.
template <int NS, int RING = kRingOne, bool WT = false>
hipError_t launch_decode_window(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                                hipEvent_t e1) {
  if (a.chunk > NS * kBlockTokens || a.kv_fp8) return hipErrorInvalidValue;
  if (head_dim == 256) return launch_decode_d<256, NS, RING, WT>(a, group, st, e0, e1);
  if (head_dim == 128) return launch_decode_d<128, NS, RING, WT>(a, group, st, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pkv
