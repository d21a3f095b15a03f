// Multi-row (speculative verify) paged attention for gfx950: up to 16 new
// query rows per sequence (the same count for every sequence, or per sequence
// through cu_seqlens_q), each with its own causal bound, sharing one
// walk over the paged K/V. This is the case where q.k and p.v become small
// dense contractions, so they run on MFMA.
//
// Following "Qwen3.8 auf MI350P betreiben", Lektion 3: every K/V tile is
// reused by all verify rows of the request (here the G * q_len rows of one KV
// head, at most 128), each row applies its own causal mask, and partial
// softmax statistics are merged (by the LSE merge kernel across splits).
// Addresses follow "DCU page832 attention" §1/§5 as in the decode kernel.
//
// Workgroup = one split (<= 512 tokens) of one (sequence, KV head), 8 waves.
//   * All 8 waves stage 64-token K and V tiles into LDS (double buffered, rows
//     padded to 544 bytes for D = 256) with 16-byte loads through the block table; FP8
//     caches are decoded to bf16 (exactly) on the way into LDS.
//   * Wave w owns query rows f = 16w .. 16w + 15 of the flattened
//     (head, position) list, head-major (f = h_local * q_len + i); waves past
//     the last row only stage tiles.
//   * S^T = K Q^T per 16-token block with v_mfma_f32_16x16x32_bf16 (A = K rows
//     from LDS, B = the wave's Q rows held in registers). Its accumulator
//     layout (lane l: tokens 4(l/16)..+3 of row l%16) is exactly the A-operand
//     layout of P for O = P V, so P never leaves registers.
//   * Online softmax per row with the exact tile max (log2 units); rows are
//     reduced across the four 16-lane groups with two lane swaps
//     (v_permlane32_swap, v_permlane16_swap), no LDS round trip.
//   * P is split into bf16 hi + lo (hi = bf16(p), lo = bf16(p - hi)), two MFMAs
//     per block, so the bf16 operand costs about 2^-16 relative error instead of
//     2^-9. V enters as the B operand through ds_read_b64_tr_b16: lane j of a
//     16-lane group points at V[4q + j/4][d0 + 4(j%4)] and lane i receives the
//     column V[4q..4q+3][d0 + i].
//   * O (16 rows x D) stays in MFMA accumulators; the split writes it
//     un-normalised with the row's (max, sum), or normalised when the
//     sequence has a single split.
#include <hip/hip_ext.h>

#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kVWaves = 8;
constexpr int kVThreads = 64 * kVWaves;
constexpr int kVTile = 64;      // tokens per K/V tile
constexpr int kRowsPerWave = 16;
constexpr float kMinitV = -1.0e30f;   // floor of a row's running max (finite: no inf - inf)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t* lds_short4_ptr;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two floats as a packed bf16 pair (one v_cvt_pk_bf16_f32); x in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){x, y}, bf16x2_t));
}

// A row's softmax reference moves only when a tile's max exceeds it by more
// than this (log2 units), so probabilities stay <= 2^8 and most tiles need no
// rescale of O.
constexpr float kLazyMax = 8.0f;

// Stand-in K/V rows (up to 512 bytes) for tokens a tile must not count (past
// its range, or behind an invalid table entry): keys are NaN (bf16 NaN pairs;
// FP8 E4M3FN NaN codes), so such a token's score is NaN and the score filter
// drops it, and values are zero, so nothing reaches O.
struct StandInRows {
  uint32_t nan_key[2][128];   // [bf16, FP8]
  uint32_t zero[128];
};
constexpr StandInRows make_stand_in_rows() {
  StandInRows r{};
  for (int i = 0; i < 128; ++i) {
    r.nan_key[0][i] = 0x7fc07fc0u;
    r.nan_key[1][i] = 0x7f7f7f7fu;
    r.zero[i] = 0u;
  }
  return r;
}
__device__ __attribute__((aligned(16))) const StandInRows kStandIn = make_stand_in_rows();
constexpr uint32_t kNanBf16Pair = 0x7fc07fc0u;

// Padding of an LDS token row: for D = 256, 32 bytes shift consecutive rows
// by 8 banks, which suits the transposed V reads (4 lanes x 8 bytes per row)
// better than 16 (measured: about 5% on prefill blocks, neutral on verify).
// D = 128 keeps 16 so that two workgroups still fit in one CU's LDS.
template <int D>
constexpr int kRowPad = D >= 256 ? 32 : 16;

// PF (prefill): the workgroup is a block of a.pf_rows query positions of one
// (sequence, KV head) stream instead of a KV split, and covers its whole
// visible range in one pass. The 1-D grid lists blocks largest first (the
// last positions see the most tokens), each rank interleaved over all
// streams: with workgroups dealt round-robin to the 8 XCDs, the blocks of one
// stream stay on the same XCDs (shared L2) when the stream count divides 8
// or 8 divides it, and every XCD gets a balanced share. Token offsets come
// from the block table in global memory, one lane per token, staged in LDS
// two tiles ahead (the range can exceed what the LDS table holds).
template <int D, bool FP8, bool PF, bool WT>
__global__ __launch_bounds__(kVThreads, 1) void verify_split_kernel(DecodeArgs a) {
  constexpr int kPitch = D * 2 + kRowPad<D>;         // LDS bytes per token row (padded)
  constexpr int kElems = FP8 ? 16 : 8;            // elements per 16-byte chunk of a cache row
  constexpr int kChunks = D / kElems;             // 16-byte chunks per row
  constexpr int kLoads = kVTile * kChunks / kVThreads;   // K (and V) chunks per thread per tile
  constexpr int kKSteps = D / 32;                 // 32-wide k steps of q.k
  constexpr int kDBlocks = D / 16;                // 16-column blocks of O
  static_assert(kLoads >= 1 && kVTile * kChunks % kVThreads == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint8_t kv[2][2][kVTile * kPitch];
  __shared__ PageOffs tbl[PF ? 1 : kMaxChunk + 2];   // PF reads the table from global memory
  // K and V byte offsets of a tile's tokens, a ring of 3 tiles (the one being
  // loaded, the next one, and the one being staged).
  __shared__ __attribute__((aligned(16))) int64_t toff[3][kVTile][2];

  int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int p0 = 0;                                     // PF: first query position of the block
  bool lead = s == 0;                             // reports inconsistent rows of the stream
  if constexpr (PF) {
    const int streams = a.hkv * a.num_seqs;
    const int rank = int(blockIdx.x) / streams, stream = int(blockIdx.x) - rank * streams;
    const int nblk = (a.q_len + a.pf_rows - 1) / a.pf_rows;
    g = stream % a.hkv;
    b = stream / a.hkv;
    s = 0;
    p0 = (nblk - 1 - rank) * a.pf_rows;
    lead = rank == 0;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, ln = lane & 15;
  const QRows qr = seq_q_rows(a, b);
  const int q_len = PF ? min(a.pf_rows, qr.n - p0) : qr.n;   // query rows of this workgroup
  const int row_base = qr.base + p0;
  const int G = a.hq / a.hkv;
  const int R = G * q_len;                        // rows of this KV head (<= 128)
  if (q_len <= 0) {                               // no rows, or inconsistent cu_seqlens_q
    if (!qr.ok && lead && g == 0 && tid == 0 && a.err) atomicOr(a.err, 2u);
    return;
  }
  SplitPages pages{0, 0};
  SplitSpan sp;
  if constexpr (PF) {
    sp = prefill_span(a, b, qr.n, p0, q_len);
  } else {
    // The table slots do not depend on the sequence length: fetch them while
    // seq_lens is still in flight.
    pages = split_pages(a, s);
    if (a.window == 0) stage_table(a, b, g, pages.p_first, pages.n, tbl);
    sp = split_span(a, b, s, q_len);
  }
  flag_clamped(a, sp, lead && g == 0 && tid == 0);

  if (sp.begin >= sp.L) {
    if (s == 0)   // empty sequence: zeros (log-sum-exp -inf) for every row of this KV head
      for (int i = tid; i < R * D; i += kVThreads) {
        const int f = i / D, d = i - f * D;
        const int64_t prow = (int64_t(row_base) + f % q_len) * a.hq + int64_t(g) * G + f / q_len;
        store_out(a, prow * D + d, 0.0f);
        if (d == 0) store_lse(a, prow, 0.0f, 0.0f);
      }
    return;
  }
  if (!PF && a.window > 0) {   // the split starts at the first token of the rows' windows
    pages = span_pages(a, sp);
    stage_table(a, b, g, pages.p_first, pages.n, tbl);
  }
  const int p_first = pages.p_first;

  // This lane's S^T row (row ln of the wave's block).
  const bool computes = wave * kRowsPerWave < R;  // uniform per wave
  const int f_row = wave * kRowsPerWave + ln;
  const bool row_valid = f_row < R;
  const int h_row = row_valid ? f_row / q_len : 0;
  const int i_row = row_valid ? f_row % q_len : 0;
  const int pos_row = sp.L - q_len + i_row;      // last visible token of the row

  // Q of row ln, as the B operand of S^T: k step kk holds d = 32 kk + 8 grp .. +8.
  // Padding rows hold NaN, so all their scores fail the score filter.
  uint4 qreg[kKSteps];
  {
    const int64_t qoff = ((int64_t(row_base) + i_row) * a.hq + int64_t(g) * G + h_row) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
      qreg[kk] = (computes && row_valid) ? *reinterpret_cast<const uint4*>(a.q + qoff + 32 * kk)
                                         : make_uint4(kNanBf16Pair, kNanBf16Pair, kNanBf16Pair, kNanBf16Pair);
  }
  __syncthreads();   // table staged
  if constexpr (!PF) flag_invalid_entries(a, tbl, int(magic_div(uint32_t(sp.end - 1), a.bdiv)) - p_first + 1);

  float4_t o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) o[db] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kMinitV, l_run = 0.0f;            // stats of row ln

  // Tile staging: thread tid moves chunks c = tid + kVThreads * k of K and V.
  u32x4_t stk[kLoads], stv[kLoads];   // native vectors: kept in registers
  auto load_tile = [&](int tile) __attribute__((always_inline)) {
    static_for<0, kLoads>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const int c = tid + kVThreads * k;
      const int tt = c / kChunks, piece = c - tt * kChunks;
      // Staged byte offsets (stand-in rows for tokens that must not count).
      const int64_t* to = toff[tile % 3][tt];
      stk[k] = *(reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(a.k) + to[0]) + piece);
      stv[k] = *(reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(a.v) + to[1]) + piece);
    });
  };
  // FP8: 16 codes -> 16 exact bf16 values (32 bytes).
  auto fp8_to_bf16 = [&](const u32x4_t& x, u32x4_t& lo, u32x4_t& hi) __attribute__((always_inline)) {
    lo = u32x4_t{fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
                 fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
    hi = u32x4_t{fp8x2_to_bf16x2<false>(x[2]), fp8x2_to_bf16x2<true>(x[2]),
                 fp8x2_to_bf16x2<false>(x[3]), fp8x2_to_bf16x2<true>(x[3])};
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    static_for<0, kLoads>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const int c = tid + kVThreads * k;
      const int tt = c / kChunks, piece = c - tt * kChunks;
      if constexpr (FP8) {
        u32x4_t lo, hi;
        fp8_to_bf16(stk[k], lo, hi);
        *reinterpret_cast<u32x4_t*>(&kv[buf][0][tt * kPitch + piece * 32]) = lo;
        *reinterpret_cast<u32x4_t*>(&kv[buf][0][tt * kPitch + piece * 32 + 16]) = hi;
        fp8_to_bf16(stv[k], lo, hi);
        *reinterpret_cast<u32x4_t*>(&kv[buf][1][tt * kPitch + piece * 32]) = lo;
        *reinterpret_cast<u32x4_t*>(&kv[buf][1][tt * kPitch + piece * 32 + 16]) = hi;
      } else {
        *reinterpret_cast<u32x4_t*>(&kv[buf][0][tt * kPitch + piece * 16]) = stk[k];
        *reinterpret_cast<u32x4_t*>(&kv[buf][1][tt * kPitch + piece * 16]) = stv[k];
      }
    });
  };

  // Token offsets, one lane per token: lane `tid` (wave 0) stages token tid
  // of a tile two tiles ahead. PF reads the block table from global memory:
  // the entry is fetched early and the offsets written after the tile's
  // compute, so its wait on the entry does not also wait on that tile's K/V
  // loads. Otherwise the entry comes from the LDS table.
  int pf_entry = 0;
  bool pf_bad = false;                            // an entry outside [0, num_pages) was met
  auto fetch_entry = [&](int tile) __attribute__((always_inline)) {
    if constexpr (PF) {
      const int t = sp.begin + tile * kVTile + tid;
      if (tid < kVTile && t < sp.end)
        pf_entry = a.table[int64_t(b) * a.max_pages + magic_div(uint32_t(t), a.bdiv)];
    }
  };
  auto commit_offsets = [&](int tile) __attribute__((always_inline)) {
    if (tid < kVTile) {
      constexpr int kEb = FP8 ? 1 : 2;   // bytes per element
      const int t = sp.begin + tile * kVTile + tid;
      // Byte offsets from a.k / a.v; tokens that must not count point at
      // the stand-in rows.
      int64_t ko = int64_t(reinterpret_cast<uintptr_t>(kStandIn.nan_key[FP8 ? 1 : 0]) -
                           reinterpret_cast<uintptr_t>(a.k));
      int64_t vo = int64_t(reinterpret_cast<uintptr_t>(kStandIn.zero) - reinterpret_cast<uintptr_t>(a.v));
      if (t < sp.end) {
        if constexpr (PF) {
          const int off = t - int(magic_div(uint32_t(t), a.bdiv) * a.bdiv.d);
          if (uint32_t(pf_entry) < uint32_t(a.num_pages)) {
            ko = (int64_t(pf_entry) * a.k_sp + int64_t(g) * a.k_sh + int64_t(off * int32_t(a.k_st))) * kEb;
            vo = (int64_t(pf_entry) * a.v_sp + int64_t(g) * a.v_sh + int64_t(off * int32_t(a.v_st))) * kEb;
          } else {
            pf_bad = true;
          }
        } else {
          int64_t ke, ve;
          if (token_row(a, tbl, p_first, t, ke, ve)) {
            ko = ke * kEb;
            vo = ve * kEb;
          }
        }
      }
      toff[tile % 3][tid][0] = ko;
      toff[tile % 3][tid][1] = vo;
    }
  };

  const int n_tiles = (sp.end - sp.begin + kVTile - 1) / kVTile;
  fetch_entry(0);
  commit_offsets(0);
  fetch_entry(1);
  commit_offsets(1);
  __syncthreads();
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < n_tiles;
    fetch_entry(tile + 2);
    if (more) load_tile(tile + 1);
    if (computes) {
      const uint8_t* kb = kv[buf][0];
      // S^T for the 4 token blocks: st[tb][r] = score of token tb*16 + 4 grp + r, row ln.
      float4_t st[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        st[tb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const uint4 kr = *reinterpret_cast<const uint4*>(kb + (tb * 16 + ln) * kPitch + (32 * kk + 8 * grp) * 2);
          st[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr), as_bf16x8(qreg[kk]), st[tb], 0, 0, 0);
        }
      }
      // Scale, causal / window mask, tile max of row ln. Tokens past the
      // split or behind an invalid table entry were staged with NaN keys:
      // their scores are NaN and fail the s == s test.
      // Token (tile start + 4 grp + c) is visible to the row when c <= dist
      // and c > wdist (dist clamped at -1: nothing visible; a window of 2^30
      // or more covers every position).
      const int dist = max(pos_row - (sp.begin + tile * kVTile + 4 * grp), -1);
      const int wdist = (a.window > 0 && a.window < (1 << 30)) ? dist - a.window : -(1 << 30) - 2;
      float mt = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = tb * 16 + r;
          const float sc = st[tb][r];
          const bool vis = sc == sc && c <= dist && c > wdist;
          const float x = vis ? sc * a.scale_log2 : -INFINITY;
          st[tb][r] = x;
          mt = fmaxf(mt, x);
        }
      mt = rows_max(mt);   // the 4 lane groups hold the same row's tokens: lane swaps, no LDS
      const float m_new = mt > m_run + kLazyMax ? mt : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      float ls = 0.0f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(st[tb][r] - m_new);
          st[tb][r] = p;
          ls += p;
        }
      ls = rows_sum(ls);
      const bool moved = m_new != m_run;
      l_run = l_run * alpha + ls;
      m_run = m_new;
      // O rows 4 grp + r take the alpha of that row (held by lane 4 grp + r of
      // the group); skipped when no row of the wave moved its reference.
      if (__any(moved ? 1 : 0)) {
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 16 * grp + 4 * grp + r);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[db][r] *= al[r];
      }
      // P as A operands (hi and lo) of the two 32-token halves.
      static_for<0, 2>([&](auto hc) {
        constexpr int hh = decltype(hc)::value;
        uint32_t hi[4], lo[4];
        static_for<0, 4>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const float p0 = st[2 * hh + (t >> 1)][(t & 1) * 2];
          const float p1 = st[2 * hh + (t >> 1)][(t & 1) * 2 + 1];
          const uint32_t h = bf16_pair(p0, p1);
          hi[t] = h;
          lo[t] = bf16_pair(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
        });
        const bf16x8_t ph = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8_t pl = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        // V (32 tokens x 16 columns) per column block: two transposed reads.
        const int rowa = (2 * hh) * 16 + 4 * grp + (ln >> 2);
        const int rowb = rowa + 16;
        static_for<0, kDBlocks>([&](auto dc) {
          constexpr int db = decltype(dc)::value;
          const int colb = (16 * db + 4 * (ln & 3)) * 2;
          const short4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_short4_ptr)(kv[buf][1] + rowa * kPitch + colb));
          const short4_t vb2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_short4_ptr)(kv[buf][1] + rowb * kPitch + colb));
          const uint4 vu = make_uint4(uint32_t(uint16_t(va[0])) | (uint32_t(uint16_t(va[1])) << 16),
                                      uint32_t(uint16_t(va[2])) | (uint32_t(uint16_t(va[3])) << 16),
                                      uint32_t(uint16_t(vb2[0])) | (uint32_t(uint16_t(vb2[1])) << 16),
                                      uint32_t(uint16_t(vb2[2])) | (uint32_t(uint16_t(vb2[3])) << 16));
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, as_bf16x8(vu), o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, as_bf16x8(vu), o[db], 0, 0, 0);
        });
      });
    }
    if (more) store_tile(buf ^ 1);
    commit_offsets(tile + 2);   // slot (tile + 2) % 3 was last read in the previous iteration
    __syncthreads();
  }
  if (PF && pf_bad && a.err) atomicOr(a.err, 1u);

  if (!computes) return;
  // Rows 4 grp + r of O; their (max, sum) are held by lane 4 grp + r of each group.
  const int64_t prow_base = int64_t(row_base) * a.hq + int64_t(g) * G;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int src = 16 * grp + 4 * grp + r;
    const float lr = __shfl(l_run, src);
    const float mr = __shfl(m_run, src);
    const int f = wave * kRowsPerWave + 4 * grp + r;
    if (f >= R) continue;
    const int h = f / q_len, i = f % q_len;
    const int64_t prow = prow_base + int64_t(i) * a.hq + h;
    if (sp.nsplit == 1) {
      const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) store_out(a, prow * D + 16 * db + ln, o[db][r] * inv);
      if (ln == 0) store_lse(a, prow, mr, lr);
    } else {
      const int64_t pr = prow * a.num_splits + s;
      if constexpr (WT) {   // written through to memory (agent-scope relaxed stores)
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
          __hip_atomic_store(a.part_acc + pr * D + 16 * db + ln, o[db][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (ln == 0)
          __hip_atomic_store(reinterpret_cast<uint64_t*>(a.part_ml + pr * 2),
                             __builtin_bit_cast(uint64_t, make_float2(mr, lr)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      } else {
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) a.part_acc[pr * D + 16 * db + ln] = o[db][r];
        if (ln == 0) {
          a.part_ml[pr * 2] = mr;
          a.part_ml[pr * 2 + 1] = lr;
        }
      }
    }
  }
}

template <int D, bool FP8, bool PF, bool WT>
hipError_t launch_verify_k(const DecodeArgs& a, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (e0 && e1)
    hipExtLaunchKernelGGL((verify_split_kernel<D, FP8, PF, WT>), grid, dim3(kVThreads), 0, st, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((verify_split_kernel<D, FP8, PF, WT>), grid, dim3(kVThreads), 0, st, a);
  return hipGetLastError();
}

template <bool PF>
hipError_t launch_verify_any(const DecodeArgs& a, int head_dim, dim3 grid, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1) {
  // Split grids of at most one workgroup per CU (head_dim 256) write their
  // partials through to memory: the whole grid ends at once and the merge
  // reads them next. Larger grids keep ordinary stores.
  if (head_dim == 256) {
    if (!PF && !a.many_wg)
      return a.kv_fp8 ? launch_verify_k<256, true, false, true>(a, grid, st, e0, e1)
                      : launch_verify_k<256, false, false, true>(a, grid, st, e0, e1);
    return a.kv_fp8 ? launch_verify_k<256, true, PF, false>(a, grid, st, e0, e1)
                    : launch_verify_k<256, false, PF, false>(a, grid, st, e0, e1);
  }
  return a.kv_fp8 ? launch_verify_k<128, true, PF, false>(a, grid, st, e0, e1)
                  : launch_verify_k<128, false, PF, false>(a, grid, st, e0, e1);
}

}  // namespace

bool verify_supported(int head_dim, int group, int q_len) {
  return (head_dim == 128 || head_dim == 256) && group >= 1 && q_len >= 1 && q_len <= 16 &&
         group * q_len <= kVWaves * kRowsPerWave;
}

hipError_t launch_verify_split(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
  if (!verify_supported(head_dim, group, a.q_len)) return hipErrorInvalidValue;
  dim3 grid(a.num_splits, a.hkv, a.num_seqs);
  return launch_verify_any<false>(a, head_dim, grid, st, e0, e1);
}

hipError_t launch_prefill(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                          hipEvent_t e1) {
  // A block holds pf_rows positions of all `group` heads: at most 128 MFMA rows.
  if ((head_dim != 128 && head_dim != 256) || group < 1 || a.pf_rows < 1 ||
      group * a.pf_rows > kVWaves * kRowsPerWave)
    return hipErrorInvalidValue;
  const int64_t blocks = int64_t((a.q_len + a.pf_rows - 1) / a.pf_rows) * a.hkv * a.num_seqs;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(uint32_t(blocks), 1, 1);
  return launch_verify_any<true>(a, head_dim, grid, st, e0, e1);
}

}  // namespace pkv
