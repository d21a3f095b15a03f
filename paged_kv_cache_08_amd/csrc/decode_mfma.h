// The single-query split kernel on MFMA, for gfx950 (wave64, CDNA4): the same
// computation and work split as decode_split_kernel (decode_split.h), with
// q.k and p.v as small dense contractions on v_mfma_f32_16x16x32_bf16 instead
// of VALU dot products. It serves FP8 E4M3 caches, where the VALU kernel is
// bound by its arithmetic (each code is widened, then multiplied into every
// query head of the group) rather than by the bytes it reads; MFMA takes the
// products, and the VALU is left with the code conversion (exact: every E4M3
// value is a bf16 value) and the softmax.
//
// What is computed follows "DCU page832 attention" (luanjiahao.me): §1 and §5
// for the address of a token row (logical page = t / B, offset t % B,
// physical page from the block table, then page / token / head strides) and
// §5 for score = dot(q, k) * scale with a softmax-weighted sum of V. The
// 8-bit cache is the quantised-KV variant of the RTX 3090 page (coreui.cn):
// codes times one scale per tensor (the K scale is folded into the score
// scale, the V scale into the output). Splits are those of the split-KV
// paragraph of "vLLM 下双卡 Radeon 上的混合 SSM 解码速率", dealt out in strided
// 32-token blocks exactly as in the VALU kernel (strided_token()).
//
// Work mapping (one workgroup = one split of one (sequence, KV head), 4 waves,
// one per SIMD):
//   * Wave w takes the split's strided blocks w, w + 4, w + 8, ... (32 tokens
//     each). All K and V loads of the wave go through a register ring and are
//     issued ahead of their use; the wave never waits at a barrier before the
//     epilogue.
//   * K and V rows are loaded whole: 16 lanes read one row's 16-byte chunks
//     with one instruction (A/B: loads of 16 rows x 64 bytes per instruction,
//     read straight into the MFMA layout, were slower: 32K 20.6 against 19.6
//     us, 16-sequence mixed batch 48.3 against 43.9 us).
//   * The G query heads of the group are the rows of a 16-row MFMA tile (rows
//     past G carry no weight). S^T = K Q^T per 16 tokens: the A operand is K
//     (lane l: token l % 16, 8 head-dim elements of k slot l / 16), read back
//     from the wave's LDS tile; B is Q (lane l: head l % 16), held in
//     registers. Since q.k sums over the head dim, the order in which head-dim
//     elements meet the k slots only has to agree between K and Q: lane
//     group g takes 16-byte chunks g, g + 4, g + 8, ... of a row.
//   * The accumulator of S^T (lane l: head l % 16, tokens 4 (l / 16) .. + 3)
//     is the A-operand layout of P for O = P V (k slot l / 16 = tokens
//     4 (l / 16) .. + 3 and 16 + 4 (l / 16) .. + 3 of the block), so P never
//     leaves registers. It is split into bf16 hi + lo parts (two MFMAs per
//     column block), so the bf16 operand costs about 2^-16 relative error.
//   * The wave writes each block's K rows, later its V rows, to a private LDS
//     tile (rows padded by 16 bytes). K comes back as 16-byte A operands. V
//     needs the token index along k: it comes back transposed,
//     ds_read_b64_tr_b8 for codes (lane i of a 16-lane group gets column i of
//     the 8 rows its group points at) or ds_read_b64_tr_b16 for bf16 (4 rows
//     per read, two reads).
//   * Exact softmax per wave: a K pass over all the wave's blocks keeps every
//     score (log2 units), the wave's maximum is taken once, and the V pass
//     uses it, so O is never rescaled. Masked tokens (past the split, or
//     behind an invalid table entry) read stand-in rows: NaN keys, whose
//     scores fail the s == s test, and zero values.
//   * Epilogue as in the VALU kernel: each wave publishes O of its G heads
//     with its (max, sum) in LDS; after one barrier the workgroup rescales
//     the waves to a common max and adds them in a fixed order, and writes the
//     split's partial (max, sum, accumulator), or the normalised output when
//     the sequence has a single split.
//   * MR (several query rows per sequence; "Qwen3.8 auf MI350P betreiben",
//     Lektion 3: one K/V walk for all verify rows, each with its own causal
//     bound): up to 32 rows per KV head (G heads x n rows, head-major: row f
//     is head f / n at position f % n) in two 16-row tiles that share every
//     K and V operand read. A score counts only when its token is at most the
//     row's position L - n + i (and within the row's window); the epilogue
//     merges the waves one tile at a time. bf16 and FP8 caches, head_dim 256.
// Every reduction order depends only on logical token indices and the split
// plan, never on block_size or physical page ids.
#pragma once

#include <math.h>

#include <hip/hip_ext.h>

#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kMMaxG = 8;                 // query heads per KV head (rows of the 16-row tile used)
constexpr float kMMinit = -1.0e30f;       // floor of a row's max (finite: no inf - inf)

typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef float mfloat4_t __attribute__((ext_vector_type(4)));
typedef float mfloat2_t __attribute__((ext_vector_type(2)));
typedef __bf16 mbf16x2_t __attribute__((ext_vector_type(2)));
typedef short mshort4_t __attribute__((ext_vector_type(4)));
typedef int mint2_t __attribute__((ext_vector_type(2)));
typedef uint32_t mu32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mshort4_t* lds_mshort4_ptr;
typedef __attribute__((address_space(3))) mint2_t* lds_mint2_ptr;

__device__ __forceinline__ mbf16x8_t m_as_bf16x8(const uint4& u) { return __builtin_bit_cast(mbf16x8_t, u); }

// Two floats as a packed bf16 pair (round to nearest even); x in the low half.
__device__ __forceinline__ uint32_t m_bf16_pair(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mfloat2_t){x, y}, mbf16x2_t));
}

// Stand-in rows (512 bytes each, enough for any row of D <= 256) for tokens
// that must not count: keys whose every element is NaN (bf16 0x7fc0; E4M3
// code 0x7f), and zero values.
struct MStandIn {
  uint32_t nan_bf16[128];
  uint32_t nan_fp8[128];
  uint32_t zero[128];
};
constexpr MStandIn make_m_stand_in() {
  MStandIn r{};
  for (int i = 0; i < 128; ++i) {
    r.nan_bf16[i] = 0x7fc07fc0u;
    r.nan_fp8[i] = 0x7f7f7f7fu;
    r.zero[i] = 0u;
  }
  return r;
}
__device__ __attribute__((aligned(16))) const MStandIn kMStandIn = make_m_stand_in();

// 16 bytes read with a non-temporal load (each K/V byte is read once per call).
__device__ __forceinline__ uint4 m_load16(const uint8_t* p) {
  const mu32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const mu32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Eight E4M3 codes (two words, low byte first) as eight exact bf16 values.
__device__ __forceinline__ uint4 m_fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                    fp8x2_to_bf16x2<true>(w1));
}

// MR: several query rows per sequence (uniform q_len or varlen rows), at
// most 32 rows (G x rows) per KV head in two 16-row tiles; each row keeps its
// own causal (and window) bound.
template <int D, int NBLK, bool FP8, int WAVES, int RING, bool MR = false>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int kMWaves = WAVES;
  constexpr int kMThreads = 64 * WAVES;
  constexpr int kEsz = FP8 ? 1 : 2;             // bytes per cache element
  constexpr int kRowB = D * kEsz;               // bytes per K or V row
  constexpr int kChunks = kRowB / 16;           // 16-byte chunks per row
  constexpr int kKLd = kChunks / 4;             // 16-byte K chunks per lane per 16 tokens
  constexpr int kStepLd = kChunks / 2;          // loads per lane per step (32 tokens of K, or of V)
  constexpr int kKSteps = D / 32;               // k steps of one S^T tile
  constexpr int kDBlocks = D / 16;              // 16-column blocks of O
  constexpr int kPitch = kRowB + 16;            // LDS bytes per V row of the transpose tile
  constexpr int kWin = NBLK * kBlockTokens;     // tokens of the split's window
  constexpr int kBpw = (NBLK + kMWaves - 1) / kMWaves;   // blocks per wave
  constexpr int kSteps = 2 * kBpw;              // K steps, then V steps
  constexpr int kRing = kSteps < RING ? kSteps : RING;   // ring depth: steps in flight + 1
  constexpr int kNT = MR ? 2 : 1;               // 16-row MFMA tiles
  constexpr int kMrgRows = MR ? 16 : kMMaxG;    // rows merged across the waves at a time
  static_assert(kChunks % 4 == 0 && kStepLd * 64 * 16 == kBlockTokens * kRowB, "rows split evenly");
  static_assert(kWin <= kMaxChunk, "window of at most kMaxChunk tokens");

  __shared__ int64_t tok_k[kWin];   // element offset of each window token's K row (masked: the NaN row)
  __shared__ int64_t tok_v[kWin];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kMWaves][kBlockTokens * kPitch];
  __shared__ __attribute__((aligned(16))) float mrg_acc[kMWaves][kMrgRows][D];
  __shared__ __attribute__((aligned(16))) float mrg_m[kMrgRows][kMWaves];
  __shared__ __attribute__((aligned(16))) float mrg_l[kMrgRows][kMWaves];
  static_assert(kMWaves % 4 == 0, "whole float4 rows of (max, sum)");

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, ln = lane & 15;
  const int G = a.hq / a.hkv;
  const int64_t out_row0 = (int64_t(b) * a.hq + int64_t(g) * G) * D;   // q_len == 1

  // Stand-in rows as element offsets from the cache bases (all 16-byte aligned).
  const int64_t kstand =
      (int64_t(reinterpret_cast<uintptr_t>(FP8 ? kMStandIn.nan_fp8 : kMStandIn.nan_bf16)) -
       int64_t(reinterpret_cast<uintptr_t>(a.k))) / kEsz;
  const int64_t vstand =
      (int64_t(reinterpret_cast<uintptr_t>(kMStandIn.zero)) - int64_t(reinterpret_cast<uintptr_t>(a.v))) / kEsz;

  // Token offsets, one thread per window slot, exactly as in the VALU kernel:
  // the sequence length and the slot's table entry are loaded together
  // (without a sliding window the entry is fetched for the stride of a
  // sequence that uses every planned split, clamped into the mapped range).
  const int L_in = a.seq_lens[b];
  constexpr int kPer = (kWin + kMThreads - 1) / kMThreads;
  int e_tok[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    e_tok[r] = -1;
    if (a.window == 0) {
      const int t = min(strided_token(0, a.num_splits, s, min(tid + r * kMThreads, kWin - 1)), planned_cap(a) - 1);
      e_tok[r] = table_entry(a, b, t);
    }
  }
  // MR: the sequence's query rows [row_base, row_base + n_rows); row f of the
  // KV head is head f / n_rows at position f % n_rows. (Read after the loads
  // above are issued: they do not depend on the rows.)
  int n_rows = 1, row_base = b;
  if constexpr (MR) {
    const QRows qr = seq_q_rows(a, b);
    if (qr.n <= 0) {   // no rows, or inconsistent cu_seqlens_q
      if (!qr.ok && s == 0 && g == 0 && tid == 0 && a.err) atomicOr(a.err, 2u);
      return;
    }
    n_rows = qr.n;
    row_base = qr.base;
  }
  const int R = G * n_rows;   // rows of this KV head
  auto prow_of = [&](int f) {
    return (int64_t(row_base) + f % n_rows) * a.hq + int64_t(g) * G + f / n_rows;
  };
  const SplitSpan sp = split_span_len(a, L_in, s, n_rows);
  flag_clamped(a, sp, s == 0 && g == 0 && tid == 0);
  if (sp.begin >= sp.L) {
    if (s == 0) {   // empty sequence: zeros (log-sum-exp -inf)
      if constexpr (MR) {
        for (int i = tid; i < R * D; i += kMThreads) {
          const int f = i / D, d = i - f * D;
          store_out(a, prow_of(f) * D + d, 0.0f);
          if (d == 0) store_lse(a, prow_of(f), 0.0f, 0.0f);
        }
      } else {
        for (int i = tid; i < G * D; i += kMThreads) store_out(a, out_row0 + i, 0.0f);
        if (tid < G) store_lse(a, out_row0 / D + tid, 0.0f, 0.0f);
      }
    }
    return;
  }
  bool bad_entry = false;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int slot = tid + r * kMThreads;
    const int t_tok = strided_token(sp.lo, sp.nsplit, s, min(slot, kWin - 1));
    const bool live = slot < kWin && t_tok < sp.L;
    if ((a.window > 0 || sp.nsplit != a.num_splits) && live) e_tok[r] = table_entry(a, b, t_tok);
    int64_t ko = kstand, vo = vstand;
    const bool entry_ok = token_row_entry(a, e_tok[r], g, t_tok, ko, vo);
    if (slot < kWin) {
      const bool ok = live && entry_ok;
      tok_k[slot] = ok ? ko : kstand;
      tok_v[slot] = ok ? vo : vstand;
    }
    bad_entry |= live && !entry_ok;
  }
  if (a.err && __any(bad_entry) && lane == 0) atomicOr(a.err, 1u);

  // Q of head ln as the B operand of S^T: k step kk holds the 8 head-dim
  // elements that K's lane group grp brings to that step. Rows past G repeat
  // head 0 (their probabilities are set to zero below), so the loads need no
  // branch and nothing waits for them before the first product.
  auto q_dim = [&](int kk) {
    return FP8 ? 16 * (4 * (kk / 2) + grp) + 8 * (kk % 2) : 8 * (4 * kk + grp);
  };
  uint4 qb[kNT][kKSteps];
  bool rvalid[kNT];    // lane's row (ln of tile t) exists
  int pos_row[kNT];    // MR: last token the row sees
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    int64_t q_off;
    if constexpr (MR) {
      const int f = 16 * t + ln;
      rvalid[t] = f < R;
      const int fv = rvalid[t] ? f : 0;
      q_off = prow_of(fv) * D;
      pos_row[t] = sp.L - n_rows + fv % n_rows;
    } else {
      rvalid[t] = ln < G;
      q_off = out_row0 + int64_t(rvalid[t] ? ln : 0) * D;
      pos_row[t] = 0;
    }
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) qb[t][kk] = *reinterpret_cast<const uint4*>(a.q + q_off + q_dim(kk));
  }
  const bool win = MR && a.window > 0 && a.window < (1 << 30);
  __syncthreads();   // offsets staged

  const int n_blk = strided_blocks(sp, s);   // <= NBLK
  const uint8_t* const kb8 = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* const vb8 = reinterpret_cast<const uint8_t*>(a.v);
  uint8_t* const my_vt = vt[wave];

  // Step j < kBpw: K rows of the wave's block i = j; step kBpw + i: V rows
  // of block i. kStepLd loads each: flat 16-byte piece f = 64 c + lane is
  // chunk f % kChunks of row f / kChunks.
  uint4 ring[kRing][kStepLd];
  auto fetch = [&](int j, uint4 (&buf)[kStepLd]) __attribute__((always_inline)) {
    const int i = j < kBpw ? j : j - kBpw;
    // A block past the window (waves beyond the window's blocks) reads the
    // stand-in rows; its data is not used.
    const int slot0 = (wave + kMWaves * i) * kBlockTokens;
    const bool past = slot0 >= kWin;                         // uniform per wave
    const int sl = past ? 0 : slot0;
    if (j < kBpw) {
#pragma unroll
      for (int c = 0; c < kStepLd; ++c) {
        const int f = 64 * c + lane;
        const int64_t off = past ? kstand : tok_k[sl + f / kChunks];
        buf[c] = m_load16(kb8 + off * kEsz + 16 * (f % kChunks));
      }
    } else {
#pragma unroll
      for (int c = 0; c < kStepLd; ++c) {
        const int f = 64 * c + lane;
        const int64_t off = past ? vstand : tok_v[sl + f / kChunks];
        buf[c] = m_load16(vb8 + off * kEsz + 16 * (f % kChunks));
      }
    }
  };

  mfloat4_t st[kBpw][2][kNT];   // scores (log2 units) of row ln of tile t, tokens 16 h + 4 grp + r of block i
  mfloat4_t o[kNT][kDBlocks];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) o[t][db] = mfloat4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_w[kNT], l_w[kNT];   // row ln of tile t: the wave's max and sum of probabilities
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    m_w[t] = kMMinit;
    l_w[t] = 0.0f;
  }

  auto consume_k = [&](int i, const uint4 (&buf)[kStepLd]) __attribute__((always_inline)) {
    // Whole K rows into the wave's tile, then each lane reads its token's
    // 16-byte chunks 4 c + grp back as MFMA A operands.
#pragma unroll
    for (int c = 0; c < kStepLd; ++c) {
      const int f = 64 * c + lane;
      *reinterpret_cast<uint4*>(my_vt + (f / kChunks) * kPitch + 16 * (f % kChunks)) = buf[c];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      mfloat4_t acc[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) acc[t] = mfloat4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kKLd; ++c) {
        const uint4 x = *reinterpret_cast<const uint4*>(my_vt + (16 * h + ln) * kPitch + 16 * (4 * c + grp));
        if constexpr (FP8) {
          const uint4 xa = m_fp8x8_to_bf16(x.x, x.y), xb = m_fp8x8_to_bf16(x.z, x.w);
#pragma unroll
          for (int t = 0; t < kNT; ++t) {
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(xa), m_as_bf16x8(qb[t][2 * c]), acc[t], 0, 0, 0);
            acc[t] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(xb), m_as_bf16x8(qb[t][2 * c + 1]), acc[t], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < kNT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(x), m_as_bf16x8(qb[t][c]), acc[t], 0, 0, 0);
        }
      }
      // A stand-in key gives NaN: the token does not count; with several
      // rows, nor does a token past the row's position (or before its window).
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int tok = 0;
        if constexpr (MR) tok = strided_token(sp.lo, sp.nsplit, s, (wave + kMWaves * i) * kBlockTokens + 16 * h + 4 * grp + r);
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          const float sc = acc[t][r];
          bool vis = sc == sc;
          if constexpr (MR) vis = vis && tok <= pos_row[t] && (!win || tok > pos_row[t] - a.window);
          const float x = vis ? sc * a.scale_log2 : -INFINITY;
          acc[t][r] = x;
          m_w[t] = fmaxf(m_w[t], x);
        }
      }
#pragma unroll
      for (int t = 0; t < kNT; ++t) st[i][h][t] = acc[t];
    }
  };

  auto consume_v = [&](int i, const uint4 (&buf)[kStepLd]) __attribute__((always_inline)) {
    // The block's V rows into the wave's transpose tile (the wave's LDS
    // operations run in order, so the reads below see these writes, and the
    // next block's writes follow this block's reads).
#pragma unroll
    for (int c = 0; c < kStepLd; ++c) {
      const int f = 64 * c + lane;
      *reinterpret_cast<uint4*>(my_vt + (f / kChunks) * kPitch + 16 * (f % kChunks)) = buf[c];
    }
    // P = 2^(s - m) of row ln of each tile (zero past the rows), as hi + lo
    // bf16 A operands; k slot grp holds tokens 4 grp .. + 3 and 16 + 4 grp .. + 3.
    mbf16x8_t ph[kNT], pl[kNT];
#pragma unroll
    for (int tt = 0; tt < kNT; ++tt) {
      uint32_t hi[4], lo[4];
      float ls = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int h = t >> 1, r0 = (t & 1) * 2;
        const float p0 = rvalid[tt] ? fast_exp2(st[i][h][tt][r0] - m_w[tt]) : 0.0f;
        const float p1 = rvalid[tt] ? fast_exp2(st[i][h][tt][r0 + 1] - m_w[tt]) : 0.0f;
        ls += p0 + p1;
        const uint32_t w = m_bf16_pair(p0, p1);
        hi[t] = w;
        lo[t] = m_bf16_pair(p0 - bf16_lo(w), p1 - bf16_hi(w));
      }
      l_w[tt] += ls;
      ph[tt] = m_as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
      pl[tt] = m_as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
      uint4 vu;
      if constexpr (FP8) {
        // Lane ln points at row T(ln / 2) (T(e) = 4 grp + e, then 16 + 4 grp + e - 4),
        // bytes 16 db + 8 (ln % 2) .. + 8; it receives column 16 db + ln of those 8 rows.
        const int e = ln >> 1;
        const int row = (e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4));
        const mint2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_mint2_ptr)(my_vt + row * kPitch + 16 * db + 8 * (ln & 1)));
        vu = m_fp8x8_to_bf16(uint32_t(w[0]), uint32_t(w[1]));
      } else {
        // Lane ln points at row 4 grp + ln / 4 (then + 16), elements
        // 16 db + 4 (ln % 4) .. + 4; it receives column 16 db + ln of those 4 rows.
        const int rowa = 4 * grp + (ln >> 2);
        const int colb = (16 * db + 4 * (ln & 3)) * 2;
        const mshort4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_mshort4_ptr)(my_vt + rowa * kPitch + colb));
        const mshort4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_mshort4_ptr)(my_vt + (rowa + 16) * kPitch + colb));
        vu = make_uint4(uint32_t(uint16_t(va[0])) | (uint32_t(uint16_t(va[1])) << 16),
                        uint32_t(uint16_t(va[2])) | (uint32_t(uint16_t(va[3])) << 16),
                        uint32_t(uint16_t(vb[0])) | (uint32_t(uint16_t(vb[1])) << 16),
                        uint32_t(uint16_t(vb[2])) | (uint32_t(uint16_t(vb[3])) << 16));
      }
#pragma unroll
      for (int tt = 0; tt < kNT; ++tt) {
        o[tt][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[tt], m_as_bf16x8(vu), o[tt][db], 0, 0, 0);
        o[tt][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[tt], m_as_bf16x8(vu), o[tt][db], 0, 0, 0);
      }
    }
  };

  // One stream of kSteps steps (K pass, then V pass) through kRing register
  // buffers, fully unrolled; loads are issued for every step (a dead block
  // reads stand-in rows) and the arithmetic of dead blocks is skipped with
  // uniform branches.
  // The scheduling barriers keep the steps' loads in step order, so each
  // step waits only for its own loads (vmcnt counts in issue order).
  static_for<0, (kRing - 1 < kSteps ? kRing - 1 : kSteps)>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    fetch(j, ring[j % kRing]);
    __builtin_amdgcn_sched_barrier(0);
  });
  static_for<0, kSteps>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int jn = j + kRing - 1;
    if constexpr (jn < kSteps) fetch(jn, ring[jn % kRing]);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int i = j < kBpw ? j : j - kBpw;
    if (wave + kMWaves * i < n_blk) {
      if constexpr (j < kBpw) consume_k(i, ring[j % kRing]);
      else consume_v(i, ring[j % kRing]);
    }
    if constexpr (j == kBpw - 1) {   // row ln's max over the wave's tokens
#pragma unroll
      for (int t = 0; t < kNT; ++t) m_w[t] = rows_max(m_w[t]);
    }
  });
#pragma unroll
  for (int t = 0; t < kNT; ++t) l_w[t] = rows_sum(l_w[t]);

  if constexpr (MR) {
    // One 16-row tile at a time: each wave publishes O of the tile's rows
    // with its (max, sum) per row; after a barrier the workgroup rescales the
    // waves to a common max, adds them in wave order and writes the rows'
    // partials (or normalised outputs and log-sum-exp for a single split).
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      if (16 * t >= R) break;   // uniform
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) mrg_acc[wave][4 * grp + r][16 * db + ln] = o[t][db][r];
      if (grp == 0) {
        mrg_m[ln][wave] = m_w[t];
        mrg_l[ln][wave] = l_w[t];
      }
      __syncthreads();
      for (int i4 = tid; i4 < 16 * D / 4; i4 += kMThreads) {
        const int rl = (4 * i4) / D, d = 4 * i4 - rl * D;
        const int f = 16 * t + rl;
        if (f >= R) continue;
        const float4 mv = *reinterpret_cast<const float4*>(&mrg_m[rl][0]);
        const float4 lv = *reinterpret_cast<const float4*>(&mrg_l[rl][0]);
        const float mw[4] = {mv.x, mv.y, mv.z, mv.w}, lw[4] = {lv.x, lv.y, lv.z, lv.w};
        float M = mw[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, mw[w]);
        float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float den = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 v4 = *reinterpret_cast<const float4*>(&mrg_acc[w][rl][d]);
          const float fw = fast_exp2(mw[w] - M);
          num.x = fmaf(fw, v4.x, num.x);
          num.y = fmaf(fw, v4.y, num.y);
          num.z = fmaf(fw, v4.z, num.z);
          num.w = fmaf(fw, v4.w, num.w);
          den = fmaf(fw, lw[w], den);
        }
        const int64_t prow = prow_of(f);
        if (sp.nsplit == 1) {
          const float4 o4 = den > 0.0f ? make_float4(num.x / den, num.y / den, num.z / den, num.w / den)
                                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          store_out4(a, prow * D + d, o4);
          if (d == 0) store_lse(a, prow, M, den);
        } else {
          const int64_t pr = prow * a.num_splits + s;
          *reinterpret_cast<float4*>(a.part_acc + pr * D + d) = num;
          if (d == 0) *reinterpret_cast<float2*>(a.part_ml + pr * 2) = make_float2(M, den);
        }
      }
      __syncthreads();   // the tile's LDS rows are read before the next tile's
    }
    return;
  }

  // Publish O of the G heads (lane: column 16 db + ln of heads 4 grp + r)
  // with the wave's (max, sum) per head.
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h < G) mrg_acc[wave][h][16 * db + ln] = o[0][db][r];
    }
  if (grp == 0 && ln < G) {
    mrg_m[ln][wave] = m_w[0];
    mrg_l[ln][wave] = l_w[0];
  }
  __syncthreads();

  // One thread per 4 consecutive outputs: rescale the waves to the workgroup
  // max and add them in wave order.
  const int64_t prow0 = int64_t(b) * a.q_len * a.hq + int64_t(g) * G;   // partial row of head 0
  for (int i4 = tid; i4 < G * D / 4; i4 += kMThreads) {
    const int h = (4 * i4) / D, d = 4 * i4 - h * D;
    float mw[kMWaves], lw[kMWaves];
#pragma unroll
    for (int w = 0; w < kMWaves; w += 4) {
      const float4 mv = *reinterpret_cast<const float4*>(&mrg_m[h][w]);
      const float4 lv = *reinterpret_cast<const float4*>(&mrg_l[h][w]);
      mw[w] = mv.x;
      mw[w + 1] = mv.y;
      mw[w + 2] = mv.z;
      mw[w + 3] = mv.w;
      lw[w] = lv.x;
      lw[w + 1] = lv.y;
      lw[w + 2] = lv.z;
      lw[w + 3] = lv.w;
    }
    float4 acc4[kMWaves];
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) acc4[w] = *reinterpret_cast<const float4*>(&mrg_acc[w][h][d]);
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < kMWaves; ++w) M = fmaxf(M, mw[w]);
    float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) {
      const float f = fast_exp2(mw[w] - M);
      num.x = fmaf(f, acc4[w].x, num.x);
      num.y = fmaf(f, acc4[w].y, num.y);
      num.z = fmaf(f, acc4[w].z, num.z);
      num.w = fmaf(f, acc4[w].w, num.w);
      den = fmaf(f, lw[w], den);
    }
    if (sp.nsplit == 1) {
      const float4 o4 = den > 0.0f ? make_float4(num.x / den, num.y / den, num.z / den, num.w / den)
                                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      store_out4(a, out_row0 + 4 * i4, o4);
    } else {
      const int64_t pr = (prow0 + h) * a.num_splits + s;
      *reinterpret_cast<float4*>(a.part_acc + pr * D + d) = num;
      if (d == 0) *reinterpret_cast<float2*>(a.part_ml + pr * 2) = make_float2(M, den);
    }
  }
  if (sp.nsplit == 1 && a.lse != nullptr && tid < G) {
    float M = mrg_m[tid][0];
#pragma unroll
    for (int w = 1; w < kMWaves; ++w) M = fmaxf(M, mrg_m[tid][w]);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) den = fmaf(fast_exp2(mrg_m[tid][w] - M), mrg_l[tid][w], den);
    store_lse(a, out_row0 / D + tid, M, den);
  }
}

// Launch the MFMA split kernel with a window of NBLK strided blocks of 32
// tokens (a.chunk <= NBLK * 32), WAVES waves per workgroup and a register
// ring of RING steps.
template <int NBLK, bool FP8, int WAVES, int RING, bool MR = false>
hipError_t launch_decode_mfma_window(const DecodeArgs& a, int head_dim, int group, hipStream_t st, hipEvent_t e0,
                                     hipEvent_t e1) {
  if (a.chunk > NBLK * kBlockTokens || bool(a.kv_fp8) != FP8 || group < 1)
    return hipErrorInvalidValue;
  if (MR ? int64_t(group) * a.q_len > 32 : group > kMMaxG) return hipErrorInvalidValue;
  dim3 grid(a.num_splits, a.hkv, a.num_seqs);
  auto go = [&](auto kern) {
    if (e0 && e1)
      hipExtLaunchKernelGGL(kern, grid, dim3(64 * WAVES), 0, st, e0, e1, 0, a);
    else
      hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), 0, st, a);
    return hipGetLastError();
  };
  if (head_dim == 256) return go(decode_mfma_kernel<256, NBLK, FP8, WAVES, RING, MR>);
  if constexpr (!MR)   // several rows: head_dim 256 only
    if (head_dim == 128) return go(decode_mfma_kernel<128, NBLK, FP8, WAVES, RING, MR>);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pkv
