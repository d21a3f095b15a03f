// Host side of the C ABI declared in include/pkv.h: argument checks, the split
// planner, workspace layout, kernel selection and launches. No device memory
// is allocated here and no call synchronises the stream (the debug readers
// excepted).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_common.h"

namespace {

thread_local std::string g_last_error;
struct VariantInfo {
  const char* split_name = nullptr;
  int head_dim = 0, group = 0, q_len = 0, window = 0, splits = 0, chunk = 0, block_size = 0;
};
thread_local VariantInfo g_last_variant;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {0};

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return PKV_ERR_HIP;
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool mult8_pos(int64_t s) { return s > 0 && (s % 8) == 0; }

static_assert(sizeof(pkv_decode_params) == 120, "pkv_decode_params layout");

// Longest token range one sequence's splits must cover: the whole context,
// or with a sliding window the union of its rows' windows (window + q_len - 1).
int64_t plan_span(const pkv_decode_params* p) {
  int64_t span = p->max_seq_len;
  if (p->window > 0 && int64_t(p->window) + p->q_len - 1 < span) span = int64_t(p->window) + p->q_len - 1;
  return span;
}

int plan(const pkv_decode_params* p, int32_t cu_count, int32_t* S, int32_t* chunk) {
  const int64_t T = pkv::kTile;
  const int64_t span = plan_span(p);
  const int64_t n_tiles = span > 0 ? cdiv64(span, T) : 1;
  const int64_t cap = pkv::kMaxTiles;
  int64_t c;
  if (p->num_splits > 0) {
    c = cdiv64(n_tiles, p->num_splits);
  } else {
    int64_t work = p->total_tokens > 0 ? p->total_tokens : int64_t(p->num_seqs) * p->max_seq_len;
    if (p->window > 0 && int64_t(p->num_seqs) * span < work) work = int64_t(p->num_seqs) * span;
    int64_t target = int64_t(cu_count) * pkv::kWgPerCu;
    if (target < 1) target = 1;
    c = cdiv64(int64_t(p->num_kv_heads) * work, target * T);
    if (c < pkv::kMinTiles) c = pkv::kMinTiles;
  }
  if (c > n_tiles) c = n_tiles;
  if (c > cap) c = cap;
  if (c < 1) c = 1;
  *S = int32_t(cdiv64(n_tiles, c));
  *chunk = int32_t(c * T);
  return PKV_OK;
}

// Workspace layout: the 256-byte header (error word), the (max, sum) pairs
// and the accumulators of every split of every output row.
struct WsLayout {
  int64_t ml, acc, total;
};

WsLayout workspace_layout(const pkv_decode_params* p, int32_t S) {
  const int64_t rows = int64_t(p->num_seqs) * p->q_len * p->num_q_heads;
  WsLayout w;
  w.ml = pkv::kWsHeaderBytes;
  w.acc = w.ml + align256(rows * S * 2 * 4);
  w.total = w.acc + align256(rows * S * int64_t(p->head_dim) * 4);
  return w;
}

int64_t workspace_for(const pkv_decode_params* p, int32_t S) { return workspace_layout(p, S).total; }

int device_cu_count(int32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < kMaxDevices && g_cu_count[dev] > 0) {
    *out = g_cu_count[dev];
    return PKV_OK;
  }
  int cu = 0;
  e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
  if (cu < 1) return fail(PKV_ERR_HIP, "device reports no compute units");
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev] = cu;
  *out = cu;
  return PKV_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

pkv::DecodeArgs make_args(const pkv_decode_params* p, int32_t S, int32_t chunk) {
  pkv::DecodeArgs a{};
  a.k_sp = p->k_stride_page;
  a.k_st = p->k_stride_tok;
  a.k_sh = p->k_stride_head;
  a.v_sp = p->v_stride_page;
  a.v_st = p->v_stride_tok;
  a.v_sh = p->v_stride_head;
  a.num_seqs = p->num_seqs;
  a.q_len = p->q_len;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.max_pages = p->max_pages_per_seq;
  a.num_pages = p->num_pages;
  a.chunk = chunk;
  a.num_splits = S;
  a.bdiv = pkv::make_magic(uint32_t(p->block_size));
  const bool fp8 = p->kv_dtype == PKV_KV_FP8_E4M3;
  // FP8 caches: K's per-tensor scale folds into the score scale, V's into the
  // stored output (partials stay unscaled).
  a.scale_log2 = float(double(p->scale) * (fp8 ? double(p->k_scale) : 1.0) * 1.4426950408889634);
  a.out_scale = fp8 ? p->v_scale : 1.0f;
  a.kv_fp8 = fp8;
  a.out_bf16 = p->out_dtype == PKV_OUT_BF16;
  a.window = p->window;
  return a;
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "pkv 0.2.0 gfx950"; }

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Query rows per sequence a prefill call accepts.
constexpr int32_t kMaxPrefillRows = 1 << 24;

// Checks shared by every call (all but the kernels' limits on the group size);
// max_q_len is 16 for the decode and varlen calls.
int validate_common(const pkv_decode_params* p, int32_t max_q_len = 16) {
  if (!p) return fail(PKV_ERR_INVALID, "params is NULL");
  if (p->num_seqs < 1 || p->q_len < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->block_size < 1 || p->max_pages_per_seq < 1 || p->num_pages < 1 || p->max_seq_len < 0 ||
      p->num_splits < 0 || p->total_tokens < 0 || p->window < 0)
    return fail(PKV_ERR_INVALID, "a size is out of range");
  if (p->kv_dtype != PKV_KV_BF16 && p->kv_dtype != PKV_KV_FP8_E4M3) return fail(PKV_ERR_INVALID, "unknown kv_dtype");
  if (p->kv_dtype == PKV_KV_FP8_E4M3 &&
      !(isfinite(p->k_scale) && p->k_scale > 0.0f && isfinite(p->v_scale) && p->v_scale > 0.0f))
    return fail(PKV_ERR_INVALID, "FP8 caches need finite, positive k_scale and v_scale");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads is not a multiple of num_kv_heads");
  if (p->head_dim != 128 && p->head_dim != 256) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 128 or 256");
  if (p->q_len > max_q_len)
    return fail(PKV_ERR_UNSUPPORTED, "q_len above " + std::to_string(max_q_len));
  if (p->max_seq_len > (1 << 30)) return fail(PKV_ERR_UNSUPPORTED, "max_seq_len above 2^30 tokens");
  if (int64_t(p->max_pages_per_seq) * p->block_size < p->max_seq_len)
    return fail(PKV_ERR_INVALID, "max_seq_len exceeds max_pages_per_seq * block_size");
  if (!mult8_pos(p->k_stride_page) || !mult8_pos(p->k_stride_tok) || !mult8_pos(p->k_stride_head) ||
      !mult8_pos(p->v_stride_page) || !mult8_pos(p->v_stride_tok) || !mult8_pos(p->v_stride_head))
    return fail(PKV_ERR_INVALID, "K/V strides must be positive multiples of 8 elements");
  if (p->kv_dtype == PKV_KV_FP8_E4M3 &&
      ((p->k_stride_page | p->k_stride_tok | p->k_stride_head | p->v_stride_page | p->v_stride_tok |
        p->v_stride_head) & 15) != 0)
    return fail(PKV_ERR_INVALID, "FP8 K/V strides must be multiples of 16 elements (16-byte rows)");
  if (p->block_size > (1 << 20)) return fail(PKV_ERR_UNSUPPORTED, "block_size above 2^20 tokens");
  if (int64_t(p->block_size) * p->k_stride_tok >= (int64_t(1) << 31) ||
      int64_t(p->block_size) * p->v_stride_tok >= (int64_t(1) << 31))
    return fail(PKV_ERR_UNSUPPORTED, "block_size * token stride must stay below 2^31 elements");
  if (!isfinite(p->scale)) return fail(PKV_ERR_INVALID, "scale is not finite");
  if (p->out_dtype != PKV_OUT_F32 && p->out_dtype != PKV_OUT_BF16)
    return fail(PKV_ERR_INVALID, "unknown out_dtype");
  return PKV_OK;
}

// The split and merge grids of the decode and varlen calls put sequences, KV
// heads and query heads in their y and z dimensions (at most 65535 each).
int validate_grid_yz(const pkv_decode_params* p) {
  if (p->num_seqs > 65535 || p->num_kv_heads > 65535 || p->num_q_heads > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "more than 65535 sequences, KV heads or query heads");
  return PKV_OK;
}

int validate_varlen(const pkv_decode_params* p) {
  int rc = validate_common(p);
  if (!rc) rc = validate_grid_yz(p);
  if (rc) return rc;
  if (!pkv::verify_supported(p->head_dim, p->num_q_heads / p->num_kv_heads, p->q_len))
    return fail(PKV_ERR_UNSUPPORTED, "varlen calls need (Hq / Hkv) * max q_len <= 128");
  return PKV_OK;
}

// Query positions per prefill workgroup: as many as fill the MFMA kernel's
// 128 rows with all query heads of one KV head.
int32_t prefill_rows(const pkv_decode_params* p) { return 128 / (p->num_q_heads / p->num_kv_heads); }

int validate_prefill(const pkv_decode_params* p) {
  int rc = validate_common(p, kMaxPrefillRows);
  if (rc) return rc;
  if (p->num_q_heads / p->num_kv_heads > 128)
    return fail(PKV_ERR_UNSUPPORTED, "prefill calls need Hq / Hkv <= 128");
  if (int64_t(p->num_seqs) * p->q_len > (int64_t(1) << 31) - 1)
    return fail(PKV_ERR_UNSUPPORTED, "num_seqs * q_len above 2^31 - 1 rows");
  const int32_t pf = prefill_rows(p);
  if ((int64_t(p->q_len) + pf - 1) / pf * p->num_kv_heads * p->num_seqs > (int64_t(1) << 31) - 1)
    return fail(PKV_ERR_UNSUPPORTED, "more than 2^31 - 1 prefill blocks");
  return PKV_OK;
}

// Shapes that the uniform or the varlen call accepts (plan and workspace
// queries serve both).
int validate_any(const pkv_decode_params* p);

// Plan, check the workspace and launch the split kernel (then the merge when
// the plan has several splits). cu_q == nullptr: uniform call, q_len rows per
// sequence (q_len 1 on the VALU decode kernel); else varlen rows on the MFMA
// kernel.
int launch_call(const pkv_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q, void* out,
                float* lse, void* workspace, int64_t workspace_bytes, void* stream,
                uint32_t* error_word = nullptr) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out || !workspace)
    return fail(PKV_ERR_INVALID, "a device pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3) != 0) return fail(PKV_ERR_INVALID, "lse must be 4-byte aligned");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "q, k_cache, v_cache and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(PKV_ERR_INVALID, "workspace must be 256-byte aligned");
  int32_t cu = 0;
  int rc = device_cu_count(&cu);
  if (rc) return rc;
  int32_t S = 0, chunk = 0;
  plan(p, cu, &S, &chunk);
  const int64_t need = workspace_for(p, S);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");

  pkv::DecodeArgs a = make_args(p, S, chunk);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.out = out;
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  const WsLayout wl = workspace_layout(p, S);
  a.err = error_word ? error_word : reinterpret_cast<uint32_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + wl.ml);
  a.part_acc = reinterpret_cast<float*>(ws + wl.acc);
  a.many_wg = int64_t(S) * p->num_kv_heads * p->num_seqs > cu ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int group = p->num_q_heads / p->num_kv_heads;
  hipError_t e;
  const char* split_name;
  int window;
  if (p->q_len == 1 && !cu_q && pkv::decode_supported(p->head_dim, group)) {
    e = pkv::launch_decode_split(a, p->head_dim, group, st, g_ev_start, g_ev_stop);
    // 4-wave workgroups for grids of several workgroups per CU (512-token window)
    split_name = a.kv_fp8 ? "decode_mfma" : "decode_valu";
    window = pkv::decode_window(chunk);
  } else if ((p->q_len > 1 || cu_q) && chunk > 256 && pkv::rows_mfma_supported(p->head_dim, group, p->q_len)) {
    // At most 32 rows per KV head and splits of more than 256 tokens: each
    // wave streams its own blocks (no shared LDS tiles, no barrier per tile),
    // two 16-row MFMA tiles. Shorter splits stay on the tiled kernel, which
    // is faster there (q_len 4: 16K 23.5 against 24.8 us, 4K 15.7 against
    // 17.9 us per step).
    e = pkv::launch_decode_mfma_rows(a, p->head_dim, group, st, g_ev_start, g_ev_stop);
    split_name = cu_q ? "varlen_rows" : "verify_rows";
    window = pkv::decode_window(chunk);
  } else {
    e = pkv::launch_verify_split(a, p->head_dim, group, st, g_ev_start, g_ev_stop);
    split_name = cu_q ? "varlen_mfma" : "verify_mfma";
    window = 64;   // 64-token K/V tiles, looped over the split
  }
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  if (S > 1) {
    e = pkv::launch_lse_merge(a, p->head_dim, st);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  }
  g_last_variant = VariantInfo{split_name, p->head_dim, group, p->q_len, window, S, chunk, p->block_size};
  return PKV_OK;
}

// Scratch memory of the call that allocates nothing: a file-scope device
// array (one copy per GPU, held until the process ends), laid out like a
// workspace. Nothing in it has to start at zero: the partials are written
// before they are read, and the error bits go to the caller's word (or to
// the array's own first word, which nothing reads).
constexpr int64_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The device address of `scratch` on the current device, found once per
// device with hipGetSymbolAddress (the host-side name of the array is not a
// device address).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255) != 0)
      return fail(PKV_ERR_HIP, "scratch array has no 256-byte aligned device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

int validate_any(const pkv_decode_params* p) {
  const int rc = pkv_validate_params(p);
  return rc && validate_varlen(p) ? rc : PKV_OK;
}

}  // namespace

extern "C" {

int pkv_validate_params(const pkv_decode_params* p) {
  int rc = validate_common(p);
  if (!rc) rc = validate_grid_yz(p);
  if (rc) return rc;
  const int group = p->num_q_heads / p->num_kv_heads;
  // q_len 1 with up to 8 query heads per KV head runs on the decode kernel;
  // larger groups and multi-row calls on the MFMA kernel.
  if (!(p->q_len == 1 && pkv::decode_supported(p->head_dim, group)) &&
      !pkv::verify_supported(p->head_dim, group, p->q_len))
    return fail(PKV_ERR_UNSUPPORTED, "needs (Hq / Hkv) * q_len <= 128");
  return PKV_OK;
}

int pkv_plan_splits(const pkv_decode_params* p, int32_t cu_count, int32_t* num_splits, int32_t* chunk_tokens) {
  int rc = validate_any(p);
  if (rc) return rc;
  if (cu_count < 1 || !num_splits || !chunk_tokens) return fail(PKV_ERR_INVALID, "bad cu_count or output pointer");
  return plan(p, cu_count, num_splits, chunk_tokens);
}

int pkv_plan_constants(int32_t* tile, int32_t* wg_per_cu, int32_t* min_tiles, int32_t* max_tiles) {
  if (tile) *tile = pkv::kTile;
  if (wg_per_cu) *wg_per_cu = pkv::kWgPerCu;
  if (min_tiles) *min_tiles = pkv::kMinTiles;
  if (max_tiles) *max_tiles = pkv::kMaxTiles;
  return PKV_OK;
}

int64_t pkv_workspace_bytes(const pkv_decode_params* p, int32_t cu_count) {
  int rc = validate_any(p);
  if (rc) return rc;
  if (cu_count <= 0) {
    rc = device_cu_count(&cu_count);
    if (rc) return rc;
  }
  int32_t S = 0, chunk = 0;
  plan(p, cu_count, &S, &chunk);
  return workspace_for(p, S);
}

int pkv_device_cu_count(int32_t* cu_count) {
  if (!cu_count) return fail(PKV_ERR_INVALID, "cu_count is NULL");
  return device_cu_count(cu_count);
}

int pkv_paged_decode_attention(const pkv_decode_params* p, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                               void* out, float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  int rc = pkv_validate_params(p);
  if (rc) return rc;
  return launch_call(p, q, k_cache, v_cache, block_table, seq_lens, nullptr, out, lse, workspace, workspace_bytes,
                     stream);
}

int pkv_paged_decode_attention_noalloc(const pkv_decode_params* p, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                       void* out, float* lse, uint32_t* error_word, void* stream) {
  int rc = pkv_validate_params(p);
  if (rc) return rc;
  if ((reinterpret_cast<uintptr_t>(error_word) & 3) != 0)
    return fail(PKV_ERR_INVALID, "error_word must be 4-byte aligned");
  int32_t cu = 0;
  rc = device_cu_count(&cu);
  if (rc) return rc;
  int32_t S = 0, chunk = 0;
  plan(p, cu, &S, &chunk);
  const int64_t need = workspace_for(p, S);
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "the call needs " + std::to_string(need) + " bytes of scratch; the library's "
                "scratch holds " + std::to_string(kScratchBytes) + " (use pkv_paged_decode_attention with a workspace)");
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return launch_call(p, q, k_cache, v_cache, block_table, seq_lens, nullptr, out, lse, ws, kScratchBytes, stream,
                     error_word);
}

int pkv_paged_varlen_attention(const pkv_decode_params* p, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* cu_seqlens_q, void* out, float* lse, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  int rc = validate_varlen(p);
  if (rc) return rc;
  if (!cu_seqlens_q) return fail(PKV_ERR_INVALID, "cu_seqlens_q is NULL");
  return launch_call(p, q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, out, lse, workspace,
                     workspace_bytes, stream);
}

int pkv_paged_prefill_attention(const pkv_decode_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* cu_seqlens_q, void* out, float* lse, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  int rc = validate_prefill(p);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !cu_seqlens_q || !out || !workspace)
    return fail(PKV_ERR_INVALID, "a device pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3) != 0) return fail(PKV_ERR_INVALID, "lse must be 4-byte aligned");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "q, k_cache, v_cache and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(PKV_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < PKV_PREFILL_WORKSPACE_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "workspace needs " + std::to_string(PKV_PREFILL_WORKSPACE_BYTES) + " bytes");
  pkv::DecodeArgs a = make_args(p, 1, 0);
  a.pf_rows = prefill_rows(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_seqlens_q;
  a.out = out;
  a.lse = lse;
  a.err = static_cast<uint32_t*>(workspace);
  const int group = p->num_q_heads / p->num_kv_heads;
  hipError_t e = pkv::launch_prefill(a, p->head_dim, group, static_cast<hipStream_t>(stream), g_ev_start, g_ev_stop);
  if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
  g_last_variant = VariantInfo{"prefill_mfma", p->head_dim, group, p->q_len, a.pf_rows, 1, 0, p->block_size};
  return PKV_OK;
}

int pkv_last_variant(char* buf, int32_t len) {
  const VariantInfo& v = g_last_variant;
  char tmp[256];
  int n = 0;
  if (v.split_name)
    n = snprintf(tmp, sizeof tmp, "%s d%d g%d q%d w%d%s splits=%d chunk=%d B=%d", v.split_name, v.head_dim,
                 v.group, v.q_len, v.window, v.splits > 1 ? " + lse_merge" : "", v.splits, v.chunk, v.block_size);
  else
    tmp[0] = '\0';
  if (buf && len > 0) {
    const int c = n < len - 1 ? n : len - 1;
    memcpy(buf, tmp, size_t(c));
    buf[c] = '\0';
  }
  return n;
}

int pkv_set_timing_events(void* ev_start, void* ev_stop) {
  if ((ev_start == nullptr) != (ev_stop == nullptr))
    return fail(PKV_ERR_INVALID, "pass both events or neither");
  g_ev_start = static_cast<hipEvent_t>(ev_start);
  g_ev_stop = static_cast<hipEvent_t>(ev_stop);
  return PKV_OK;
}

int pkv_debug_token_offsets(const pkv_decode_params* p, const int32_t* block_table, const int32_t* seq_lens,
                            int32_t kv_head, int64_t* k_off, int64_t* v_off, void* stream) {
  int rc = pkv_validate_params(p);
  if (rc) return rc;
  if (!block_table || !seq_lens || !k_off || !v_off) return fail(PKV_ERR_INVALID, "a device pointer is NULL");
  if (kv_head < 0 || kv_head >= p->num_kv_heads) return fail(PKV_ERR_INVALID, "kv_head out of range");
  int32_t cu = 0;
  rc = device_cu_count(&cu);
  if (rc) return rc;
  int32_t S = 0, chunk = 0;
  plan(p, cu, &S, &chunk);
  pkv::DecodeArgs a = make_args(p, S, chunk);
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.err = nullptr;   // debug path: invalid entries still read as -2, nothing is flagged
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const size_t n = size_t(p->num_seqs) * size_t(p->max_seq_len) * sizeof(int64_t);
  if (n > 0) {
    if ((e = hipMemsetAsync(k_off, 0xff, n, st)) != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    if ((e = hipMemsetAsync(v_off, 0xff, n, st)) != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  }
  e = pkv::launch_debug_offsets(a, kv_head, p->max_seq_len, k_off, v_off, st);
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return PKV_OK;
}

int pkv_debug_split_ranges(const pkv_decode_params* p, const int32_t* seq_lens, int32_t* ranges, void* stream) {
  int rc = pkv_validate_params(p);
  if (rc) return rc;
  if (!seq_lens || !ranges) return fail(PKV_ERR_INVALID, "a device pointer is NULL");
  int32_t cu = 0;
  rc = device_cu_count(&cu);
  if (rc) return rc;
  int32_t S = 0, chunk = 0;
  plan(p, cu, &S, &chunk);
  pkv::DecodeArgs a = make_args(p, S, chunk);
  a.seq_lens = seq_lens;
  hipError_t e = pkv::launch_debug_ranges(a, ranges, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return PKV_OK;
}

int pkv_debug_token_splits(const pkv_decode_params* p, const int32_t* seq_lens, int32_t* slots, void* stream) {
  int rc = pkv_validate_params(p);
  if (rc) return rc;
  if (!seq_lens || !slots) return fail(PKV_ERR_INVALID, "a device pointer is NULL");
  if (p->q_len != 1) return fail(PKV_ERR_INVALID, "the strided splits are those of q_len == 1 calls");
  int32_t cu = 0;
  rc = device_cu_count(&cu);
  if (rc) return rc;
  int32_t S = 0, chunk = 0;
  plan(p, cu, &S, &chunk);
  pkv::DecodeArgs a = make_args(p, S, chunk);
  a.seq_lens = seq_lens;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const size_t n = size_t(p->num_seqs) * size_t(p->max_seq_len) * 2 * sizeof(int32_t);
  if (n > 0 && (e = hipMemsetAsync(slots, 0xff, n, st)) != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  e = pkv::launch_debug_token_splits(a, p->max_seq_len, slots, st);
  if (e != hipSuccess) return hip_fail(e, "debug kernel launch");
  return PKV_OK;
}

int64_t pkv_magic_div_check(int32_t divisor, int64_t n_max) {
  if (divisor < 1 || n_max < 0 || n_max > 0xffffffffLL) return -2;
  const pkv::MagicDiv md = pkv::make_magic(uint32_t(divisor));
  // The reference quotient and remainder are carried along n (no division
  // per step), so whole ranges of 2^30 numbers take about a second.
  uint32_t q = 0, r = 0;
  for (int64_t n = 0; n <= n_max; ++n) {
    if (pkv::magic_div(uint32_t(n), md) != q) return n;
    if (++r == uint32_t(divisor)) {
      r = 0;
      ++q;
    }
  }
  return -1;
}

int pkv_read_error_word(const void* workspace, int32_t* value) {
  if (!workspace || !value) return fail(PKV_ERR_INVALID, "NULL pointer");
  hipError_t e = hipMemcpy(value, workspace, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  return PKV_OK;
}

}  // extern "C"
