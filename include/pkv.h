/*
 * pkv.h — C ABI of the paged decode-attention library for AMD MI355X (gfx950).
 *
 * The operation (what one call computes) follows the statement of the problem
 * in "DCU page832 attention" (luanjiahao.me): a token's logical page is
 * token / BLOCK_SIZE, its in-page offset token % BLOCK_SIZE, the block table
 * maps logical to physical page, and strides for page, token and KV head give
 * the element address (§1, §4); per key tile, score = dot(Q, K) * scale and an
 * online softmax accumulates V (§5); decode reads every logical page of the
 * sequence (§7). The KV range of one (sequence, KV head) is cut into splits
 * that run on separate workgroups and are merged afterwards, as the split-KV
 * paragraph of "vLLM 下双卡 Radeon 上的混合 SSM 解码速率" describes; several
 * query rows of one request share each K/V walk with a per-row causal mask and
 * a merge of partial softmax statistics, as in "Qwen3.8 auf MI350P betreiben",
 * Lektion 3.
 *
 * For sequence b, query row i and query head h (G = Hq / Hkv, KV head h / G):
 *     out[b,i,h,:] = softmax_j( scale * q[b,i,h,:] . K_j ) V_j,
 *     j over tokens 0 .. seq_lens[b] - q_len + i   (bottom-right causal window)
 * With a sliding window W > 0, row i sees only its last W of those tokens
 * (j > seq_lens[b] - q_len + i - W): "如何在单张 RTX 3090 上让 Qwen3.5-27B
 * token 生成速度提升 6 倍" restricts decode attention to the most recent
 * 2,048 KV positions this way.
 *
 * Conventions shared by every entry point:
 *   - All pointers named *device* point to device memory on the current HIP
 *     device; everything else is host memory. The caller owns every buffer.
 *   - bf16 is IEEE bfloat16 (uint16 storage). Strides are in elements.
 *   - Functions return 0 (PKV_OK) or a negative PKV_ERR_* code and never throw.
 *     pkv_strerror() turns a code into text; PKV_ERR_HIP also records the HIP
 *     error string, available from pkv_last_error().
 *   - Entry points that take a stream enqueue work on it and return without
 *     synchronising. The library keeps no pointer after it returns.
 *   - The library allocates no device memory in these calls; the caller passes
 *     a workspace sized by pkv_workspace_bytes().
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK               0
#define PKV_ERR_INVALID     -1  /* null pointer, bad size, Hq % Hkv != 0, stride or alignment error */
#define PKV_ERR_UNSUPPORTED -2  /* head_dim not 128/256, q_len out of range, too many query rows per KV head, ... */
#define PKV_ERR_WORKSPACE   -3  /* workspace smaller than pkv_workspace_bytes() */
#define PKV_ERR_HIP         -4  /* a HIP runtime call or launch failed */

#define PKV_OUT_F32  0
#define PKV_OUT_BF16 1

/* Element type of the K/V caches (pkv_decode_params.kv_dtype). */
#define PKV_KV_BF16 0
#define PKV_KV_FP8_E4M3 1   /* OCP FP8 E4M3 (E4M3FN) codes; value = decoded code * k_scale / v_scale */

/* Problem description. Layout is fixed: 10 x int32, 7 x int64, float, 3 x int32,
 * 2 x float (120 bytes, natural alignment). */
typedef struct pkv_decode_params {
  int32_t num_seqs;          /* sequences in the batch, >= 1 */
  int32_t q_len;             /* new query rows per sequence, 1..16 (1 = decode; prefill: up to 2^24) */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0; (Hq / Hkv) * q_len <= 128. q_len 1 with
                                Hq / Hkv <= 8 runs on the decode kernel; several rows with
                                (Hq / Hkv) * q_len <= 32, D 256 and splits of more than 256
                                tokens on the few-row MFMA kernel; everything else on the
                                tiled MFMA kernel */
  int32_t head_dim;          /* D: 128 or 256 */
  int32_t block_size;        /* tokens per physical page, any value >= 1 (e.g. 16, 784, 832) */
  int32_t max_pages_per_seq; /* row stride of block_table, in entries */
  int32_t max_seq_len;       /* host-known upper bound of seq_lens[b]; <= max_pages_per_seq * block_size */
  int32_t num_pages;         /* physical pages in the pool; table entries outside [0, num_pages) are never dereferenced */
  int32_t num_splits;        /* 0 = planner's choice; > 0 asks for that many splits of the longest sequence */
  int64_t total_tokens;      /* optional planner hint: sum of seq_lens (0 = unknown, assume num_seqs * max_seq_len) */
  int64_t k_stride_page;     /* K cache strides in elements: page, token, KV head; the dim stride is 1 */
  int64_t k_stride_tok;
  int64_t k_stride_head;
  int64_t v_stride_page;     /* V cache strides, same meaning */
  int64_t v_stride_tok;
  int64_t v_stride_head;
  float   scale;             /* softmax scale applied to q . k (e.g. 1/sqrt(D)) */
  int32_t out_dtype;         /* PKV_OUT_F32 or PKV_OUT_BF16 */
  int32_t window;            /* sliding window: the query row at position p sees only the
                                tokens j with p - window < j <= p (the most recent `window`
                                positions, its own included); 0 = the whole context */
  int32_t kv_dtype;          /* PKV_KV_BF16 or PKV_KV_FP8_E4M3 (one byte per element; strides
                                then multiples of 16 elements) */
  float   k_scale;           /* FP8 caches: K = decoded code * k_scale (per tensor, finite, > 0) */
  float   v_scale;           /* FP8 caches: V = decoded code * v_scale; both ignored for bf16 */
} pkv_decode_params;

/* Library version string (static storage). */
const char* pkv_version(void);

/* Text for a PKV_* code (static storage). */
const char* pkv_strerror(int code);

/* Detail of the most recent error on the calling thread (e.g. the HIP error
 * string); empty when none. Static thread-local storage. */
const char* pkv_last_error(void);

/* Host-only check of *p (no HIP call): sizes (num_seqs, num_kv_heads and
 * num_q_heads at most 65535 for the decode and varlen calls), group size, head_dim, q_len,
 * strides (positive, multiples of 8 so every K/V row starts on 16 bytes;
 * block_size <= 2^20 and block_size * token stride below 2^31 elements, else
 * PKV_ERR_UNSUPPORTED), max_seq_len <= 2^30 (else PKV_ERR_UNSUPPORTED) and
 * max_seq_len <= max_pages_per_seq * block_size. Returns PKV_OK or an error. */
int pkv_validate_params(const pkv_decode_params* p);

/* Host-only split plan (no HIP call). With T = 64-token tiles:
 *   span    = max_seq_len, or min(max_seq_len, window + q_len - 1) with a window;
 *   n_tiles = ceil(span / T) (1 when span is 0);
 *   work    = total_tokens, or num_seqs * max_seq_len when total_tokens == 0;
 *             with a window at most num_seqs * span;
 *   c       = max(min_tiles, ceil(Hkv * work / (cu_count * wg_per_cu * T))),
 *             or ceil(n_tiles / num_splits) when num_splits > 0;
 *   c       = clamp(c, 1, min(n_tiles, max_tiles));
 *   *num_splits = ceil(n_tiles / c); *chunk_tokens = c * T.
 * Sequence b with n_b query rows sees tokens [lo_b, L_b), lo_b = 0, or
 * max(0, L_b - n_b + 1 - window) with a window; it uses
 * n_split_b = ceil((L_b - lo_b) / chunk) splits. On the multi-row kernel
 * split s covers [lo_b + s * chunk, min(lo_b + (s + 1) * chunk, L_b)). The
 * single-query split kernel deals the same number of splits out strided:
 * [lo_b, L_b) in blocks of 32 tokens, block k to split k mod n_split_b (at
 * most chunk / 32 blocks per split); see pkv_debug_token_splits. A split
 * never exceeds max_tiles * T tokens (one unrolled window of the split
 * kernel), so a requested num_splits may be raised. cu_count must be >= 1. */
int pkv_plan_splits(const pkv_decode_params* p, int32_t cu_count,
                    int32_t* num_splits, int32_t* chunk_tokens);

/* The planner's constants: tile T, workgroups per CU, minimum and maximum
 * tiles per split. Any pointer may be NULL. */
int pkv_plan_constants(int32_t* tile, int32_t* wg_per_cu, int32_t* min_tiles, int32_t* max_tiles);

/* Bytes of device workspace a call with *p needs when planned for cu_count
 * CUs (cu_count <= 0: the current device's CU count, which initialises HIP).
 * Returns the size (>= 256), or a negative PKV_ERR_* code. */
int64_t pkv_workspace_bytes(const pkv_decode_params* p, int32_t cu_count);

/* Compute units of the current HIP device. */
int pkv_device_cu_count(int32_t* cu_count);

/*
 * The decode-attention call.
 *   q           device bf16 [num_seqs, q_len, Hq, D], contiguous.
 *   k_cache     device bf16 (or FP8 E4M3 codes, kv_dtype), row (page, token, kv_head) at
 *               page * k_stride_page + token * k_stride_tok + kv_head * k_stride_head;
 *               both [P, B, Hkv, D] and views of [P, 2, B, Hkv, D] fit.
 *   v_cache     device bf16, same with the v_* strides.
 *   block_table device int32 [num_seqs, max_pages_per_seq], all of it
 *               allocated: entries past a sequence's last page may be read
 *               (the kernels fetch a split's entries before its length is
 *               known) but are never dereferenced, so they may hold anything.
 *   seq_lens    device int32 [num_seqs]; tokens in the cache for each sequence,
 *               the q_len new ones included. L = 0 gives zeros; a query row
 *               with no visible token gives zeros.
 *   out         device [num_seqs, q_len, Hq, D], float32 or bf16 (out_dtype).
 *   lse         device float32 [num_seqs, q_len, Hq], 4-byte aligned, or NULL
 *               (not written): the natural-log log-sum-exp of each row's
 *               scaled scores, ln sum_j exp(scale * q . K_j) over the tokens
 *               the row sees (FP8: K_j including k_scale), -inf for a row
 *               that sees none. Written wherever out is written. With it a
 *               caller can merge this result with attention over other keys
 *               (the same statistic the split merge combines).
 *   workspace   device, >= pkv_workspace_bytes(p, 0) bytes, 256-byte aligned;
 *               zero all of it once after allocating. Its first 4 bytes are a
 *               sticky error word:
 *                 bit 0: a block-table entry outside [0, num_pages) was met
 *                        and its tokens skipped;
 *                 bit 1: a sequence's cu_seqlens_q rows were inconsistent and
 *                        the sequence was skipped (varlen calls only);
 *                 bit 2: seq_lens[b] exceeded what the call can map (the
 *                        table's max_pages_per_seq * block_size tokens, or the
 *                        splits planned for max_seq_len) and the sequence was
 *                        cut to that range, so its newest tokens were dropped.
 *               Calls that share a workspace must not overlap in time.
 *   stream      hipStream_t (NULL = default stream).
 * q, k_cache, v_cache and out must be 16-byte aligned. No input is written.
 */
int pkv_paged_decode_attention(const pkv_decode_params* p,
                               const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               void* out, float* lse, void* workspace, int64_t workspace_bytes,
                               void* stream);

/*
 * The decode call for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * pkv_paged_decode_attention without a workspace argument. The split partials
 * live in a scratch array inside the library, a
 * file-scope device array of PKV_NOALLOC_SCRATCH_BYTES per GPU, held from the
 * library's first call on that GPU until the process ends; no call allocates
 * or frees memory.
 *   p, q, k_cache, v_cache, block_table, seq_lens, out, lse, stream: as for
 *               pkv_paged_decode_attention (same kernels, same plan, so the
 *               same bits in out).
 *   error_word  device uint32, 4-byte aligned, or NULL: receives the error
 *               bits described for the workspace's error word (ORed in; the
 *               caller zeroes it). With NULL the bits go to the scratch
 *               array's own word, which nobody reads.
 * Returns PKV_ERR_WORKSPACE, before any device work, when the call would need
 * more than PKV_NOALLOC_SCRATCH_BYTES (pkv_workspace_bytes(p, 0) bytes;
 * e.g. 24 query heads, head_dim 256 and q_len 1 fit about 1,300 splits of
 * 512 tokens). Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

int pkv_paged_decode_attention_noalloc(const pkv_decode_params* p,
                                       const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       void* out, float* lse, uint32_t* error_word, void* stream);

/*
 * Varlen multi-row call: sequence b has its own number of new query rows,
 * n_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] in [0, q_len], in one batched
 * call (batched speculative verify). The rows of all sequences are packed:
 *   q            device bf16 [total_q, Hq, D], total_q = cu_seqlens_q[num_seqs];
 *                sequence b's rows are cu_seqlens_q[b] .. cu_seqlens_q[b + 1].
 *   cu_seqlens_q device int32 [num_seqs + 1], non-decreasing, cu_seqlens_q[0] = 0
 *                and total_q <= num_seqs * q_len (the workspace's rows).
 *   out          device [total_q, Hq, D], float32 or bf16.
 *   lse          device float32 [total_q, Hq] or NULL, as for the uniform call.
 * p->q_len is the largest n_b (a host-known bound, like max_seqlen_q of the
 * vendor interface in "DCU page832 attention" §6); (Hq / Hkv) * q_len <= 128.
 * Row i of sequence b sees the tokens j <= seq_lens[b] - n_b + i (the n_b new
 * tokens are the last ones in the cache), as in the uniform call; seq_lens[b]
 * must be >= n_b. All rows run on the MFMA kernel, whatever n_b is. The other
 * arguments, the workspace (pkv_workspace_bytes with the same p) and the
 * error word are as for pkv_paged_decode_attention; a sequence whose row
 * range is inconsistent with the rules above is skipped (its out rows are not
 * written) and sets bit 1 of the error word.
 */
int pkv_paged_varlen_attention(const pkv_decode_params* p,
                               const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* cu_seqlens_q,
                               void* out, float* lse, void* workspace, int64_t workspace_bytes,
                               void* stream);

/* Workspace bytes of a prefill call: the error word's header only. */
#define PKV_PREFILL_WORKSPACE_BYTES 256

/*
 * Chunked-prefill call: sequence b appends n_b = cu_seqlens_q[b + 1] -
 * cu_seqlens_q[b] new tokens (a chunk of a long prompt, whose K/V rows the
 * caller has already written into the paged cache) and each new row attends
 * causally to everything before it, the cached prefix included. "DCU page832
 * attention" §6 serves prompts in chunks of 4096 query rows plus a shorter
 * tail chunk (1 < q <= 4096) with full causal attention over the paged
 * context; this call takes any chunk length. Arguments, packing and the
 * causal rule are those of pkv_paged_varlen_attention, except:
 *   - p->q_len (the largest n_b) may be up to 2^24 and num_seqs * q_len at
 *     most 2^31 - 1; Hq / Hkv <= 128;
 *   - the rows of a sequence are cut into blocks of floor(128 / (Hq / Hkv))
 *     positions; each block runs as one workgroup per KV head over its whole
 *     visible range (no split and no merge), so the output is written
 *     directly and the workspace holds only the error word: it must be
 *     >= PKV_PREFILL_WORKSPACE_BYTES bytes and 256-byte aligned;
 *   - num_splits and total_tokens are ignored.
 * A block-table entry outside [0, num_pages) sets bit 0 of the error word and
 * its tokens are skipped; inconsistent cu_seqlens_q rows set bit 1.
 */
int pkv_paged_prefill_attention(const pkv_decode_params* p,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* cu_seqlens_q,
                                void* out, float* lse, void* workspace, int64_t workspace_bytes,
                                void* stream);

/* Which kernels the last successful attention call on this thread launched,
 * with the split plan, e.g. "decode_valu d256 g6 q1 w512 + lse_merge
 * splits=64 chunk=512 B=784" (for prefill, w is the query positions per
 * workgroup). Split kernels: decode_valu (bf16, q_len 1),
 * decode_mfma (FP8, q_len 1), verify_rows / varlen_rows (several rows, at
 * most 32 per KV head, splits of more than 256 tokens), verify_mfma /
 * varlen_mfma (several rows, otherwise), prefill_mfma. It is this library's run-time marker of the path that ran:
 * "DCU page832 attention" §8 accepts a measurement only when the run's log
 * shows the decode marker of the kernel under test, and §11.3 asks to print
 * that marker and to check that no fallback ran instead. Copies at most
 * len-1 characters plus a terminator; returns the full length. */
int pkv_last_variant(char* buf, int32_t len);

/* Profiling hook: when both are non-NULL, later calls on this thread launch
 * the split kernel with hipExtLaunchKernel so that ev_start and ev_stop
 * (hipEvent_t handles) are stamped at the start and end of its execution.
 * NULL, NULL turns it off. */
int pkv_set_timing_events(void* ev_start, void* ev_stop);

/* Debug: the element offset of every live token row of KV head kv_head, as the
 * kernels compute it (same device code: split range, division by block_size,
 * stride arithmetic), found both ways they find it: from the page table staged
 * in LDS (the multi-row kernel) and from the block-table row in global memory
 * (the single-query split kernel). k_off, v_off: device int64
 * [num_seqs, max_seq_len]; a live token whose page entry is outside
 * [0, num_pages) gets -2, one on which the two ways disagree gets -3; slots
 * j >= L_b get -1. */
int pkv_debug_token_offsets(const pkv_decode_params* p, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t kv_head,
                            int64_t* k_off, int64_t* v_off, void* stream);

/* Debug: every split's token range [begin, end) as the multi-row kernel
 * derives it (contiguous splits, pkv_plan_splits). ranges: device int32
 * [num_seqs, num_splits, 2] for the planned num_splits (pkv_plan_splits with
 * the device CU count); unused splits get [L, L). */
int pkv_debug_split_ranges(const pkv_decode_params* p, const int32_t* seq_lens,
                           int32_t* ranges, void* stream);

/* Debug: which split, and which slot of its window, the single-query split
 * kernel reads each token with (same device code as the kernel: sequence
 * span, split count, strided block mapping, sub-steps per split). p must
 * describe a q_len == 1 call (else PKV_ERR_INVALID). slots: device int32
 * [num_seqs, max_seq_len, 2], (split, slot) per token, where slot
 * j * 32 + r is row r of sub-step j; tokens no split reads (outside
 * [lo_b, L_b)) get (-1, -1). The split plan of the call
 * (pkv_plan_splits with the device CU count) gives num_splits and chunk. */
int pkv_debug_token_splits(const pkv_decode_params* p, const int32_t* seq_lens,
                           int32_t* slots, void* stream);

/* Host self-check of the division by an invariant integer used for
 * token / block_size (Granlund & Montgomery, PLDI 1994, unsigned case): returns
 * the first n in [0, n_max] whose quotient differs from n / divisor, or -1. */
int64_t pkv_magic_div_check(int32_t divisor, int64_t n_max);

/* Reads the workspace error word (synchronous copy to the host). */
int pkv_read_error_word(const void* workspace, int32_t* value);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
