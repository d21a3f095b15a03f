"""Plain CPU oracle for paged decode attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
product path never imports it, and this module imports nothing from the
product package: the two share no code.

Sources (page titles as they appear on the pages):
  * "DCU page832 attention" (luanjiahao.me, 2026-07-17):
      §1  a token's logical page is ``token // BLOCK_SIZE``, its page offset is
          ``token % BLOCK_SIZE``, and the block table maps the logical page to a
          physical page; K/V stride, KV head and head dim complete the address.
      §4  the cache shape ``[num_physical_pages, BLOCK_SIZE, Hkv, D]`` per
          component (``unbind(1)`` of ``[num_physical_pages, 2, ...]``).
      §5  per key tile: gather K/V through the table, ``score = dot(Q, K) * scale``,
          then an online-softmax update with V; the causal range is kept.
      §7  q=1 decode reads every logical page of the sequence and skips none.
  * "vLLM 下双卡 Radeon 上的混合 SSM 解码速率" (cadamcat.github.io), the
    paragraph on the upstream split-KV patch: the KV range of one
    (sequence, KV head) is cut among several workgroups and the pieces are
    reduced afterwards.
  * "Qwen3.8 auf MI350P betreiben", Lektion 3: several verify rows share one
    K/V walk, each row keeps its own causal mask, and partial softmax
    statistics are merged.
  * "如何在单张 RTX 3090 上让 Qwen3.5-27B token 生成速度提升 6 倍": decode
    attention over the most recent 2,048 KV positions only (sliding window),
    and a quantised KV cache (here OCP FP8 E4M3 with per-tensor scales).

What is computed (the plain definition; split-KV is an exact re-association of
it, so the oracle evaluates the definition directly):
    for sequence b, query row i, query head h:
        g   = h // G                        (G = Hq / Hkv, consecutive groups)
        pos = L_b - q_len + i               (bottom-right causal alignment)
        lo  = 0, or max(0, pos - W + 1) with a sliding window W
        s_j = sigma * sum_d q[b,i,h,d] * K_j[d]     for j in [lo, pos]
        out = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s)
with K_j, V_j read through the block table and widened exactly to fp64 (bf16
bits, or FP8 E4M3 codes decoded from the OCP definition times the float32
per-tensor scale), and sigma = float64(float32(scale)), the value the kernel
receives. Varlen calls apply this to each sequence's own rows (q_len = n_b);
so do chunked-prefill calls, whose n_b new rows may number in the thousands
("DCU page832 attention" §6 serves prompts in chunks of 4096 rows and a
shorter tail chunk, each as causal attention over the paged context).

Readings where the pages are silent:
GQA head h uses KV head h // G; a sequence with L = 0 yields zeros; the
multi-row causal window is bottom-right aligned (row i sees j <= L - q_len + i);
a sliding window counts positions and includes the row's own token.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against brute force, closed forms, invariants, a library routine, and the
worked integers the pages print.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "fp8_e4m3_to_f64", "kv_widen", "page_of", "token_offsets_ref", "gather_token_rows",
    "kv_head_of", "last_visible", "first_visible", "paged_attention_ref", "paged_attention_varlen_ref",
    "paged_attention_lse_ref", "paged_attention_varlen_lse_ref",
    "partial_stats_ref", "merge_partials_ref", "split_attention_ref", "split_plan_ref", "split_ranges_ref",
    "decode_token_splits_ref",
    "kv_bytes_ref",
]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 (E4M3FN) codes: a sign bit, 4 exponent bits
    with bias 7 and 3 mantissa bits; exponent 0 holds the subnormals
    m / 8 * 2^-6; S.1111.111 is NaN and there is no infinity (largest 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where(c & 0x80, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def kv_widen(kv_dtype: str, scale: float = 1.0):
    """Element decoder of a K or V cache: bf16 bits, or FP8 E4M3 codes times
    the per-tensor scale (as the float32 the kernel receives)."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64
    if kv_dtype == "fp8_e4m3":
        s = float(np.float32(scale))
        return lambda codes: fp8_e4m3_to_f64(codes) * s
    raise ValueError(f"unknown kv_dtype {kv_dtype!r}")


# ---------------------------------------------------------------------------
# Address translation ("DCU page832 attention", §1 and §5).
# ---------------------------------------------------------------------------

def page_of(token: int, block_size: int) -> tuple[int, int]:
    """(logical page, offset in page) of a logical token index."""
    return token // block_size, token % block_size


def token_offsets_ref(block_table, seq_lens, block_size: int, stride_page: int,
                      stride_tok: int, stride_head: int, kv_head: int) -> list:
    """Element offset of every live token's row start, per sequence.

    offset(b, j) = block_table[b, j // B] * stride_page + (j % B) * stride_tok
                   + kv_head * stride_head          (Python integers, no overflow)
    """
    out = []
    for b, L in enumerate(np.asarray(seq_lens).tolist()):
        row = []
        for j in range(int(L)):
            p, o = page_of(j, block_size)
            phys = int(block_table[b][p])
            row.append(phys * stride_page + o * stride_tok + kv_head * stride_head)
        out.append(np.asarray(row, dtype=np.int64))
    return out


def gather_token_rows(cache, table_row, n_tokens: int, block_size: int, kv_head: int,
                      widen=bf16_bits_to_f64) -> np.ndarray:
    """Rows cache[block_table[j // B], j % B, kv_head, :] for j < n_tokens, as fp64."""
    j = np.arange(n_tokens, dtype=np.int64)
    logical_page = j // block_size
    page_offset = j % block_size
    physical_page = np.asarray(table_row, dtype=np.int64)[logical_page]
    return widen(np.asarray(cache)[physical_page, page_offset, kv_head, :])


def _gather_kv(k_cache, v_cache, table_row, L: int, block_size: int, hkv: int, kv_dtype: str,
               k_scale: float, v_scale: float):
    """K and V rows of every KV head of one sequence, decoded to fp64."""
    if kv_dtype == "bf16":   # the plain call (the planted-mistake pins replace gather_token_rows)
        K = [gather_token_rows(k_cache, table_row, L, block_size, g) for g in range(hkv)]
        V = [gather_token_rows(v_cache, table_row, L, block_size, g) for g in range(hkv)]
    else:
        wk, wv = kv_widen(kv_dtype, k_scale), kv_widen(kv_dtype, v_scale)
        K = [gather_token_rows(k_cache, table_row, L, block_size, g, wk) for g in range(hkv)]
        V = [gather_token_rows(v_cache, table_row, L, block_size, g, wv) for g in range(hkv)]
    return K, V


# ---------------------------------------------------------------------------
# Attention by definition.
# ---------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """KV head of query head h: consecutive groups of `group` query heads share
    one KV head (the pages give 24 query / 4 KV heads, group 6, and no order)."""
    return h // group


def last_visible(L: int, q_len: int, i: int) -> int:
    """Last token query row i sees: the q_len new rows are the last q_len
    tokens of the cache (bottom-right alignment); at q_len 1 that is L - 1."""
    return L - q_len + i


def first_visible(pos: int, window: int) -> int:
    """First token a row whose last visible token is pos sees: 0, or with a
    sliding window the start of its most recent `window` positions (the RTX
    3090 page attends to the most recent 2,048 KV positions this way)."""
    return max(0, pos - window + 1) if window > 0 else 0


def _scaled_scores(keys: np.ndarray, qv: np.ndarray, sigma: float) -> np.ndarray:
    """score_j = sigma * dot(q, k_j) (the DCU page, §5)."""
    return sigma * (keys @ qv)


def _softmax_weighted_sum(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s) for one row of scores."""
    if scores.size == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    e = np.exp(scores - scores.max())
    return (e @ values) / e.sum()


def paged_attention_ref(q, k_cache, v_cache, block_table, seq_lens, block_size: int,
                        scale: float, window: int = 0, kv_dtype: str = "bf16", k_scale: float = 1.0,
                        v_scale: float = 1.0) -> np.ndarray:
    """fp64 paged attention for all sequences, query rows and query heads.

    q: uint16 bf16 bits [num_seqs, q_len, Hq, D]; k_cache / v_cache: uint16
    [num_pages, B, Hkv, D] (any strides); block_table: int [num_seqs, max_pages];
    seq_lens: [num_seqs]. Returns float64 [num_seqs, q_len, Hq, D].
    """
    q = np.asarray(q)
    ns, q_len, hq, d = q.shape
    hkv = np.asarray(k_cache).shape[2]
    assert hq % hkv == 0
    G = hq // hkv
    sigma = float(np.float32(scale))
    out = np.zeros((ns, q_len, hq, d), dtype=np.float64)
    for b in range(ns):
        L = int(seq_lens[b])
        if L == 0:
            continue
        assert L >= q_len, "a sequence must hold at least its q_len new tokens"
        K, V = _gather_kv(k_cache, v_cache, block_table[b], L, block_size, hkv, kv_dtype, k_scale, v_scale)
        for i in range(q_len):
            pos = last_visible(L, q_len, i)
            lo = first_visible(pos, window)
            for h in range(hq):
                g = kv_head_of(h, G)
                qv = bf16_bits_to_f64(q[b, i, h])
                s = _scaled_scores(K[g][lo: pos + 1], qv, sigma)
                out[b, i, h] = _softmax_weighted_sum(s, V[g][lo: pos + 1])
    return out


def paged_attention_varlen_ref(q_packed, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens,
                               block_size: int, scale: float, window: int = 0, kv_dtype: str = "bf16",
                               k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Varlen multi-row attention: sequence b owns query rows
    q_packed[cu[b]:cu[b+1]] (n_b of them, [total_q, Hq, D] bf16 bits) and row i
    sees tokens j <= L_b - n_b + i, exactly as a call with q_len = n_b on that
    sequence alone (the vendor interface of the DCU page, §6, passes such rows
    through cu_seqlens_q). Returns float64 [total_q, Hq, D]."""
    q_packed = np.asarray(q_packed)
    cu = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    out = np.zeros((q_packed.shape[0],) + q_packed.shape[1:], dtype=np.float64)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            continue
        out[lo:hi] = paged_attention_ref(q_packed[None, lo:hi], k_cache, v_cache, block_table[b:b + 1],
                                         np.asarray(seq_lens)[b:b + 1], block_size, scale, window, kv_dtype,
                                         k_scale, v_scale)[0]
    return out


def paged_attention_lse_ref(q, k_cache, block_table, seq_lens, block_size: int, scale: float,
                            window: int = 0, kv_dtype: str = "bf16", k_scale: float = 1.0) -> np.ndarray:
    """Log-sum-exp of every row's scaled scores, the softmax normaliser of the
    definition above: lse[b,i,h] = ln sum_j exp(sigma * q[b,i,h,:] . K_j) over
    the row's visible tokens j (natural log), -inf for a row that sees none.
    It is what a caller needs to merge this attention with attention over
    other keys, the same (max, sum) statistic the split merge combines.
    Returns float64 [num_seqs, q_len, Hq]."""
    q = np.asarray(q)
    ns, q_len, hq, _ = q.shape
    hkv = np.asarray(k_cache).shape[2]
    G = hq // hkv
    sigma = float(np.float32(scale))
    lse = np.full((ns, q_len, hq), -np.inf, dtype=np.float64)
    for b in range(ns):
        L = int(seq_lens[b])
        if L == 0:
            continue
        widen = kv_widen(kv_dtype, k_scale)
        K = [gather_token_rows(k_cache, block_table[b], L, block_size, g, widen) for g in range(hkv)]
        for i in range(q_len):
            pos = last_visible(L, q_len, i)
            lo = first_visible(pos, window)
            if pos < lo:
                continue
            for h in range(hq):
                s = _scaled_scores(K[kv_head_of(h, G)][lo: pos + 1], bf16_bits_to_f64(q[b, i, h]), sigma)
                m = float(s.max())
                lse[b, i, h] = m + math.log(float(np.exp(s - m).sum()))
    return lse


def paged_attention_varlen_lse_ref(q_packed, cu_seqlens_q, k_cache, block_table, seq_lens, block_size: int,
                                   scale: float, window: int = 0, kv_dtype: str = "bf16",
                                   k_scale: float = 1.0) -> np.ndarray:
    """paged_attention_lse_ref for packed varlen rows: float64 [total_q, Hq]."""
    q_packed = np.asarray(q_packed)
    cu = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    lse = np.full(q_packed.shape[:2], -np.inf, dtype=np.float64)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            continue
        lse[lo:hi] = paged_attention_lse_ref(q_packed[None, lo:hi], k_cache, block_table[b:b + 1],
                                             np.asarray(seq_lens)[b:b + 1], block_size, scale, window,
                                             kv_dtype, k_scale)[0]
    return lse


# ---------------------------------------------------------------------------
# Split mode: partial softmax statistics and their merge (split-KV paragraph of
# the dual-Radeon page; Lektion 3 of the MI350P page).
# ---------------------------------------------------------------------------

def partial_stats_ref(scores: np.ndarray, values: np.ndarray):
    """(m, Z, A) of one split: m = max s, Z = sum exp(s - m), A = sum exp(s - m) v.

    An empty split returns (-inf, 0, 0).
    """
    if scores.size == 0:
        return -math.inf, 0.0, np.zeros(values.shape[1], dtype=np.float64)
    m = float(scores.max())
    e = np.exp(scores - m)
    return m, float(e.sum()), e @ values


def merge_partials_ref(parts) -> np.ndarray:
    """Merge [(m_s, Z_s, A_s)]: M = max over non-empty splits,
    out = sum e^(m_s - M) A_s / sum e^(m_s - M) Z_s. All-empty gives zeros."""
    live = [(m, z, a) for (m, z, a) in parts if z > 0.0]
    if not live:
        return np.zeros_like(parts[0][2])
    M = max(m for m, _, _ in live)
    num = sum(math.exp(m - M) * a for m, _, a in live)
    den = sum(math.exp(m - M) * z for m, z, _ in live)
    return num / den


def split_attention_ref(q, k_cache, v_cache, block_table, seq_lens, block_size: int,
                        scale: float, ranges, window: int = 0, kv_dtype: str = "bf16", k_scale: float = 1.0,
                        v_scale: float = 1.0) -> np.ndarray:
    """Same result as paged_attention_ref, evaluated split by split and merged.

    ranges[b] is a list of [begin, end) token ranges that partition [0, L_b).
    """
    q = np.asarray(q)
    ns, q_len, hq, d = q.shape
    hkv = np.asarray(k_cache).shape[2]
    G = hq // hkv
    sigma = float(np.float32(scale))
    out = np.zeros((ns, q_len, hq, d), dtype=np.float64)
    for b in range(ns):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K, V = _gather_kv(k_cache, v_cache, block_table[b], L, block_size, hkv, kv_dtype, k_scale, v_scale)
        for i in range(q_len):
            pos = last_visible(L, q_len, i)
            first = first_visible(pos, window)
            for h in range(hq):
                g = kv_head_of(h, G)
                qv = bf16_bits_to_f64(q[b, i, h])
                parts = []
                for (lo, hi) in ranges[b]:
                    lo_vis, hi_vis = max(lo, first), min(hi, pos + 1)
                    if hi_vis <= lo_vis:
                        parts.append(partial_stats_ref(np.zeros(0), V[g][:0]))
                        continue
                    s = _scaled_scores(K[g][lo_vis:hi_vis], qv, sigma)
                    parts.append(partial_stats_ref(s, V[g][lo_vis:hi_vis]))
                out[b, i, h] = merge_partials_ref(parts)
    return out


# ---------------------------------------------------------------------------
# Split plan. The pages do not give the upstream split heuristic; this is the
# plan this library defines, restated here in plain integers so the library's
# planner can be checked against it exactly.
#
#   T          tile of logical tokens; splits are whole tiles from a sequence's
#              first visible token
#   span       = max_seq_len, or min(max_seq_len, window + q_len - 1) with a
#              sliding window (the union of a sequence's rows' windows)
#   n_tiles    = ceil(span / T)
#   work       = total_tokens if given, else num_seqs * max_seq_len; with a
#              window at most num_seqs * span
#   c (tiles)  = ceil(Hkv * work / (cu_count * wg_per_cu * T)), at least min_tiles;
#                a forced split count S_f instead gives c = ceil(n_tiles / S_f);
#                then at most n_tiles and at most max_tiles (a split is one
#                window of the split kernel)
#   S          = ceil(n_tiles / c);   chunk = c * T tokens
#   sequence b with n_b query rows sees [lo_b, L_b), lo_b = 0, or
#   max(0, L_b - n_b + 1 - window) with a window; it uses
#   S_b = ceil((L_b - lo_b) / chunk) splits and split s covers
#   [lo_b + s * chunk, min(lo_b + (s + 1) * chunk, L_b)).
#   The single-query kernel deals the same S_b splits out strided instead:
#   [lo_b, L_b) in blocks of 32 tokens, block k to split k mod S_b, where it
#   is the (k div S_b)-th block of that split (window slots of 32 tokens).
#   The merge is exact for any partition of the tokens, so only the grouping
#   (hence the rounding order) differs; the mapping itself is index work.
# ---------------------------------------------------------------------------

def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def split_plan_ref(num_seqs: int, num_kv_heads: int, max_seq_len: int, block_size: int,
                   cu_count: int, *, total_tokens: int = 0, forced_splits: int = 0,
                   tile: int = 64, wg_per_cu: int = 1, min_tiles: int = 1,
                   max_tiles: int = 8, window: int = 0, q_len: int = 1) -> tuple[int, int]:
    """Return (S, chunk_tokens). block_size does not enter the plan."""
    span = min(max_seq_len, window + q_len - 1) if window > 0 else max_seq_len
    n_tiles = max(1, _cdiv(span, tile))
    if forced_splits > 0:
        c = _cdiv(n_tiles, forced_splits)
    else:
        work = total_tokens if total_tokens > 0 else num_seqs * max_seq_len
        if window > 0:
            work = min(work, num_seqs * span)
        target = max(1, cu_count * wg_per_cu)
        c = max(min_tiles, _cdiv(num_kv_heads * work, target * tile))
    c = max(1, min(c, n_tiles, max_tiles))
    return _cdiv(n_tiles, c), c * tile


def split_ranges_ref(seq_lens, num_splits: int, chunk: int, window: int = 0, rows: int = 1) -> np.ndarray:
    """[num_seqs, num_splits, 2] array of [begin, end); unused splits are [L, L).
    With a window, sequence b's splits start at max(0, L - rows + 1 - window)."""
    seq_lens = [int(x) for x in np.asarray(seq_lens).tolist()]
    r = np.zeros((len(seq_lens), num_splits, 2), dtype=np.int32)
    for b, L in enumerate(seq_lens):
        first = max(0, L - rows + 1 - window) if window > 0 else 0
        for s in range(num_splits):
            lo = min(first + s * chunk, L)
            hi = min(first + (s + 1) * chunk, L)
            r[b, s] = (lo, hi)
    return r


def decode_token_splits_ref(seq_lens, num_splits: int, chunk: int, window: int = 0,
                            max_seq_len: int | None = None, block: int = 32) -> np.ndarray:
    """[num_seqs, max_seq_len, 2] int32: (split, window slot) of every token the
    single-query kernel reads; (-1, -1) outside the sequence's visible range.
    Written token by token from the rule above: offset u = t - lo_b, block
    k = u // block, split k % S_b, slot (k // S_b) * block + u % block."""
    seq_lens = [int(x) for x in np.asarray(seq_lens).tolist()]
    width = max(seq_lens + [1]) if max_seq_len is None else max(int(max_seq_len), 1)
    r = np.full((len(seq_lens), width, 2), -1, dtype=np.int32)
    for b, L in enumerate(seq_lens):
        lo = max(0, L - window) if window > 0 else 0
        S_b = _cdiv(L - lo, chunk)
        assert S_b <= num_splits, "the plan covers every visible token"
        for t in range(lo, L):
            u = t - lo
            k = u // block
            r[b, t] = (k % S_b, (k // S_b) * block + u % block)
    return r


def kv_bytes_ref(seq_lens, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """K and V bytes one call must read: every live (token, KV head) row once, K and V."""
    return 2 * sum(int(x) for x in np.asarray(seq_lens).tolist()) * num_kv_heads * head_dim * elem_bytes
