"""Seeded synthetic inputs for paged decode attention.

This module only *builds inputs*: random numbers, bf16 rounding of those
numbers, page pools and block tables. It holds none of the attention
arithmetic, and both the HIP path and the CPU oracle consume what it returns.

Shapes follow the full-attention layers described in "DCU page832 attention"
(luanjiahao.me), §4 (24 query heads, 4 KV heads, head size 256, BF16, cache
``[num_physical_pages, BLOCK_SIZE, 4, 256]`` per component, or the combined
``[num_physical_pages, 2, BLOCK_SIZE, 4, 256]``), with page sizes 784 and 832
from §1-§2 of the same page and 16 as the common default.

Random-number recipe (the pages only say "from a seed"):
  * ``numpy.random.SeedSequence(seed).spawn(6)`` gives six independent PCG64
    streams, used in the fixed order ``[q, k, v, mask, pages, lengths]``.
  * Normal draws are float32 ``standard_normal`` values rounded to bf16 by
    round-to-nearest-even on the bit pattern.
  * Logical K/V are drawn per sequence in token order ``[L, Hkv, D]`` *before*
    paging, so the same seed gives the same logical K/V for every page size.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)      # OCP FP8 E4M3 NaN code
STREAMS = ("q", "k", "v", "mask", "pages", "lengths")


def f32_to_bf16_bits_np(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the 16-bit patterns.

    Finite and infinite inputs only (the rounding add cannot wrap for them)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r
    u >>= 16
    return u.astype(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Same rounding as :func:`f32_to_bf16_bits_np`; uses torch's multithreaded
    float32 -> bfloat16 conversion (also round-to-nearest-even) when present."""
    try:
        import torch
    except ImportError:
        return f32_to_bf16_bits_np(x)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def log_uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn log-uniform in [lo, hi] from the ``lengths`` stream."""
    rng = streams(seed)["lengths"]
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


@dataclasses.dataclass
class DecodeCase:
    q: np.ndarray            # uint16 bf16 bits, [num_seqs, q_len, Hq, D]
    k_cache: np.ndarray      # uint16 bf16 bits, [num_pages, B, Hkv, D] (may be a strided view)
    v_cache: np.ndarray      # same layout as k_cache
    block_table: np.ndarray  # int32 [num_seqs, max_pages]; entries past a sequence's pages are -1
    seq_lens: np.ndarray     # int32 [num_seqs]
    block_size: int
    scale: float             # exactly representable in float32
    logical_k: list          # per sequence: uint16 [L, Hkv, D] in token order (test convenience)
    logical_v: list
    kv_pool: np.ndarray | None = None   # combined [num_pages, 2, B, Hkv, D] when requested
    meta: dict = dataclasses.field(default_factory=dict)
    kv_dtype: str = "bf16"   # "bf16" (uint16 bits) or "fp8_e4m3" (uint8 codes; value = decoded * scale)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_len(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


def _deal_pages(perm: np.ndarray, n_pages: Sequence[int], interleave: bool) -> list:
    """Split a permutation of physical page ids into per-sequence page lists."""
    out = [[] for _ in n_pages]
    if not interleave:
        pos = 0
        for b, n in enumerate(n_pages):
            out[b] = list(perm[pos:pos + n])
            pos += n
        return out
    pos = 0
    for r in range(max(n_pages, default=0)):
        for b, n in enumerate(n_pages):
            if r < n:
                out[b].append(perm[pos])
                pos += 1
    return out


def make_case(
    seed: int,
    seq_lens: Sequence[int],
    *,
    q_len: int = 1,
    num_q_heads: int = 24,
    num_kv_heads: int = 4,
    head_dim: int = 256,
    block_size: int = 16,
    scale: float | None = None,
    pool_factor: float = 1.25,
    pool_pages: int | None = None,
    boost_frac: float = 0.0,
    boost: float = 4.0,
    poison: bool = True,
    combined: bool = False,
    interleave: bool = False,
    extra_table_cols: int = 0,
    kv_dtype: str = "bf16",
) -> DecodeCase:
    """Build one paged decode input.

    ``boost_frac`` scales exactly ``round(boost_frac * L * Hkv)`` logical
    (token, KV head) key rows of each sequence by ``boost`` (a power of two, so
    exact in bf16); this gives the peaked softmax of the long-context workloads.
    With ``poison`` every slot that no sequence owns (unused pages and the tail
    of each last page) holds NaN, and table entries past a sequence's pages
    are -1, so any read outside the live range shows up in the output.

    ``kv_dtype="fp8_e4m3"`` quantises the bf16 K and V draws to OCP FP8 E4M3
    codes with one scale per tensor, amax / 448 as float32 (round to nearest
    even, by torch's float8_e4m3fn conversion).
    """
    seq_lens = [int(x) for x in seq_lens]
    ns, hq, hkv, d, bs = len(seq_lens), num_q_heads, num_kv_heads, head_dim, block_size
    assert hq % hkv == 0 and bs >= 1 and ns >= 1
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    scale = float(np.float32(scale))
    rng = streams(seed)

    q = normal_bf16(rng["q"], (ns, q_len, hq, d))
    logical_k, logical_v = [], []
    for L in seq_lens:
        k = normal_bf16(rng["k"], (L, hkv, d))
        v = normal_bf16(rng["v"], (L, hkv, d))
        if boost_frac > 0.0 and L > 0:
            n_boost = int(round(boost_frac * L * hkv))
            rows = rng["mask"].choice(L * hkv, size=n_boost, replace=False)
            kf = k.reshape(L * hkv, d)
            vals = (kf[rows].astype(np.uint32) << 16).view(np.float32) * np.float32(boost)
            kf[rows] = f32_to_bf16_bits(vals)
        logical_k.append(k)
        logical_v.append(v)

    k_scale = v_scale = 1.0
    if kv_dtype == "fp8_e4m3":
        logical_k, k_scale = _quantize_fp8(logical_k)
        logical_v, v_scale = _quantize_fp8(logical_v)
    elif kv_dtype != "bf16":
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    n_pages = [-(-L // bs) for L in seq_lens]
    total = sum(n_pages)
    if pool_pages is None:
        pool_pages = max(1, math.ceil(pool_factor * total))
    assert pool_pages >= total
    perm = rng["pages"].permutation(pool_pages).astype(np.int32)
    pages = _deal_pages(perm, n_pages, interleave)

    max_pages = max(max(n_pages, default=0), 1) + extra_table_cols
    table = np.full((ns, max_pages), -1, dtype=np.int32)
    fp8 = kv_dtype == "fp8_e4m3"
    if fp8:
        fill = FP8_NAN if poison else np.uint8(0)
    else:
        fill = BF16_NAN if poison else np.uint16(0)
    pool = np.full((pool_pages, 2, bs, hkv, d), fill, dtype=np.uint8 if fp8 else np.uint16)
    for b, L in enumerate(seq_lens):
        table[b, : n_pages[b]] = pages[b]
        # Fill page by page: logical page p holds tokens [p*bs, min((p+1)*bs, L)).
        for p, phys in enumerate(pages[b]):
            lo, hi = p * bs, min((p + 1) * bs, L)
            pool[phys, 0, : hi - lo] = logical_k[b][lo:hi]
            pool[phys, 1, : hi - lo] = logical_v[b][lo:hi]

    if combined:
        k_cache, v_cache, kv_pool = pool[:, 0], pool[:, 1], pool
    else:
        k_cache = np.ascontiguousarray(pool[:, 0])
        v_cache = np.ascontiguousarray(pool[:, 1])
        kv_pool = None
        del pool

    return DecodeCase(
        q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
        seq_lens=np.asarray(seq_lens, dtype=np.int32), block_size=bs, scale=scale,
        logical_k=logical_k, logical_v=logical_v, kv_pool=kv_pool,
        meta=dict(seed=seed, q_len=q_len, hq=hq, hkv=hkv, d=d, block_size=bs,
                  pool_pages=pool_pages, boost_frac=boost_frac, poison=poison,
                  combined=combined, interleave=interleave),
        kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
    )


def _quantize_fp8(rows: list) -> tuple[list, float]:
    """bf16 bit arrays -> OCP FP8 E4M3 codes with one float32 scale, amax / 448."""
    import torch
    vals = [(np.asarray(r, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) for r in rows]
    amax = max((float(np.abs(v).max()) for v in vals if v.size), default=0.0)
    scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    codes = [torch.from_numpy(np.ascontiguousarray(v / np.float32(scale))).to(torch.float8_e4m3fn)
             .view(torch.uint8).numpy().copy() for v in vals]
    return codes, scale


# ---------------------------------------------------------------------------
# Named workloads. Seeds: 1001-1004 for the four decode workloads, 1005 for the
# multi-row verify workload, 1006 for the dense-model control.
# ---------------------------------------------------------------------------

HYBRID_CONTEXTS = (1024, 4096, 16384, 32768)


def single_seq_b16(**kw) -> DecodeCase:
    """Batch 1, q_len 1, 24/4/256, page 16, 512 tokens; 32 pages of a 64-page pool."""
    return make_case(1001, [512], block_size=16, pool_pages=64, **kw)


def hybrid_long_context(context: int, block_size: int = 784, **kw) -> DecodeCase:
    """Batch 1, q_len 1, 24/4/256, 5% of key rows x4, pool 1.25x the pages needed."""
    return make_case(1002, [context], block_size=block_size, boost_frac=0.05, **kw)


def mixed_batch(**kw) -> DecodeCase:
    """16 sequences, lengths log-uniform in [500, 32000], page 784, pages dealt round-robin."""
    lens = log_uniform_lengths(1004, 16, 500, 32000)
    return make_case(1004, lens, block_size=784, interleave=True, **kw)


def spec_verify(context: int = 32768, q_len: int = 16, **kw) -> DecodeCase:
    """Batch 1, 16 causal query rows, 24/4/256, page 784."""
    return make_case(1005, [context], q_len=q_len, block_size=784, **kw)


def pack_varlen(case: DecodeCase, q_lens) -> tuple[np.ndarray, np.ndarray]:
    """Packed query rows [total_q, Hq, D] and cu_seqlens_q [num_seqs + 1] for
    per-sequence row counts q_lens (each <= case.q_len): sequence b keeps the
    first q_lens[b] of its drawn rows."""
    q_lens = [int(x) for x in q_lens]
    assert len(q_lens) == case.num_seqs and all(0 <= n <= case.q_len for n in q_lens)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    rows = [case.q[b, :n] for b, n in enumerate(q_lens)]
    q = np.concatenate(rows, axis=0) if rows else case.q[:0, 0]
    return np.ascontiguousarray(q), cu


def batched_verify(num_seqs: int = 32, max_rows: int = 5, lo: int = 512, hi: int = 2048,
                   **kw) -> tuple[DecodeCase, np.ndarray, np.ndarray]:
    """Batched speculative verify: num_seqs requests with 1..max_rows new rows
    each (four drafted tokens give up to five positions), contexts log-uniform
    in [lo, hi], 24/4/256, page 784, pages dealt round-robin. The row counts
    continue the lengths stream. Returns (case, packed q, cu_seqlens_q)."""
    seed = 1007
    rng = streams(seed)["lengths"]
    u = rng.uniform(math.log(lo), math.log(hi), size=num_seqs)
    lens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    q_lens = rng.integers(1, max_rows + 1, size=num_seqs)
    case = make_case(seed, lens, q_len=max_rows, block_size=784, interleave=True, **kw)
    q, cu = pack_varlen(case, q_lens)
    return case, q, cu


def chunked_prefill(chunk: int = 4096, context: int = 8192, block_size: int = 784,
                    **kw) -> tuple[DecodeCase, np.ndarray, np.ndarray]:
    """One prompt chunk: `chunk` new query rows whose K/V are the last `chunk`
    tokens of a `context`-token cache (the earlier tokens are the prefix that
    previous chunks left), 24/4/256, page 784. The default is the second
    4096-row chunk of an 8192-token prompt. Returns (case, packed q, cu_seqlens_q)."""
    case = make_case(1011, [context], q_len=chunk, block_size=block_size, boost_frac=0.05, **kw)
    q, cu = pack_varlen(case, [chunk])
    return case, q, cu


def attention_flops(seq_lens, q_lens, num_q_heads: int, head_dim: int, *, window: int = 0) -> int:
    """Algorithmic flops of a causal multi-row call: 4 * D per (query row, query
    head, visible token), i.e. 2 * D for q.k and 2 * D for p.v. Row i of a
    sequence with n new rows and L tokens sees L - n + i + 1 tokens (at most
    `window` of them with a sliding window)."""
    total = 0
    for L, n in zip(np.asarray(seq_lens, dtype=np.int64).tolist(), np.asarray(q_lens, dtype=np.int64).tolist()):
        vis = np.arange(L - n + 1, L + 1, dtype=np.int64)
        vis = np.maximum(vis, 0)
        if window > 0:
            vis = np.minimum(vis, window)
        total += int(vis.sum())
    return int(4 * head_dim * num_q_heads * total)


def dense_control(context: int = 32768, **kw) -> DecodeCase:
    """Batch 1, q_len 1, 32 query heads, 8 KV heads, head_dim 128, page 16."""
    return make_case(1006, [context], num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=16, **kw)


def kv_read_bytes(seq_lens, num_kv_heads: int, head_dim: int, elem_bytes: int = 2, *, window: int = 0,
                  rows=None) -> int:
    """Algorithmic K+V bytes one call must read: every token some query row of
    its sequence sees, once. With a sliding window, sequence b's rows (rows[b],
    default 1) see the last min(L_b, window + rows[b] - 1) tokens."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    if window > 0:
        r = np.ones_like(lens) if rows is None else np.asarray(rows, dtype=np.int64)
        lens = np.minimum(lens, window + r - 1)
    return int(2 * int(lens.sum()) * num_kv_heads * head_dim * elem_bytes)
