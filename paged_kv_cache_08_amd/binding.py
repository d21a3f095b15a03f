"""ctypes binding of the C ABI in include/pkv.h.

Argument marshalling only: every step of the attention runs in the HIP library.
PyTorch supplies device memory and the current stream. There is no fallback:
if ``libpkv.so`` is missing or a call fails, a RuntimeError says so.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_OUT_F32 = 0
PKV_PREFILL_WORKSPACE_BYTES = 256   # prefill calls: the error-word header only
PKV_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024   # the no-allocation call's scratch array per GPU
PKV_OUT_BF16 = 1
PKV_KV_BF16 = 0
PKV_KV_FP8_E4M3 = 1


class DecodeParams(ctypes.Structure):
    """Mirror of ``pkv_decode_params``."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("k_stride_page", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("out_dtype", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


assert ctypes.sizeof(DecodeParams) == 120

_lock = threading.Lock()
_lib = None

_P = ctypes.POINTER(DecodeParams)
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_SIGNATURES = {
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_validate_params": (ctypes.c_int, [_P]),
    "pkv_plan_splits": (ctypes.c_int, [_P, ctypes.c_int32, _i32p, _i32p]),
    "pkv_plan_constants": (ctypes.c_int, [_i32p, _i32p, _i32p, _i32p]),
    "pkv_workspace_bytes": (ctypes.c_int64, [_P, ctypes.c_int32]),
    "pkv_device_cu_count": (ctypes.c_int, [_i32p]),
    "pkv_paged_decode_attention": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                                  _vp]),
    "pkv_paged_decode_attention_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pkv_paged_varlen_attention": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                  ctypes.c_int64, _vp]),
    "pkv_paged_prefill_attention": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                   ctypes.c_int64, _vp]),
    "pkv_last_variant": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int32]),
    "pkv_set_timing_events": (ctypes.c_int, [_vp, _vp]),
    "pkv_debug_token_offsets": (ctypes.c_int, [_P, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp]),
    "pkv_debug_split_ranges": (ctypes.c_int, [_P, _vp, _vp, _vp]),
    "pkv_debug_token_splits": (ctypes.c_int, [_P, _vp, _vp, _vp]),
    "pkv_magic_div_check": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int64]),
    "pkv_read_error_word": (ctypes.c_int, [_vp, _i32p]),
}
EXPORTED = tuple(_SIGNATURES)


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            # torch ships its own HIP runtime (same soname as /opt/rocm's). Load it
            # first so libpkv.so binds to it: one runtime per process, and torch's
            # stream handles are valid in the library's launches.
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                                   "(run `python -m paged_kv_cache_08_amd.build`)")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def check(rc: int, what: str) -> None:
    if rc != PKV_OK:
        L = lib()
        raise RuntimeError(f"{what} failed: {L.pkv_strerror(rc).decode()} ({rc}): {L.pkv_last_error().decode()}")


def version() -> str:
    return lib().pkv_version().decode()


def plan_constants() -> dict:
    vals = [ctypes.c_int32() for _ in range(4)]
    check(lib().pkv_plan_constants(*[ctypes.byref(v) for v in vals]), "pkv_plan_constants")
    return dict(zip(("tile", "wg_per_cu", "min_tiles", "max_tiles"), (v.value for v in vals)))


def validate(p: DecodeParams) -> int:
    return lib().pkv_validate_params(ctypes.byref(p))


def plan_splits(p: DecodeParams, cu_count: int) -> tuple[int, int]:
    s, c = ctypes.c_int32(), ctypes.c_int32()
    check(lib().pkv_plan_splits(ctypes.byref(p), cu_count, ctypes.byref(s), ctypes.byref(c)), "pkv_plan_splits")
    return s.value, c.value


def workspace_bytes(p: DecodeParams, cu_count: int = 0) -> int:
    n = lib().pkv_workspace_bytes(ctypes.byref(p), cu_count)
    if n < 0:
        check(int(n), "pkv_workspace_bytes")
    return int(n)


def device_cu_count() -> int:
    c = ctypes.c_int32()
    check(lib().pkv_device_cu_count(ctypes.byref(c)), "pkv_device_cu_count")
    return c.value


def magic_div_check(divisor: int, n_max: int) -> int:
    return int(lib().pkv_magic_div_check(divisor, n_max))


def last_variant() -> str:
    buf = ctypes.create_string_buffer(512)
    lib().pkv_last_variant(buf, 512)
    return buf.value.decode()


def set_timing_events(ev_start, ev_stop) -> None:
    check(lib().pkv_set_timing_events(ev_start, ev_stop), "pkv_set_timing_events")


# ---------------------------------------------------------------------------
# torch-facing helpers (torch only for memory and streams).
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _alloc(shape, dtype, device, fill=None):
    """Device buffers the binding allocates for the caller (out, workspace,
    debug outputs): uninitialised, or filled with `fill`. A module-level
    function so that tests can put every such buffer between guard zones."""
    torch = _torch()
    if fill is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return torch.full(shape, fill, dtype=dtype, device=device)


def make_params(q, k_cache, v_cache, block_table, block_size: int, scale: float, *, max_seq_len: int,
                num_splits: int = 0, total_tokens: int = 0, out_dtype: int = PKV_OUT_F32,
                window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0) -> DecodeParams:
    """Fill DecodeParams from tensor shapes and strides.

    q: [num_seqs, q_len, Hq, D]; k_cache / v_cache: [num_pages, B, Hkv, D] with
    unit stride on D, bf16, or one byte per element (FP8 E4M3 codes, as uint8 or
    float8_e4m3fn) with per-tensor k_scale / v_scale; block_table:
    [num_seqs, max_pages]."""
    ns, ql, hq, d = q.shape
    P, B, hkv, d2 = k_cache.shape
    assert d2 == d and tuple(v_cache.shape) == tuple(k_cache.shape) and B == block_size
    assert k_cache.stride(-1) == 1 and v_cache.stride(-1) == 1
    p = DecodeParams()
    p.num_seqs, p.q_len, p.num_q_heads, p.num_kv_heads, p.head_dim = ns, ql, hq, hkv, d
    p.block_size = block_size
    p.max_pages_per_seq = block_table.shape[1]
    p.max_seq_len = int(max_seq_len)
    p.num_pages = P
    p.num_splits = int(num_splits)
    p.total_tokens = int(total_tokens)
    p.k_stride_page, p.k_stride_tok, p.k_stride_head = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    p.v_stride_page, p.v_stride_tok, p.v_stride_head = v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)
    p.scale = float(scale)
    p.out_dtype = out_dtype
    p.window = int(window)
    fp8 = k_cache.element_size() == 1
    assert v_cache.element_size() == k_cache.element_size()
    p.kv_dtype = PKV_KV_FP8_E4M3 if fp8 else PKV_KV_BF16
    p.k_scale, p.v_scale = (float(k_scale), float(v_scale)) if fp8 else (1.0, 1.0)
    return p


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, block_size: int, scale: float, *,
                           max_seq_len: int | None = None, total_tokens: int = 0, num_splits: int = 0,
                           out=None, out_dtype=None, workspace=None, stream=None, window: int = 0,
                           k_scale: float = 1.0, v_scale: float = 1.0, lse=None):
    """out[b,i,h,:] = softmax(scale * q[b,i,h,:] . K_j) V_j over the visible tokens of sequence b
    (with window > 0, only the last `window` of them for each row). lse: optional float32
    [num_seqs, q_len, Hq] on the GPU that receives ln sum_j exp(scale * q . K_j) per row.

    q: bf16 [num_seqs, q_len, Hq, D] (contiguous, on the GPU); k_cache / v_cache:
    bf16 [num_pages, B, Hkv, D] (views of a combined [num_pages, 2, B, Hkv, D]
    cache are fine); block_table / seq_lens: int32 on the GPU. max_seq_len is the
    host-known bound of seq_lens (read from the GPU, with a sync, when omitted).
    Returns out ([num_seqs, q_len, Hq, D], float32 unless out_dtype/out say bf16).
    """
    torch = _torch()
    assert q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous()
    assert k_cache.dtype in _KV_DTYPES() and v_cache.dtype == k_cache.dtype
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.is_contiguous() and seq_lens.is_contiguous()
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    if out is None:
        out = _alloc(q.shape, out_dtype or torch.float32, q.device)
    odt = PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32
    assert out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous() and out.shape == q.shape
    p = make_params(q, k_cache, v_cache, block_table, block_size, scale, max_seq_len=max_seq_len,
                    num_splits=num_splits, total_tokens=total_tokens, out_dtype=odt, window=window,
                    k_scale=k_scale, v_scale=v_scale)
    need = workspace_bytes(p, 0)
    if workspace is None:
        workspace = _alloc((need,), torch.uint8, q.device, 0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().pkv_paged_decode_attention(
        ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), _lse_ptr(lse, q.shape[:-1]), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), stream)
    check(rc, "pkv_paged_decode_attention")
    return out


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_table, seq_lens, block_size: int, scale: float,
                                   *, max_seq_len: int, out, total_tokens: int = 0, num_splits: int = 0,
                                   stream=None, window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                                   lse=None, error_word=None):
    """paged_decode_attention through the entry point that allocates nothing:
    the split partials live in the library's scratch array, so there is no
    workspace, and ``out`` (and ``lse``) must be given. error_word: optional
    int32 tensor of one element on the GPU that receives the error bits."""
    torch = _torch()
    assert q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous()
    assert k_cache.dtype in _KV_DTYPES() and v_cache.dtype == k_cache.dtype
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.is_contiguous() and seq_lens.is_contiguous()
    odt = PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32
    assert out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous() and out.shape == q.shape
    p = make_params(q, k_cache, v_cache, block_table, block_size, scale, max_seq_len=max_seq_len,
                    num_splits=num_splits, total_tokens=total_tokens, out_dtype=odt, window=window,
                    k_scale=k_scale, v_scale=v_scale)
    err = None
    if error_word is not None:
        assert error_word.is_cuda and error_word.dtype == torch.int32 and error_word.numel() == 1
        err = error_word.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().pkv_paged_decode_attention_noalloc(
        ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), _lse_ptr(lse, q.shape[:-1]), err, stream)
    check(rc, "pkv_paged_decode_attention_noalloc")
    return out


def _lse_ptr(lse, rows_shape):
    """Device pointer of the optional float32 log-sum-exp output (None: not written)."""
    if lse is None:
        return None
    torch = _torch()
    assert lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
    assert tuple(lse.shape) == tuple(rows_shape), "lse has one float per (query row, head)"
    return lse.data_ptr()


def _KV_DTYPES():
    torch = _torch()
    return (torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


def paged_varlen_attention(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, block_size: int,
                           scale: float, *, max_q_len: int, max_seq_len: int, total_tokens: int = 0,
                           num_splits: int = 0, out=None, out_dtype=None, workspace=None, stream=None,
                           window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0, lse=None):
    """Varlen multi-row call: sequence b's query rows are q[cu_seqlens_q[b]:cu_seqlens_q[b+1]].

    q: bf16 [total_q, Hq, D] packed rows (contiguous, on the GPU); cu_seqlens_q:
    int32 [num_seqs + 1] on the GPU; max_q_len: the largest row count (host
    bound); max_seq_len: host bound of seq_lens. Returns out [total_q, Hq, D];
    lse (optional float32 [total_q, Hq]) receives each row's log-sum-exp.
    """
    torch = _torch()
    assert q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3
    assert cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.is_contiguous()
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.is_contiguous() and seq_lens.is_contiguous()
    ns = seq_lens.shape[0]
    assert cu_seqlens_q.shape[0] == ns + 1 and block_table.shape[0] == ns
    if out is None:
        out = _alloc(q.shape, out_dtype or torch.float32, q.device)
    odt = PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32
    assert out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous() and out.shape == q.shape
    shape4 = torch.empty((ns, int(max_q_len), q.shape[1], q.shape[2]), device="meta")
    p = make_params(shape4, k_cache, v_cache, block_table, block_size, scale, max_seq_len=max_seq_len,
                    num_splits=num_splits, total_tokens=total_tokens, out_dtype=odt, window=window,
                    k_scale=k_scale, v_scale=v_scale)
    need = workspace_bytes(p, 0)
    if workspace is None:
        workspace = _alloc((need,), torch.uint8, q.device, 0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().pkv_paged_varlen_attention(
        ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), cu_seqlens_q.data_ptr(), out.data_ptr(), _lse_ptr(lse, q.shape[:-1]),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    check(rc, "pkv_paged_varlen_attention")
    return out


def paged_prefill_attention(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, block_size: int,
                            scale: float, *, max_q_len: int, max_seq_len: int, out=None, out_dtype=None,
                            workspace=None, stream=None, window: int = 0, k_scale: float = 1.0,
                            v_scale: float = 1.0, lse=None):
    """Chunked prefill: like paged_varlen_attention (packed rows q [total_q, Hq, D],
    cu_seqlens_q, causal rows ending at seq_lens[b]) for any number of new rows
    per sequence; one pass per block of query positions, no split workspace
    (the workspace holds only the 256-byte error-word header). lse (optional
    float32 [total_q, Hq]) receives each row's log-sum-exp."""
    torch = _torch()
    assert q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3
    assert cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.is_contiguous()
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.is_contiguous() and seq_lens.is_contiguous()
    ns = seq_lens.shape[0]
    assert cu_seqlens_q.shape[0] == ns + 1 and block_table.shape[0] == ns
    if out is None:
        out = _alloc(q.shape, out_dtype or torch.float32, q.device)
    odt = PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32
    assert out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous() and out.shape == q.shape
    shape4 = torch.empty((ns, int(max_q_len), q.shape[1], q.shape[2]), device="meta")
    p = make_params(shape4, k_cache, v_cache, block_table, block_size, scale, max_seq_len=max_seq_len,
                    out_dtype=odt, window=window, k_scale=k_scale, v_scale=v_scale)
    if workspace is None:
        workspace = _alloc((PKV_PREFILL_WORKSPACE_BYTES,), torch.uint8, q.device, 0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().pkv_paged_prefill_attention(
        ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), cu_seqlens_q.data_ptr(), out.data_ptr(), _lse_ptr(lse, q.shape[:-1]),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    check(rc, "pkv_paged_prefill_attention")
    return out


def debug_token_offsets(p: DecodeParams, block_table, seq_lens, kv_head: int):
    """Per-token K and V row offsets as the kernels compute them ([num_seqs, max_seq_len] int64;
    -2 for an invalid page entry, -3 where the staged-table and direct-table paths disagree)."""
    torch = _torch()
    shape = (p.num_seqs, max(p.max_seq_len, 1))
    k_off = _alloc(shape, torch.int64, block_table.device)
    v_off = _alloc(shape, torch.int64, block_table.device)
    stream = torch.cuda.current_stream(block_table.device).cuda_stream
    check(lib().pkv_debug_token_offsets(ctypes.byref(p), block_table.data_ptr(), seq_lens.data_ptr(), kv_head,
                                        k_off.data_ptr(), v_off.data_ptr(), stream), "pkv_debug_token_offsets")
    return k_off, v_off


def debug_split_ranges(p: DecodeParams, seq_lens):
    """[num_seqs, S, 2] contiguous split ranges as the multi-row kernel derives them."""
    torch = _torch()
    S, _ = plan_splits(p, device_cu_count())
    r = _alloc((p.num_seqs, S, 2), torch.int32, seq_lens.device)
    stream = torch.cuda.current_stream(seq_lens.device).cuda_stream
    check(lib().pkv_debug_split_ranges(ctypes.byref(p), seq_lens.data_ptr(), r.data_ptr(), stream),
          "pkv_debug_split_ranges")
    return r


def debug_token_splits(p: DecodeParams, seq_lens):
    """[num_seqs, max_seq_len, 2] int32 (split, window slot) with which the single-query
    split kernel reads each token; (-1, -1) for tokens no split reads. q_len must be 1."""
    torch = _torch()
    r = _alloc((p.num_seqs, max(p.max_seq_len, 1), 2), torch.int32, seq_lens.device)
    stream = torch.cuda.current_stream(seq_lens.device).cuda_stream
    check(lib().pkv_debug_token_splits(ctypes.byref(p), seq_lens.data_ptr(), r.data_ptr(), stream),
          "pkv_debug_token_splits")
    return r


def read_error_word(workspace) -> int:
    v = ctypes.c_int32()
    check(lib().pkv_read_error_word(workspace.data_ptr(), ctypes.byref(v)), "pkv_read_error_word")
    return v.value


class PreparedDecode:
    """A decode call whose arguments are checked and marshalled once; ``run()``
    then only crosses into the C library (for tight loops and benchmarks).

    ``run(k_cache, v_cache)`` may swap in another pool with the same shape and
    strides as the one given at construction. With ``cu_seqlens_q`` (int32 on
    the GPU) and ``max_q_len`` the call is the varlen one on packed rows
    q [total_q, Hq, D]; ``prefill=True`` makes it the chunked-prefill call on
    the same packed rows. ``lse`` (float32, one value per query row and head)
    receives each row's log-sum-exp on every run."""

    def __init__(self, q, k_cache, v_cache, block_table, seq_lens, block_size: int, scale: float, *,
                 max_seq_len: int, total_tokens: int = 0, num_splits: int = 0, out=None, workspace=None,
                 stream=None, cu_seqlens_q=None, max_q_len: int | None = None, window: int = 0,
                 k_scale: float = 1.0, v_scale: float = 1.0, prefill: bool = False, lse=None):
        torch = _torch()
        assert q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous()
        assert block_table.is_contiguous() and seq_lens.is_contiguous()
        if out is None:
            out = _alloc(q.shape, torch.float32, q.device)
        odt = PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32
        self.varlen = cu_seqlens_q is not None
        assert self.varlen or not prefill, "prefill calls take packed rows and cu_seqlens_q"
        if self.varlen:
            assert q.dim() == 3 and cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.is_contiguous()
            assert max_q_len is not None and max_q_len >= 1
            shape = torch.empty((block_table.shape[0], max_q_len, q.shape[1], q.shape[2]), device="meta")
        else:
            shape = q
        self.params = make_params(shape, k_cache, v_cache, block_table, block_size, scale, max_seq_len=max_seq_len,
                                  num_splits=num_splits, total_tokens=total_tokens, out_dtype=odt, window=window,
                                  k_scale=k_scale, v_scale=v_scale)
        if not self.varlen:
            check(validate(self.params), "pkv_validate_params")
        need = PKV_PREFILL_WORKSPACE_BYTES if prefill else workspace_bytes(self.params, 0)
        if workspace is None:
            workspace = _alloc((need,), torch.uint8, q.device, 0)
        assert workspace.numel() * workspace.element_size() >= need
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        self.out, self.workspace = out, workspace
        self._shape = (tuple(k_cache.shape), tuple(k_cache.stride()), tuple(v_cache.stride()))
        self._keep = (q, k_cache, v_cache, block_table, seq_lens)
        self._keep = self._keep + (cu_seqlens_q,)
        self._pp = ctypes.byref(self.params)
        self._fixed = (q.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                       _lse_ptr(lse, q.shape[:-1]), workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), stream)
        self.lse = lse
        self._cu = cu_seqlens_q.data_ptr() if self.varlen else None
        self._name = ("pkv_paged_prefill_attention" if prefill else
                      "pkv_paged_varlen_attention" if self.varlen else "pkv_paged_decode_attention")
        self._fn = getattr(lib(), self._name)
        self._k, self._v = k_cache.data_ptr(), v_cache.data_ptr()

    def run_ptrs(self, k_ptr: int, v_ptr: int) -> None:
        """Like run() with raw device pointers of a pool laid out like the original."""
        qp, tp, lp, op, sp, wp, wn, st = self._fixed
        if self._cu is None:
            rc = self._fn(self._pp, qp, k_ptr, v_ptr, tp, lp, op, sp, wp, wn, st)
        else:
            rc = self._fn(self._pp, qp, k_ptr, v_ptr, tp, lp, self._cu, op, sp, wp, wn, st)
        if rc != PKV_OK:
            check(rc, self._name)

    def run(self, k_cache=None, v_cache=None):
        kp, vp = self._k, self._v
        if k_cache is not None:
            assert (tuple(k_cache.shape), tuple(k_cache.stride()), tuple(v_cache.stride())) == self._shape
            kp, vp = k_cache.data_ptr(), v_cache.data_ptr()
        self.run_ptrs(kp, vp)
        return self.out
