"""Shared helpers for the GPU tests: move a seeded case to the device, run the
HIP path through the C ABI, and the tolerance check against the fp64 oracle."""
import sys

import numpy as np

ATOL = 2e-3        # max |gpu - oracle| over all elements
RTOL = 1e-2        # max |gpu - oracle| / max(|oracle|, REL_FLOOR)
REL_FLOOR = 1e-3


# Guard zones: every device buffer a GPU test hands to the library for writing
# (out, lse, workspace, error word, debug outputs; the binding's own
# allocations go through the same allocator during GPU tests) sits between two
# GUARD_BYTES regions filled with GUARD_BYTE; after each GPU test the regions
# are checked, so a kernel that writes past either end of a buffer fails the
# test that ran it.
GUARD_BYTES = 4096
GUARD_BYTE = 0xA5
_guarded = []


def guarded(shape, dtype, device="cuda", fill=None):
    """A tensor of `shape` / `dtype` inside a guard-zone slab; uninitialised
    (the guard pattern) unless `fill` is given."""
    import torch
    shape = tuple(int(x) for x in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
    slab = torch.full((2 * GUARD_BYTES + n,), GUARD_BYTE, dtype=torch.uint8, device=device)
    t = slab[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)
    if fill is not None:
        t.fill_(fill)
    _guarded.append((slab, n))
    return t


def check_guards():
    """Synchronise and check every guard zone handed out since the last check."""
    import torch
    torch.cuda.synchronize()
    bad = []
    for slab, n in _guarded:
        head = slab[:GUARD_BYTES].cpu().numpy()
        tail = slab[GUARD_BYTES + n:].cpu().numpy()
        if np.any(head != GUARD_BYTE) or np.any(tail != GUARD_BYTE):
            bad.append((n, int(np.count_nonzero(head != GUARD_BYTE)), int(np.count_nonzero(tail != GUARD_BYTE))))
    _guarded.clear()
    assert not bad, f"writes into guard zones (buffer bytes, bytes changed before, after): {bad}"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(arr, device="cuda"):
    import torch
    a = np.ascontiguousarray(arr)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def cache_tensor(arr, device="cuda"):
    """A K/V cache on the device: bf16 bits as bfloat16, FP8 codes as uint8."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    return bf16_tensor(a, device)


def kv_kwargs(case) -> dict:
    """The cache scales for an FP8 case (nothing for bf16)."""
    return dict(k_scale=case.k_scale, v_scale=case.v_scale) if case.kv_dtype == "fp8_e4m3" else {}


def oracle_kv(case) -> dict:
    """The oracle's cache arguments for a case."""
    return dict(kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)


def to_device(case, device="cuda"):
    import torch
    q = bf16_tensor(case.q, device)
    if case.kv_pool is not None:
        pool = cache_tensor(case.kv_pool, device)
        k, v = pool[:, 0], pool[:, 1]
    else:
        k = cache_tensor(case.k_cache, device)
        v = cache_tensor(case.v_cache, device)
    table = torch.from_numpy(np.ascontiguousarray(case.block_table)).to(device)
    lens = torch.from_numpy(np.ascontiguousarray(case.seq_lens)).to(device)
    return q, k, v, table, lens


def run_gpu(case, **kw):
    import torch
    import paged_kv_cache_08_amd as P
    q, k, v, table, lens = to_device(case)
    out = P.paged_decode_attention(q, k, v, table, lens, case.block_size, case.scale,
                                   max_seq_len=case.max_seq_len, **kv_kwargs(case), **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def errors(gpu, ref):
    err = np.abs(gpu - ref)
    rel = err / np.maximum(np.abs(ref), REL_FLOOR)
    return float(err.max(initial=0.0)), float(rel.max(initial=0.0))


def unfloored_rel(gpu, ref):
    """p99 and max of |gpu - ref| / |ref| over elements with ref != 0 (reported only)."""
    nz = ref != 0
    if not np.any(nz):
        return 0.0, 0.0
    r = np.abs(gpu[nz] - ref[nz]) / np.abs(ref[nz])
    return float(np.percentile(r, 99)), float(r.max())


def assert_matches_oracle(gpu, ref, what=""):
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    mx, rel = errors(gpu, ref)
    p99, umax = unfloored_rel(gpu, ref)
    log(f"  {what}: max abs err {mx:.3e}, max rel err {rel:.3e} "
        f"(unfloored relative: p99 {p99:.3e}, max {umax:.3e})")
    assert mx <= ATOL, f"{what}: max abs err {mx} > {ATOL}"
    assert rel <= RTOL, f"{what}: max rel err {rel} > {RTOL}"


def run_gpu_varlen(case, q_packed, cu, *, out=None, workspace=None, **kw):
    """The varlen call through the C ABI on packed rows; returns (out as float64, workspace)."""
    import torch
    import paged_kv_cache_08_amd as P
    _, k, v, table, lens = to_device(case)
    q = bf16_tensor(q_packed)
    cu_t = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).cuda()
    max_q = int(np.diff(cu).max(initial=1)) if kw.get("max_q_len") is None else kw.pop("max_q_len")
    kw.pop("max_q_len", None)
    if workspace is None:
        p = P.make_params(torch.empty((case.num_seqs, max(max_q, 1), q.shape[1], q.shape[2]), device="meta"),
                          k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                          num_splits=kw.get("num_splits", 0))
        workspace = guarded(P.workspace_bytes(p, 0), torch.uint8, fill=0)
    got = P.paged_varlen_attention(q, k, v, table, lens, cu_t, case.block_size, case.scale,
                                   max_q_len=max(max_q, 1), max_seq_len=case.max_seq_len, out=out,
                                   workspace=workspace, **kv_kwargs(case), **kw)
    torch.cuda.synchronize()
    return got.float().cpu().numpy().astype(np.float64), workspace


def ref_without_tokens(case, b, q_rows, rows, drop):
    """fp64 attention of rows `rows` (indices into q_rows [n, Hq, D], the n new
    rows of sequence b) over their causal prefixes with the tokens in the
    boolean mask `drop` removed (a bf16 case; skipped-page checks)."""
    import oracle.paged_attention as O
    n, hq = q_rows.shape[0], q_rows.shape[1]
    hkv = case.k_cache.shape[2]
    G = hq // hkv
    L = int(case.seq_lens[b])
    sig = float(np.float32(case.scale))
    out = np.zeros((len(rows), hq, q_rows.shape[2]))
    for r, i in enumerate(rows):
        pos = L - n + i
        keep = ~np.asarray(drop[:pos + 1])
        for h in range(hq):
            K = O.bf16_bits_to_f64(case.logical_k[b][:pos + 1][keep, h // G])
            V = O.bf16_bits_to_f64(case.logical_v[b][:pos + 1][keep, h // G])
            s = sig * (K @ O.bf16_bits_to_f64(q_rows[i, h]))
            e = np.exp(s - s.max())
            out[r, h] = e @ V / e.sum()
    return out


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in bf16 steps between two arrays of bf16 bit patterns (uint16),
    on the monotone ordering of the values (the two zeros coincide)."""
    def order(x):
        x = np.asarray(x, dtype=np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(order(a_bits) - order(b_bits))
