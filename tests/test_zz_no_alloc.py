"""The decode entry point that allocates nothing (partials in the library's
scratch array) against the workspace entry point, through the C ABI: the same
bits on consecutive calls of different sizes, the oracle's tolerance, the size
limit and the error word."""
import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import assert_matches_oracle, kv_kwargs, log, oracle_kv, to_device
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _oracle(case):
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale, **oracle_kv(case))


def _both(case, **kw):
    """(workspace call, no-allocation call) outputs of one case, as float64."""
    import torch
    import paged_kv_cache_08_amd as P
    q, k, v, table, lens = to_device(case)
    kw = dict(kw, **kv_kwargs(case))
    ref = P.paged_decode_attention(q, k, v, table, lens, case.block_size, case.scale,
                                   max_seq_len=case.max_seq_len, **kw)
    torch.cuda.synchronize()
    v_ws = P.last_variant()
    out = H.guarded(q.shape, torch.float32, fill=float("nan"))
    err = H.guarded(1, torch.int32, fill=0)
    P.paged_decode_attention_noalloc(q, k, v, table, lens, case.block_size, case.scale,
                                     max_seq_len=case.max_seq_len, out=out, error_word=err, **kw)
    torch.cuda.synchronize()
    assert P.last_variant() == v_ws
    assert int(err.item()) == 0
    return ref.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64), v_ws


# Consecutive calls of different shapes on the one scratch array: it keeps the
# previous call's partials, which the next call must not read.
SEQUENCE = [
    ("L32768 B784 (split kernel, merge kernel)", lambda: W.hybrid_long_context(32768), {}),
    ("L32768 B784 FP8 (MFMA split kernel, merge kernel)",
     lambda: W.hybrid_long_context(32768, kv_dtype="fp8_e4m3"), {}),
    ("mixed batch (merge kernel)", lambda: W.mixed_batch(), "total"),
    ("L4096 B784", lambda: W.hybrid_long_context(4096), {}),
    ("verify q16 L4096 (MFMA kernel, merge kernel)", lambda: W.spec_verify(4096), {}),
    ("L1024 B784", lambda: W.hybrid_long_context(1024), {}),
    ("b1 L512 B16", lambda: W.single_seq_b16(), {}),
]


def test_noalloc_matches_workspace_call_on_consecutive_shapes():
    for name, make, kw in SEQUENCE:
        log(f"case: no-alloc vs workspace call, {name}")
        case = make()
        if kw == "total":
            kw = dict(total_tokens=int(case.seq_lens.sum()))
        ref, got, variant = _both(case, **kw)
        log(f"  variant: {variant}")
        np.testing.assert_array_equal(got, ref)
        assert_matches_oracle(got, _oracle(case), name)


def test_noalloc_twice_in_a_row_second_smaller():
    import torch
    import paged_kv_cache_08_amd as P
    big, small = W.hybrid_long_context(16384), W.make_case(306, [700, 0, 2300], block_size=16, interleave=True)
    outs = []
    for case in (big, small):
        log(f"case: no-alloc call, lengths {case.seq_lens.tolist()}")
        q, k, v, table, lens = to_device(case)
        out = H.guarded(q.shape, torch.float32)
        P.paged_decode_attention_noalloc(q, k, v, table, lens, case.block_size, case.scale,
                                         max_seq_len=case.max_seq_len, out=out)
        outs.append((case, out))
    torch.cuda.synchronize()
    for case, out in outs:
        ref = P.paged_decode_attention(*to_device(case), case.block_size, case.scale, max_seq_len=case.max_seq_len)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref.cpu().numpy())
        assert_matches_oracle(out.cpu().numpy().astype(np.float64), _oracle(case), "consecutive no-alloc")


def test_noalloc_rejects_calls_beyond_its_scratch():
    import torch
    import paged_kv_cache_08_amd as P
    log("case: q_len 16 at 65536 tokens needs more scratch than the library holds")
    q = torch.zeros((1, 16, 24, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 784, 4, 256), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 84), dtype=torch.int32, device="cuda")
    lens = torch.full((1,), 65536, dtype=torch.int32, device="cuda")
    out = H.guarded(q.shape, torch.float32, fill=5.0)
    p = P.make_params(q, k, k, table, 784, 0.0625, max_seq_len=65536)
    assert P.workspace_bytes(p, 0) > P.binding.PKV_NOALLOC_SCRATCH_BYTES
    with pytest.raises(RuntimeError, match="scratch"):
        P.paged_decode_attention_noalloc(q, k, k, table, lens, 784, 0.0625, max_seq_len=65536, out=out)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all()), "a rejected call wrote its output"


def test_noalloc_reports_errors_in_the_callers_word():
    import torch
    import paged_kv_cache_08_amd as P
    log("case: no-alloc call with an out-of-range table entry")
    case = W.make_case(307, [100], block_size=16, poison=False)
    q, k, v, table, lens = to_device(case)
    table[0, 2] = case.num_pages + 5
    out = H.guarded(q.shape, torch.float32)
    err = H.guarded(1, torch.int32, fill=0)
    P.paged_decode_attention_noalloc(q, k, v, table, lens, 16, case.scale, max_seq_len=100, out=out,
                                     error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    ref = P.paged_decode_attention(q, k, v, table, lens, 16, case.scale, max_seq_len=100)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref.cpu().numpy())
