"""GPU parity of sliding-window decode and multi-row calls (each query row sees
only its most recent `window` positions) against the fp64 oracle, through the C
ABI; the window's split ranges against the oracle's plan, bit for bit."""
import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import assert_matches_oracle, log, run_gpu, run_gpu_varlen, to_device

pytestmark = pytest.mark.gpu


def oracle_w(case, window):
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale, window)


def test_decode_window_2048_at_32k():
    log("case: decode, 32768 tokens, window 2048, page 784")
    case = W.hybrid_long_context(32768)
    assert_matches_oracle(run_gpu(case, window=2048), oracle_w(case, 2048), "decode W2048")


@pytest.mark.parametrize("window", [1, 63, 64, 65, 777])
@pytest.mark.parametrize("bs", [784, 16])
def test_decode_window_sizes(window, bs):
    log(f"case: decode, lengths [3000, 40, 1], window {window}, page {bs}")
    case = W.make_case(980 + bs, [3000, 40, 1], block_size=bs, interleave=True, boost_frac=0.05)
    assert_matches_oracle(run_gpu(case, window=window), oracle_w(case, window), f"decode W{window} B{bs}")


@pytest.mark.parametrize("splits", [1, 5, 64])
def test_decode_window_forced_splits(splits):
    log(f"case: decode, 9000 tokens, window 1500, {splits} splits")
    case = W.make_case(983, [9000], block_size=784)
    assert_matches_oracle(run_gpu(case, window=1500, num_splits=splits), oracle_w(case, 1500),
                          f"decode W1500 S={splits}")


def test_verify_window_at_32k_and_narrow_windows():
    log("case: verify q16, 32768 tokens, window 2048; then windows 4 and 20 on 3000 tokens")
    case = W.spec_verify()
    assert_matches_oracle(run_gpu(case, window=2048), oracle_w(case, 2048), "verify W2048")
    small = W.make_case(984, [3000, 700], q_len=16, block_size=784, interleave=True, boost_frac=0.05)
    for window in (4, 20):
        assert_matches_oracle(run_gpu(small, window=window), oracle_w(small, window), f"verify W{window}")


def test_varlen_window():
    log("case: varlen rows [1, 5, 0, 16, 3], window 300, page 16")
    case = W.make_case(985, [700, 1500, 300, 4000, 17], q_len=16, block_size=16, interleave=True)
    q, cu = W.pack_varlen(case, [1, 5, 0, 16, 3])
    got, _ = run_gpu_varlen(case, q, cu, window=300)
    ref = O.paged_attention_varlen_ref(q, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                       case.block_size, case.scale, 300)
    assert_matches_oracle(got, ref, "varlen W300")


def test_window_wider_than_the_context_is_bitwise_the_full_call():
    log("case: decode and verify, window above the context length")
    for ql in (1, 8):
        case = W.make_case(986, [2500, 900], q_len=ql, block_size=784, interleave=True)
        np.testing.assert_array_equal(run_gpu(case, window=2500), run_gpu(case))


def test_window_page_sizes_bitwise():
    outs = []
    for bs in (784, 832, 16):
        log(f"case: decode window 2048, 20000 tokens, page {bs}")
        outs.append(run_gpu(W.make_case(987, [20000], block_size=bs, boost_frac=0.05), window=2048))
    case = W.make_case(987, [20000], block_size=784, boost_frac=0.05)
    assert_matches_oracle(outs[0], oracle_w(case, 2048), "window layouts")
    np.testing.assert_array_equal(outs[1], outs[0])
    np.testing.assert_array_equal(outs[2], outs[0])


@pytest.mark.parametrize("window,forced", [(2048, 0), (300, 3), (1, 0), (40000, 0)])
def test_window_strided_token_splits_bit_exact(window, forced):
    import torch
    import paged_kv_cache_08_amd as P
    log(f"case: strided token splits with window {window}, forced {forced}")
    case = W.make_case(989, [32768, 5000, 2047, 3, 0], block_size=784, interleave=True, poison=False)
    q, k, v, table, lens = to_device(case)
    p = P.make_params(q, k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                      num_splits=forced, window=window)
    S, chunk = P.plan_splits(p, P.device_cu_count())
    r = P.debug_token_splits(p, lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r.cpu().numpy(), O.decode_token_splits_ref(
        case.seq_lens, S, chunk, window=window, max_seq_len=case.max_seq_len))


@pytest.mark.parametrize("ql,window,forced", [(1, 2048, 0), (1, 300, 3), (16, 2048, 0), (4, 1, 0)])
def test_window_split_ranges_bit_exact(ql, window, forced):
    import torch
    import paged_kv_cache_08_amd as P
    log(f"case: split ranges with window {window}, q_len {ql}, forced {forced}")
    case = W.make_case(988, [32768, 5000, 2047, 3], q_len=ql, block_size=784, interleave=True, poison=False)
    q, k, v, table, lens = to_device(case)
    cu = P.device_cu_count()
    p = P.make_params(q, k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                      num_splits=forced, window=window)
    S, chunk = P.plan_splits(p, cu)
    assert (S, chunk) == O.split_plan_ref(p.num_seqs, p.num_kv_heads, p.max_seq_len, p.block_size, cu,
                                          forced_splits=forced, window=window, q_len=ql)
    r = P.debug_split_ranges(p, lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r.cpu().numpy(), O.split_ranges_ref(case.seq_lens, S, chunk, window=window,
                                                                       rows=ql))
