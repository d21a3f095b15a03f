"""GPU parity of the multi-row (speculative verify) path, q_len in [2, 16]: the
MFMA split kernel plus the LSE merge, against the fp64 oracle through the C ABI."""
import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import assert_matches_oracle, log, ref_without_tokens, run_gpu, to_device
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def oracle_out(case):
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale)


def test_spec_verify_16_rows_32k_page784():
    log("case: verify, 16 causal rows, 24/4/256, page 784, context 32768")
    case = W.spec_verify()
    assert_matches_oracle(run_gpu(case), oracle_out(case), "verify q16 L32768")


@pytest.mark.parametrize("ql,hq,hkv,d,bs,lens", [
    (2, 24, 4, 256, 784, [1000]),
    (3, 24, 4, 256, 16, [17, 300]),
    (5, 12, 1, 256, 7, [5, 64, 129]),
    (16, 24, 4, 256, 832, [16, 600]),
    (16, 8, 1, 128, 16, [2048]),
    (4, 32, 8, 128, 16, [777, 31]),
    (8, 16, 2, 256, 1, [200]),
    (16, 4, 4, 256, 784, [2500]),
    # 65 to 84 rows per KV head: five or six row tiles of 16, the last one partly filled.
    (13, 24, 4, 256, 784, [3000]),
    (10, 16, 2, 256, 16, [900, 33]),
    (11, 12, 2, 256, 7, [40, 11]),
    (14, 24, 4, 256, 784, [1200]),
])
def test_verify_shapes(ql, hq, hkv, d, bs, lens):
    log(f"case: verify q_len {ql}, {hq}/{hkv}/{d}, page {bs}, lengths {lens}")
    case = W.make_case(900 + ql + d + bs, lens, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=bs, interleave=True, boost_frac=0.05)
    assert_matches_oracle(run_gpu(case), oracle_out(case), f"q{ql} {hq}/{hkv}/{d} B{bs}")


def test_verify_page_sizes_bitwise():
    outs = []
    for bs in (784, 832, 16):
        log(f"case: verify q16 context 4100 page {bs}")
        case = W.make_case(950, [4100], q_len=16, block_size=bs, boost_frac=0.05)
        outs.append(run_gpu(case))
    assert_matches_oracle(outs[0], oracle_out(case), "verify layouts")
    np.testing.assert_array_equal(outs[1], outs[0])
    np.testing.assert_array_equal(outs[2], outs[0])


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_verify_forced_splits(splits):
    log(f"case: verify q16 context 8000 page 784, {splits} splits")
    case = W.make_case(951, [8000], q_len=16, block_size=784)
    assert_matches_oracle(run_gpu(case, num_splits=splits), oracle_out(case), f"verify S={splits}")


def test_verify_rows_match_decode_of_shorter_prefix():
    # Row i of a verify call sees the first L - q_len + i + 1 tokens; a decode
    # call on that prefix computes the same quantity with the other kernel.
    log("case: verify rows vs decode calls on prefixes")
    L, ql = 3000, 6
    case = W.make_case(952, [L], q_len=ql, block_size=784, boost_frac=0.05)
    multi = run_gpu(case)
    for i in range(ql):
        c1 = W.make_case(952, [L], q_len=ql, block_size=784, boost_frac=0.05)
        c1.q = np.ascontiguousarray(case.q[:, i:i + 1])
        c1.seq_lens = np.array([L - ql + i + 1], np.int32)
        single = run_gpu(c1)
        assert np.abs(multi[:, i] - single[:, 0]).max() <= 2e-3


def test_verify_mixed_batch_and_empty():
    log("case: verify q4 batch with an empty sequence, page 784")
    case = W.make_case(953, [0, 4, 1500, 9000], q_len=4, block_size=784, interleave=True)
    got = run_gpu(case)
    assert np.all(got[0] == 0.0)
    assert_matches_oracle(got, oracle_out(case), "verify batch")


def test_verify_repeat_bitwise_and_bf16_out():
    import torch
    log("case: verify repeat + bf16 out")
    case = W.make_case(954, [5000], q_len=16, block_size=784)
    a, b = run_gpu(case), run_gpu(case)
    np.testing.assert_array_equal(a, b)
    b16 = run_gpu(case, out_dtype=torch.bfloat16).astype(np.float32)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(b16), W.f32_to_bf16_bits(a.astype(np.float32)))


@pytest.mark.parametrize("ql", [1, 16])
def test_late_dominant_keys_move_the_softmax_reference(ql):
    # Keys scaled x16 (exact in bf16) at tokens deep inside a split: many rows
    # see their running max jump by far more than 2^8 after the accumulator
    # already holds earlier tokens, so the rescale of that accumulator must run.
    log(f"case: q_len {ql}, late dominant keys, 1500 tokens, page 784, forced 512-token splits")
    case = W.make_case(956, [1500], q_len=ql, block_size=784)
    for t in (400, 470, 1100, 1490):
        page, off = int(case.block_table[0, t // 784]), t % 784
        rows = case.k_cache[page, off].astype(np.uint32) << 16
        case.k_cache[page, off] = W.f32_to_bf16_bits(rows.view(np.float32) * np.float32(16.0))
    assert_matches_oracle(run_gpu(case, num_splits=1), oracle_out(case), f"late keys q{ql}")
    assert_matches_oracle(run_gpu(case), oracle_out(case), f"late keys q{ql} planned")


@pytest.mark.parametrize("splits", [1, 3])
def test_invalid_table_entry_is_skipped_and_flagged(splits):
    import torch
    import paged_kv_cache_08_amd as P
    # Page 8 (tokens 128..143) points outside the pool: bit 0 of the error word
    # is set and every row attends to all of its tokens but those 16.
    log(f"case: verify q8 on 200 tokens, page 16, one out-of-range entry, {splits} splits")
    case = W.make_case(960 + splits, [200], q_len=8, block_size=16, poison=False)
    q, k, v, table, lens = to_device(case)
    table[0, 8] = case.num_pages + 3
    p = P.make_params(q, k, v, table, 16, case.scale, max_seq_len=200, num_splits=splits)
    ws = H.guarded(P.workspace_bytes(p, 0), torch.uint8, fill=0)
    out = P.paged_decode_attention(q, k, v, table, lens, 16, case.scale, max_seq_len=200, num_splits=splits,
                                   workspace=ws)
    torch.cuda.synchronize()
    assert P.read_error_word(ws) & 1
    drop = np.zeros(200, bool)
    drop[128:144] = True
    ref = ref_without_tokens(case, 0, case.q[0], list(range(8)), drop)
    assert_matches_oracle(out[0].cpu().numpy().astype(np.float64), ref, f"verify without page 8 S={splits}")
