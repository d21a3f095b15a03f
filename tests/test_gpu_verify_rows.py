"""GPU parity of calls with a few query rows per sequence (at most 32 rows per
KV head: G x rows) and splits of 256 tokens or more, which run on the
single-query MFMA kernel's structure with two 16-row tiles and per-row causal
bounds (variants verify_rows / varlen_rows), against the fp64 oracle, through
the C ABI. Every case checks that this kernel ran."""
import dataclasses

import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import assert_matches_oracle, log, ref_without_tokens, run_gpu, run_gpu_varlen
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def oracle_out(case, window=0):
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale, window=window, **H.oracle_kv(case))


def oracle_varlen(case, q, cu):
    return O.paged_attention_varlen_ref(q, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                        case.block_size, case.scale)


def ran(name):
    import paged_kv_cache_08_amd as P
    v = P.last_variant()
    assert v.startswith(name), v
    return v


@pytest.mark.parametrize("ql", [2, 3, 4, 5])
def test_rows_20k_page784(ql):
    log(f"case: verify q_len {ql}, 24/4/256, page 784, context 20000")
    case = W.make_case(1300 + ql, [20000], q_len=ql, block_size=784, boost_frac=0.05)
    got = run_gpu(case)
    ran("verify_rows")
    assert_matches_oracle(got, oracle_out(case), f"rows q{ql}")


def test_rows_window():
    # Eight sequences, so that the plan over their windows still gives splits of 256+ tokens.
    log("case: verify q_len 4, window 2048, 8 sequences of 2100..20000 tokens, page 784")
    case = W.make_case(1310, [20000, 2500, 9000, 2100, 15000, 4000, 7000, 3000], q_len=4, block_size=784,
                       interleave=True, boost_frac=0.05)
    got = run_gpu(case, window=2048)
    ran("verify_rows")
    assert_matches_oracle(got, oracle_out(case, window=2048), "rows window")


def test_rows_fp8():
    log("case: verify q_len 4, FP8 K/V, context 20000, page 784")
    case = W.make_case(1311, [20000], q_len=4, block_size=784, boost_frac=0.05, kv_dtype="fp8_e4m3")
    got = run_gpu(case)
    ran("verify_rows")
    assert_matches_oracle(got, oracle_out(case), "rows fp8")


def test_rows_batch_with_empty_and_short_sequences():
    log("case: verify q_len 4, lengths [0, 5, 1500, 20000], page 784")
    case = W.make_case(1312, [0, 5, 1500, 20000], q_len=4, block_size=784, interleave=True, boost_frac=0.05)
    got = run_gpu(case)
    ran("verify_rows")
    assert np.all(got[0] == 0.0)
    assert_matches_oracle(got, oracle_out(case), "rows batch")


def test_rows_single_split():
    log("case: verify q_len 3, 400 tokens, one split of 448 tokens, page 16")
    case = W.make_case(1313, [400], q_len=3, block_size=16, boost_frac=0.05)
    got = run_gpu(case, num_splits=1)
    v = ran("verify_rows")
    assert "splits=1" in v, v
    assert_matches_oracle(got, oracle_out(case), "rows one split")


def test_rows_page_sizes_bitwise():
    outs = []
    for bs in (784, 832, 16):
        log(f"case: verify q_len 4, context 20000, page {bs}")
        case = W.make_case(1314, [20000], q_len=4, block_size=bs, boost_frac=0.05)
        outs.append(run_gpu(case))
        ran("verify_rows")
    assert_matches_oracle(outs[0], oracle_out(case), "rows layouts")
    np.testing.assert_array_equal(outs[1], outs[0])
    np.testing.assert_array_equal(outs[2], outs[0])


def test_rows_repeat_bitwise_and_bf16_out():
    import torch
    log("case: verify q_len 5, context 20000, repeat + bf16 out")
    case = W.make_case(1315, [20000], q_len=5, block_size=784)
    a, b = run_gpu(case), run_gpu(case)
    ran("verify_rows")
    np.testing.assert_array_equal(a, b)
    b16 = run_gpu(case, out_dtype=torch.bfloat16).astype(np.float32)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(b16), W.f32_to_bf16_bits(a.astype(np.float32)))


def test_varlen_rows():
    log("case: varlen rows [1, 5, 0, 3], lengths [20000, 9000, 500, 3000], page 784")
    case = W.make_case(1316, [20000, 9000, 500, 3000], q_len=5, block_size=784, interleave=True,
                       boost_frac=0.05)
    q, cu = W.pack_varlen(case, [1, 5, 0, 3])
    got, _ = run_gpu_varlen(case, q, cu)
    ran("varlen_rows")
    assert_matches_oracle(got, oracle_varlen(case, q, cu), "varlen rows")


def test_varlen_rows_inconsistent_row_counts_are_flagged_and_skipped():
    import torch
    import paged_kv_cache_08_amd as P
    # Sequence 1 claims 5 rows with max_q_len 4: skipped (its out rows keep
    # their contents), bit 1 of the error word set, the others computed.
    log("case: varlen rows [3, 5, 2] with max_q_len 4, lengths [20000, 9000, 13000]")
    case = W.make_case(1317, [20000, 9000, 13000], q_len=16, block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [3, 5, 2])
    full = H.guarded((q.shape[0] + 4, q.shape[1], q.shape[2]), torch.float32, fill=7.0)
    got, ws = run_gpu_varlen(case, q, cu, max_q_len=4, out=full[:q.shape[0]])
    ran("varlen_rows")
    ref = oracle_varlen(case, q, cu)
    assert P.read_error_word(ws) & 2
    assert_matches_oracle(got[0:3], ref[0:3], "seq 0")
    assert_matches_oracle(got[8:10], ref[8:10], "seq 2")
    assert np.all(got[3:8] == 7.0)
    assert bool(torch.all(full[q.shape[0]:] == 7.0))


def test_varlen_rows_invalid_table_entry_is_skipped_and_flagged():
    import paged_kv_cache_08_amd as P
    # Sequence 1's page 2 (tokens 32..47, page 16) points outside the pool:
    # bit 0 is set, sequence 1's rows skip those tokens, sequence 0 is untouched.
    log("case: varlen rows [3, 4], lengths [9000, 3000], page 16, one out-of-range entry")
    case = W.make_case(1318, [9000, 3000], q_len=4, block_size=16, poison=False)
    q, cu = W.pack_varlen(case, [3, 4])
    bad = case.block_table.copy()
    bad[1, 2] = case.num_pages + 1
    case_bad = dataclasses.replace(case, block_table=bad)
    got, ws = run_gpu_varlen(case_bad, q, cu)
    ran("varlen_rows")
    assert P.read_error_word(ws) & 1
    assert_matches_oracle(got[:3], oracle_varlen(case, q, cu)[:3], "sequence 0")
    drop = np.zeros(3000, bool)
    drop[32:48] = True
    assert_matches_oracle(got[3:], ref_without_tokens(case, 1, q[3:], [0, 1, 2, 3], drop),
                          "sequence 1 without page 2")


@pytest.mark.parametrize("hq,hkv,ql,ctx", [(32, 4, 4, 20000), (32, 2, 2, 40000), (8, 4, 16, 20000)])
def test_rows_32_rows_per_kv_head(hq, hkv, ql, ctx):
    # G x rows = 32: both 16-row tiles full (8 heads x 4 rows, 16 x 2, 2 x 16);
    # contexts long enough for splits of more than 256 tokens.
    log(f"case: verify {hq}/{hkv}/256, q_len {ql}, context {ctx}, page 784")
    case = W.make_case(1320 + hq + ql, [ctx], q_len=ql, num_q_heads=hq, num_kv_heads=hkv, block_size=784,
                       boost_frac=0.05)
    got = run_gpu(case)
    ran("verify_rows")
    assert_matches_oracle(got, oracle_out(case), f"rows {hq}/{hkv} q{ql}")


@pytest.mark.parametrize("splits", [40, 60])
def test_rows_forced_splits(splits):
    log(f"case: verify q_len 3, lengths [20000, 700, 3], {splits} forced splits")
    case = W.make_case(1330 + splits, [20000, 700, 3], q_len=3, block_size=784, interleave=True, boost_frac=0.05)
    got = run_gpu(case, num_splits=splits)
    ran("verify_rows")
    assert_matches_oracle(got, oracle_out(case), f"rows S={splits}")


def test_varlen_rows_window_fp8():
    # Eight sequences, so that the plan over their windows gives splits of more than 256 tokens.
    lens = [20000, 9000, 3000, 2500, 15000, 4000, 7000, 2100]
    rows = [2, 4, 1, 3, 0, 4, 2, 1]
    log(f"case: varlen rows {rows}, FP8 K/V, window 2048, lengths {lens}, page 784")
    case = W.make_case(1340, lens, q_len=4, block_size=784, interleave=True, boost_frac=0.05,
                       kv_dtype="fp8_e4m3")
    q, cu = W.pack_varlen(case, rows)
    got, _ = run_gpu_varlen(case, q, cu, window=2048)
    ran("varlen_rows")
    ref = O.paged_attention_varlen_ref(q, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                       case.block_size, case.scale, window=2048, **H.oracle_kv(case))
    assert_matches_oracle(got, ref, "varlen rows window fp8")
