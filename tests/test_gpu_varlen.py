"""GPU parity of the varlen multi-row call (per-sequence query rows through
cu_seqlens_q, batched speculative verify) against the fp64 oracle, through the
C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import assert_matches_oracle, log, ref_without_tokens, run_gpu, run_gpu_varlen
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def oracle_varlen(case, q, cu):
    return O.paged_attention_varlen_ref(q, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                        case.block_size, case.scale)


def test_batched_verify_32_requests():
    log("case: 32 requests, 1..5 rows, contexts 512..2048, 24/4/256, page 784")
    case, q, cu = W.batched_verify()
    got, _ = run_gpu_varlen(case, q, cu)
    assert_matches_oracle(got, oracle_varlen(case, q, cu), "batched verify")


@pytest.mark.parametrize("bs", [784, 16, 7])
def test_mixed_row_counts(bs):
    lens = [700, 1500, 300, 4000, 17, 2, 999]
    rows = [1, 5, 0, 16, 3, 2, 8]
    log(f"case: rows {rows}, lengths {lens}, page {bs}")
    case = W.make_case(970 + bs, lens, q_len=16, block_size=bs, interleave=True, boost_frac=0.05)
    q, cu = W.pack_varlen(case, rows)
    got, _ = run_gpu_varlen(case, q, cu)
    assert_matches_oracle(got, oracle_varlen(case, q, cu), f"mixed rows B{bs}")


@pytest.mark.parametrize("splits", [1, 4, 64])
def test_varlen_forced_splits(splits):
    log(f"case: varlen rows [2, 7, 4], lengths [5000, 800, 2300], {splits} splits")
    case = W.make_case(975, [5000, 800, 2300], q_len=8, block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [2, 7, 4])
    got, _ = run_gpu_varlen(case, q, cu, num_splits=splits)
    assert_matches_oracle(got, oracle_varlen(case, q, cu), f"varlen S={splits}")


def test_equal_rows_match_the_uniform_call_bitwise():
    log("case: varlen with 16 rows each vs the uniform q_len-16 call")
    case = W.make_case(976, [3000, 1200], q_len=16, block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [16, 16])
    got, _ = run_gpu_varlen(case, q, cu)
    uni = run_gpu(case)
    np.testing.assert_array_equal(got, uni.reshape(got.shape))


def test_gqa12_five_rows_and_bf16_out():
    import torch
    # 12 query heads per KV head and five verification positions: 60 rows per KV head.
    log("case: 24 q / 2 KV heads, rows [5, 3, 5, 1], page 784, fp32 and bf16 out")
    case = W.make_case(977, [2048, 1000, 1500, 64], q_len=5, num_q_heads=24, num_kv_heads=2,
                       block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [5, 3, 5, 1])
    got, _ = run_gpu_varlen(case, q, cu)
    ref = oracle_varlen(case, q, cu)
    assert_matches_oracle(got, ref, "gqa12")
    b16, _ = run_gpu_varlen(case, q, cu, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(b16.astype(np.float32)),
                                  W.f32_to_bf16_bits(got.astype(np.float32)))


def test_inconsistent_row_counts_are_flagged_and_skipped():
    import torch
    import paged_kv_cache_08_amd as P
    # Sequence 1 claims 5 rows with max_q_len 4: it is skipped (its out rows
    # keep their contents) and bit 1 of the error word is set; the other
    # sequences are still computed, and nothing past the packed rows is written.
    log("case: varlen with one sequence above max_q_len")
    case = W.make_case(978, [900, 700, 1300], q_len=16, block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [3, 5, 2])
    full = H.guarded((q.shape[0] + 4, q.shape[1], q.shape[2]), torch.float32, fill=7.0)
    got, ws = run_gpu_varlen(case, q, cu, max_q_len=4, out=full[:q.shape[0]])
    ref = oracle_varlen(case, q, cu)
    assert P.read_error_word(ws) & 2
    assert_matches_oracle(got[0:3], ref[0:3], "seq 0")
    assert_matches_oracle(got[8:10], ref[8:10], "seq 2")
    assert np.all(got[3:8] == 7.0)
    assert bool(torch.all(full[q.shape[0]:] == 7.0))


def test_invalid_table_entry_is_skipped_and_flagged():
    import torch
    import paged_kv_cache_08_amd as P
    # Sequence 1's page 2 (tokens 32..47, page 16) points outside the pool:
    # bit 0 is set, sequence 1's rows skip those tokens, sequence 0 is untouched.
    log("case: varlen rows [3, 4], lengths [300, 90], page 16, one out-of-range entry")
    case = W.make_case(979, [300, 90], q_len=4, block_size=16, poison=False)
    q, cu = W.pack_varlen(case, [3, 4])
    bad = case.block_table.copy()
    bad[1, 2] = case.num_pages + 1
    case_bad = dataclasses.replace(case, block_table=bad)
    got, ws = run_gpu_varlen(case_bad, q, cu)
    assert P.read_error_word(ws) & 1
    assert_matches_oracle(got[:3], oracle_varlen(case, q, cu)[:3], "sequence 0")
    drop = np.zeros(90, bool)
    drop[32:48] = True
    assert_matches_oracle(got[3:], ref_without_tokens(case, 1, q[3:], [0, 1, 2, 3], drop), "sequence 1 without page 2")
