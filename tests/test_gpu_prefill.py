"""GPU parity of the chunked-prefill call (any number of new causal rows per
sequence, blocks of query positions on the MFMA kernel, one pass over the
whole visible range, no split) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests import gpu_helpers as H
from tests.gpu_helpers import (assert_matches_oracle, bf16_tensor, kv_kwargs, log, oracle_kv, ref_without_tokens,
                               run_gpu_varlen, to_device)

pytestmark = pytest.mark.gpu


def run_prefill(case, q_packed, cu, *, workspace=None, out=None, max_q_len=None, **kw):
    """The prefill call on packed rows; returns (out as float64, workspace)."""
    import torch
    import paged_kv_cache_08_amd as P
    _, k, v, table, lens = to_device(case)
    q = bf16_tensor(q_packed)
    cu_t = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).cuda()
    mq = max_q_len if max_q_len is not None else max(int(np.diff(cu).max(initial=1)), 1)
    if workspace is None:
        workspace = H.guarded(P.binding.PKV_PREFILL_WORKSPACE_BYTES, torch.uint8, fill=0)
    got = P.paged_prefill_attention(q, k, v, table, lens, cu_t, case.block_size, case.scale, max_q_len=mq,
                                    max_seq_len=case.max_seq_len, workspace=workspace, out=out,
                                    **kv_kwargs(case), **kw)
    torch.cuda.synchronize()
    assert P.last_variant().startswith("prefill_mfma")
    return got.float().cpu().numpy().astype(np.float64), workspace


def oracle_prefill(case, q, cu, window=0):
    return O.paged_attention_varlen_ref(q, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                        case.block_size, case.scale, window, **oracle_kv(case))


def oracle_rows(case, q, cu, b, rows):
    """Sampled rows of sequence b, one by one: row i of a sequence with n new
    rows sees the first L - n + i + 1 tokens, which is a one-row call on that
    prefix (the causal rule, applied by the oracle's own full call)."""
    n = int(cu[b + 1] - cu[b])
    L = int(case.seq_lens[b])
    out = []
    for i in rows:
        qi = q[None, cu[b] + i: cu[b] + i + 1]
        out.append(O.paged_attention_ref(qi, case.k_cache, case.v_cache, case.block_table[b:b + 1],
                                         np.array([L - n + i + 1]), case.block_size, case.scale,
                                         **oracle_kv(case))[0, 0])
    return np.stack(out)


def test_chunk_4096_of_8192_prompt_sampled_rows():
    # The full-size chunk: 4096 new rows on an 8192-token cache (24/4/256,
    # page 784). Rows around block edges, the first and last rows and a seeded
    # sample are checked one by one against the oracle.
    log("case: prefill chunk 4096 rows, context 8192, 24/4/256, page 784")
    case, q, cu = W.chunked_prefill()
    got, ws = run_prefill(case, q, cu)
    import paged_kv_cache_08_amd as P
    assert P.read_error_word(ws) == 0
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(5)
    rows = sorted({0, 1, 20, 21, 22, 41, 42, 2047, 2048, 4074, 4075, 4094, 4095}
                  | set(rng.integers(0, 4096, size=11).tolist()))
    log(f"  sampled rows {rows}")
    assert_matches_oracle(got[rows], oracle_rows(case, q, cu, 0, rows), "prefill 4096/8192 sampled")


def test_chunk_1024_of_4096_every_row():
    # A mid-size chunk compared in full: 1024 new rows on a 4096-token cache
    # (24/4/256, page 784), every row, head and column against the oracle's
    # whole varlen call (49 blocks of 21 positions, the last one ragged).
    log("case: prefill chunk 1024 rows, context 4096, 24/4/256, page 784, every row")
    case, q, cu = W.chunked_prefill(chunk=1024, context=4096)
    got, ws = run_prefill(case, q, cu)
    import paged_kv_cache_08_amd as P
    assert P.read_error_word(ws) == 0
    assert_matches_oracle(got, oracle_prefill(case, q, cu), "prefill 1024/4096 every row")


@pytest.mark.parametrize("rows,lens,hq,hkv,d,bs", [
    ([200], [1000], 24, 4, 256, 784),                          # 21 positions per block, ragged last block
    ([37, 0, 130, 1, 21, 22], [37, 500, 900, 1, 21, 2100], 24, 4, 256, 16),   # whole prompts, empty, one row
    ([300], [300], 8, 1, 128, 832),                            # group 8: 16 positions per block
    ([150, 64], [1500, 64], 4, 4, 256, 7),                     # group 1: 128 positions per block
    ([100], [2000], 32, 8, 128, 16),                           # dense control heads, group 4
    ([40], [500], 128, 1, 128, 16),                            # group 128: one position per block
])
def test_prefill_shapes(rows, lens, hq, hkv, d, bs):
    log(f"case: prefill rows {rows}, lengths {lens}, {hq}/{hkv}/{d}, page {bs}")
    case = W.make_case(1100 + hq + d + bs, lens, q_len=max(rows), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=bs, interleave=True, boost_frac=0.05)
    q, cu = W.pack_varlen(case, rows)
    got, _ = run_prefill(case, q, cu)
    assert_matches_oracle(got, oracle_prefill(case, q, cu), f"prefill {rows} {hq}/{hkv}/{d} B{bs}")


def test_short_chunks_match_the_varlen_call_bitwise():
    # With at most 21 rows (one block) and a context of at most 512 tokens, the
    # prefill block and a single-split varlen call run the same rows over the
    # same tiles: the results must agree bit for bit.
    log("case: prefill vs varlen (one split), rows [16, 5, 21], lengths [500, 64, 300]")
    case = W.make_case(1120, [500, 64, 300], q_len=21, block_size=784, interleave=True, boost_frac=0.05)
    q, cu = W.pack_varlen(case, [16, 5, 16])
    got, _ = run_prefill(case, q, cu)
    ref, _ = run_gpu_varlen(case, q, cu, num_splits=1)
    np.testing.assert_array_equal(got, ref)
    assert_matches_oracle(got, oracle_prefill(case, q, cu), "prefill = varlen")


def test_page_sizes_give_bitwise_identical_outputs():
    outs = []
    for bs in (784, 832, 16):
        log(f"case: prefill 333 rows, context 2500, page {bs}")
        case = W.make_case(1121, [2500], q_len=333, block_size=bs, boost_frac=0.05)
        q, cu = W.pack_varlen(case, [333])
        outs.append(run_prefill(case, q, cu)[0])
    assert_matches_oracle(outs[0], oracle_prefill(case, q, cu), "prefill layouts")
    np.testing.assert_array_equal(outs[1], outs[0])
    np.testing.assert_array_equal(outs[2], outs[0])


@pytest.mark.parametrize("window", [1, 64, 500, 5000])
def test_prefill_sliding_window(window):
    log(f"case: prefill rows [300, 50, 7], lengths [2000, 400, 7], window {window}")
    case = W.make_case(1122, [2000, 400, 7], q_len=300, block_size=784, interleave=True, boost_frac=0.05)
    q, cu = W.pack_varlen(case, [300, 50, 7])
    got, _ = run_prefill(case, q, cu, window=window)
    assert_matches_oracle(got, oracle_prefill(case, q, cu, window), f"prefill window {window}")


def test_prefill_fp8_cache():
    log("case: prefill rows [200, 90], lengths [1200, 90], FP8 E4M3 K/V, page 784")
    case = W.make_case(1123, [1200, 90], q_len=200, block_size=784, interleave=True, boost_frac=0.05,
                       kv_dtype="fp8_e4m3")
    q, cu = W.pack_varlen(case, [200, 90])
    got, _ = run_prefill(case, q, cu)
    assert_matches_oracle(got, oracle_prefill(case, q, cu), "prefill fp8")


def test_prefill_repeat_bitwise_and_bf16_out():
    import torch
    log("case: prefill 250 rows on 1800 tokens, twice, then bf16 out")
    case = W.make_case(1124, [1800], q_len=250, block_size=16, boost_frac=0.05)
    q, cu = W.pack_varlen(case, [250])
    a, _ = run_prefill(case, q, cu)
    b, _ = run_prefill(case, q, cu)
    np.testing.assert_array_equal(a, b)
    c, _ = run_prefill(case, q, cu, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(c.astype(np.float32)),
                                  W.f32_to_bf16_bits(a.astype(np.float32)))


def test_invalid_table_entry_is_skipped_and_flagged():
    import torch
    import paged_kv_cache_08_amd as P
    # Page 8 (tokens 128..143) points outside the pool: the error word gets
    # bit 0; rows that end before token 128 match the oracle on the intact
    # table, later rows see every token but those 16.
    log("case: prefill 120 rows on 200 tokens, page 16, one out-of-range entry")
    case = W.make_case(1125, [200], q_len=120, block_size=16, poison=False)
    q, cu = W.pack_varlen(case, [120])
    _, k, v, table, lens = to_device(case)
    table[0, 8] = case.num_pages + 3
    ws = H.guarded(256, torch.uint8, fill=0)
    got = P.paged_prefill_attention(bf16_tensor(q), k, v, table, lens,
                                    torch.from_numpy(cu).cuda(), 16, case.scale, max_q_len=120, max_seq_len=200,
                                    workspace=ws)
    torch.cuda.synchronize()
    assert P.read_error_word(ws) & 1
    got = got.cpu().numpy().astype(np.float64)
    # row i ends at token 80 + i
    assert_matches_oracle(got[:48], oracle_prefill(case, q, cu)[:48], "rows before page 8")
    drop = np.zeros(200, bool)
    drop[128:144] = True
    rows = [48, 55, 63, 64, 100, 119]
    assert_matches_oracle(got[rows], ref_without_tokens(case, 0, q, rows, drop), "rows without page 8")


def test_inconsistent_rows_are_flagged_and_skipped():
    import torch
    import paged_kv_cache_08_amd as P
    # Sequence 1 claims 40 rows with max_q_len 30: skipped, bit 1 set, the
    # others computed.
    log("case: prefill rows [25, 40, 10] with max_q_len 30")
    case = W.make_case(1126, [900, 700, 1300], q_len=40, block_size=784, interleave=True)
    q, cu = W.pack_varlen(case, [25, 40, 10])
    out = H.guarded((q.shape[0], q.shape[1], q.shape[2]), torch.float32, fill=7.0)
    got, ws = run_prefill(case, q, cu, max_q_len=30, out=out)
    assert P.read_error_word(ws) & 2
    ref = oracle_prefill(case, q, cu)
    assert_matches_oracle(got[:25], ref[:25], "seq 0")
    assert_matches_oracle(got[65:], ref[65:], "seq 2")
    assert np.all(got[25:65] == 7.0)


def test_chunks_match_the_whole_prompt_bitwise():
    import torch
    import paged_kv_cache_08_amd as P
    # A 2000-token prompt as one call, and as chunks of 700, 800 and 500 rows
    # with the cache length at each chunk's end. A row's result depends only
    # on its own tokens and on the fixed 64-token tile walk from the start
    # (fully masked tiles add exact zeros), not on which block holds it.
    log("case: prompt 2000 as one prefill call vs chunks 700 + 800 + 500, page 784")
    case = W.make_case(1127, [2000], q_len=2000, block_size=784, boost_frac=0.05)
    q_all, cu_all = W.pack_varlen(case, [2000])
    whole, _ = run_prefill(case, q_all, cu_all)
    _, k, v, table, _ = to_device(case)
    parts, start = [], 0
    for n in (700, 800, 500):
        lens = torch.tensor([start + n], dtype=torch.int32, device="cuda")
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        out = P.paged_prefill_attention(bf16_tensor(q_all[start:start + n]), k, v, table, lens, cu,
                                        case.block_size, case.scale, max_q_len=n, max_seq_len=start + n)
        torch.cuda.synchronize()
        parts.append(out.cpu().numpy().astype(np.float64))
        start += n
    np.testing.assert_array_equal(np.concatenate(parts), whole)
    rows = [0, 699, 700, 1499, 1500, 1999]
    assert_matches_oracle(whole[rows], oracle_rows(case, q_all, cu_all, 0, rows), "prompt rows")


def test_decode_at_a_position_matches_its_prefill_row():
    import torch
    import paged_kv_cache_08_amd as P
    # Prefill row i of a 300-row chunk on 1300 tokens and a decode call with
    # that row's query on the first 1000 + i + 1 tokens (different kernels,
    # same attention): within the tolerance of each other and of the oracle.
    log("case: prefill rows vs q_len-1 decode calls on the matching prefixes")
    case = W.make_case(1128, [1300], q_len=300, block_size=16, boost_frac=0.05)
    q, cu = W.pack_varlen(case, [300])
    pre, _ = run_prefill(case, q, cu)
    _, k, v, table, _ = to_device(case)
    for i in (0, 1, 150, 299):
        lens = torch.tensor([1000 + i + 1], dtype=torch.int32, device="cuda")
        dec = P.paged_decode_attention(bf16_tensor(q[i:i + 1][None]), k, v, table, lens, 16, case.scale,
                                       max_seq_len=1300)
        torch.cuda.synchronize()
        assert_matches_oracle(dec.cpu().numpy().astype(np.float64)[0, 0], pre[i], f"decode vs prefill row {i}")
