"""GPU parity of the single-query decode path (split kernel + LSE merge) against
the fp64 oracle, through the C ABI; bit-exact index math; layout invariance."""
import numpy as np
import pytest

import oracle.paged_attention as O
from paged_kv_cache_08_amd import workloads as W
from tests.gpu_helpers import ATOL, REL_FLOOR, assert_matches_oracle, bf16_ulp_distance, log, run_gpu, to_device
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

_cache = {}


def cached(name, make):
    """Named read-only workloads are generated once per test session."""
    if name not in _cache:
        _cache[name] = make()
    return _cache[name]


def hybrid(ctx, bs=784, **kw):
    key = ("hybrid", ctx, bs, tuple(sorted(kw.items())))
    return cached(key, lambda: W.hybrid_long_context(ctx, block_size=bs, **kw))


def oracle_out(case):
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale)


def test_single_sequence_page16_512():
    log("case: batch 1, 512 tokens, page 16, 32 of 64 pages")
    case = W.single_seq_b16()
    assert_matches_oracle(run_gpu(case), oracle_out(case), "b1 L512 B16")


@pytest.mark.parametrize("ctx", W.HYBRID_CONTEXTS)
def test_hybrid_long_context_page784(ctx):
    log(f"case: hybrid decode, context {ctx}, page 784, 5% keys x4")
    case = hybrid(ctx)
    assert_matches_oracle(run_gpu(case), oracle_out(case), f"L{ctx} B784")


def test_page_sizes_give_bitwise_identical_outputs():
    outs = {}
    ref = None
    for bs in (784, 832, 16):
        log(f"case: context 32768, page {bs}")
        case = hybrid(32768, bs)
        outs[bs] = run_gpu(case)
        if ref is None:
            ref = oracle_out(case)
        assert_matches_oracle(outs[bs], ref, f"L32768 B{bs}")
    np.testing.assert_array_equal(outs[832], outs[784])
    np.testing.assert_array_equal(outs[16], outs[784])


def test_partial_last_page16():
    log("case: context 32767, page 16 (partial last page)")
    case = hybrid(32767, 16)
    assert_matches_oracle(run_gpu(case), oracle_out(case), "L32767 B16")


def test_mixed_length_batch():
    log("case: 16 sequences, log-uniform lengths, page 784, interleaved pages")
    case = cached('mixed', W.mixed_batch)
    log(f"  lengths {case.seq_lens.tolist()}")
    total = int(case.seq_lens.sum())
    assert_matches_oracle(run_gpu(case, total_tokens=total), oracle_out(case), "mixed batch")
    # without the total-token hint the plan differs; result still within tolerance
    assert_matches_oracle(run_gpu(case), oracle_out(case), "mixed batch, no hint")


def test_dense_control_d128_gqa4():
    log("case: 32 q heads, 8 KV heads, D 128, page 16, context 32768")
    case = cached('dense', W.dense_control)
    assert_matches_oracle(run_gpu(case), oracle_out(case), "dense control")


# Forced split counts at 16384 tokens give chunks of 512, 320, 256, 192, 128 and
# 64 tokens, so every kernel window (64, 128, 256, 512 tokens) runs, full and
# with dead sub-steps.
@pytest.mark.parametrize("splits", [1, 4, 52, 64, 86, 128, 256])
def test_forced_split_counts_agree(splits):
    import paged_kv_cache_08_amd as P
    log(f"case: context 16384, page 784, {splits} splits")
    case = hybrid(16384)
    got = run_gpu(case, num_splits=splits)
    S, chunk = O.split_plan_ref(1, 4, 16384, 784, P.device_cu_count(), forced_splits=splits)
    window = next(w for w in (64, 128, 256, 512) if chunk <= w)
    assert f" w{window} " in P.last_variant()
    assert f"splits={S} chunk={chunk} " in P.last_variant()
    assert_matches_oracle(got, oracle_out(case), f"S={splits}")


# Beyond 32K: the planner's 512-token splits (137 of them), and a forced plan
# of 1094 one-tile splits, more than the merge keeps per-split weights for
# in LDS (1024), so the merge's global-memory path for the rest runs too.
@pytest.mark.parametrize("splits", [0, 1094])
def test_long_context_70000(splits):
    import paged_kv_cache_08_amd as P
    log(f"case: context 70000, page 784, splits {splits or 'planned'}")
    case = hybrid(70000)
    got = run_gpu(case, num_splits=splits)
    S, chunk = O.split_plan_ref(1, 4, 70000, 784, P.device_cu_count(), forced_splits=splits)
    assert f"splits={S} chunk={chunk} " in P.last_variant()
    assert (S, chunk) == ((137, 512) if splits == 0 else (1094, 64))
    assert_matches_oracle(got, oracle_out(case), f"L70000 S={S}")


def test_batch_of_96_short_and_empty_sequences():
    lens = np.random.default_rng(1013).integers(0, 2001, size=96)
    lens[[5, 77]] = 0
    log(f"case: 96 sequences, lengths 0..2000 (sum {int(lens.sum())}), page 16, interleaved pages")
    case = W.make_case(1013, lens.tolist(), block_size=16, interleave=True, boost_frac=0.05)
    got = run_gpu(case, total_tokens=int(lens.sum()))
    assert_matches_oracle(got, oracle_out(case), "96 sequences")
    assert np.all(got[[5, 77]] == 0.0)


def test_repeat_runs_are_bitwise_identical():
    log("case: repeat, context 4096, page 784")
    case = hybrid(4096)
    a, b = run_gpu(case), run_gpu(case)
    np.testing.assert_array_equal(a, b)


def test_page_relabelling_is_bitwise_invariant():
    log("case: physical page relabelling, 3 sequences, page 16")
    case = W.make_case(77, [3000, 129, 1], block_size=16, interleave=True, boost_frac=0.05)
    a = run_gpu(case)
    perm = np.random.default_rng(3).permutation(case.num_pages)
    k2 = np.empty_like(case.k_cache)
    v2 = np.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    case.k_cache, case.v_cache = k2, v2
    case.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    np.testing.assert_array_equal(run_gpu(case), a)


def test_poisoned_slots_do_not_change_bits():
    log("case: NaN-poisoned vs zeroed unused slots, page 784")
    a = run_gpu(W.make_case(78, [1000, 50], block_size=784, interleave=True, poison=True))
    b = run_gpu(W.make_case(78, [1000, 50], block_size=784, interleave=True, poison=False))
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)


def test_combined_cache_views():
    log("case: combined [P,2,B,Hkv,D] cache, page 832")
    a = W.make_case(79, [2500, 900], block_size=832, combined=True, interleave=True)
    b = W.make_case(79, [2500, 900], block_size=832, combined=False, interleave=True)
    ga = run_gpu(a)
    np.testing.assert_array_equal(ga, run_gpu(b))
    assert_matches_oracle(ga, oracle_out(a), "combined")


def test_bf16_output_is_rounded_f32_output():
    import torch
    log("case: bf16 output, context 4096, page 784")
    case = hybrid(4096)
    f32 = run_gpu(case).astype(np.float32)
    b16 = run_gpu(case, out_dtype=torch.bfloat16).astype(np.float32)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(b16), W.f32_to_bf16_bits(f32))
    # Against the oracle rounded to bf16: within one bf16 step wherever
    # |oracle| >= 1e-3 (below that the fp32 error can exceed a bf16 step),
    # and everywhere within the absolute tolerance plus the rounding to bf16
    # (half a step: 2^-9 of the value, bounded here by 2^-8).
    ref = oracle_out(case)
    big = np.abs(ref) >= REL_FLOOR
    d = bf16_ulp_distance(W.f32_to_bf16_bits(b16), W.f32_to_bf16_bits(ref.astype(np.float32)))
    log(f"  bf16 out vs rounded oracle: max {int(d[big].max())} steps where |oracle| >= {REL_FLOOR}")
    assert int(d[big].max()) <= 1
    assert np.all(np.abs(b16 - ref) <= ATOL + np.abs(ref) * 2.0**-8)


@pytest.mark.parametrize("bs", [1, 3, 16, 784])
def test_short_and_empty_sequences(bs):
    log(f"case: lengths [0,1,2,15,16,17,63,64,65,200], page {bs}")
    case = W.make_case(80 + bs, [0, 1, 2, 15, 16, 17, 63, 64, 65, 200], block_size=bs, interleave=True)
    got = run_gpu(case)
    assert np.all(got[0] == 0.0)
    assert_matches_oracle(got, oracle_out(case), f"short B{bs}")


def test_extra_table_columns_and_odd_pool():
    log("case: wide block table with -1 tail, page 7")
    case = W.make_case(81, [500, 333], block_size=7, interleave=True, extra_table_cols=9, pool_factor=3.0)
    assert_matches_oracle(run_gpu(case), oracle_out(case), "wide table")


def test_invalid_table_entry_is_skipped_and_flagged():
    import torch
    import paged_kv_cache_08_amd as P
    log("case: one out-of-range table entry (tokens skipped, error word set)")
    case = W.make_case(82, [100], block_size=16, poison=False)
    q, k, v, table, lens = to_device(case)
    table[0, 2] = case.num_pages + 5          # page 2 (tokens 32..47) is now invalid
    ws = H.guarded(P.workspace_bytes(P.make_params(q, k, v, table, 16, case.scale, max_seq_len=100), 0),
                   torch.uint8, fill=0)
    out = P.paged_decode_attention(q, k, v, table, lens, 16, case.scale, max_seq_len=100, workspace=ws)
    torch.cuda.synchronize()
    assert P.read_error_word(ws) & 1
    keep = np.ones(100, bool)
    keep[32:48] = False
    # oracle over the tokens that remain
    ref = np.zeros((1, 1, 24, 256))
    sig = float(np.float32(case.scale))
    for h in range(24):
        K = O.bf16_bits_to_f64(case.logical_k[0][keep, h // 6])
        V = O.bf16_bits_to_f64(case.logical_v[0][keep, h // 6])
        s = sig * (K @ O.bf16_bits_to_f64(case.q[0, 0, h]))
        e = np.exp(s - s.max())
        ref[0, 0, h] = e @ V / e.sum()
    assert_matches_oracle(out.cpu().numpy().astype(np.float64), ref, "invalid entry skipped")


# ---------------------------------------------------------------------------
# Bit-exact index math: the split kernel's own address and range code.
# ---------------------------------------------------------------------------

INDEX_CASES = [
    ("b1 L512 B16", lambda: W.single_seq_b16()),
    ("L32768 B784", lambda: hybrid(32768)),
    ("L32768 B832", lambda: hybrid(32768, 832)),
    ("L32767 B16", lambda: hybrid(32767, 16)),
    ("mixed batch", lambda: cached("mixed", W.mixed_batch)),
    ("B7 wide", lambda: W.make_case(83, [500, 333, 0], block_size=7, interleave=True, extra_table_cols=3)),
]


@pytest.mark.parametrize("name,make", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_token_offsets_bit_exact(name, make):
    import torch
    import paged_kv_cache_08_amd as P
    log(f"case: token offsets, {name}")
    case = make()
    q, k, v, table, lens = to_device(case)
    p = P.make_params(q, k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len)
    for g in sorted({0, p.num_kv_heads - 1}):
        k_off, v_off = P.debug_token_offsets(p, table, lens, g)
        torch.cuda.synchronize()
        k_off, v_off = k_off.cpu().numpy(), v_off.cpu().numpy()
        ref_k = O.token_offsets_ref(case.block_table, case.seq_lens, case.block_size,
                                    p.k_stride_page, p.k_stride_tok, p.k_stride_head, g)
        ref_v = O.token_offsets_ref(case.block_table, case.seq_lens, case.block_size,
                                    p.v_stride_page, p.v_stride_tok, p.v_stride_head, g)
        for b in range(case.num_seqs):
            L = int(case.seq_lens[b])
            np.testing.assert_array_equal(k_off[b, :L], ref_k[b])
            np.testing.assert_array_equal(v_off[b, :L], ref_v[b])
            assert np.all(k_off[b, L:] == -1)


@pytest.mark.parametrize("name,make", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_split_ranges_bit_exact(name, make):
    import torch
    import paged_kv_cache_08_amd as P
    log(f"case: split ranges, {name}")
    case = make()
    q, k, v, table, lens = to_device(case)
    cu = P.device_cu_count()
    for forced in (0, 3):
        p = P.make_params(q, k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                          num_splits=forced)
        S, chunk = P.plan_splits(p, cu)
        assert (S, chunk) == O.split_plan_ref(p.num_seqs, p.num_kv_heads, p.max_seq_len, p.block_size, cu,
                                              forced_splits=forced)
        r = P.debug_split_ranges(p, lens)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r.cpu().numpy(), O.split_ranges_ref(case.seq_lens, S, chunk))


@pytest.mark.parametrize("name,make", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_strided_token_splits_bit_exact(name, make):
    import torch
    import paged_kv_cache_08_amd as P
    log(f"case: strided token splits, {name}")
    case = make()
    q, k, v, table, lens = to_device(case)
    cu = P.device_cu_count()
    for forced in (0, 3, 1000):
        p = P.make_params(q, k, v, table, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                          num_splits=forced)
        S, chunk = P.plan_splits(p, cu)
        r = P.debug_token_splits(p, lens)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r.cpu().numpy(), O.decode_token_splits_ref(
            case.seq_lens, S, chunk, max_seq_len=case.max_seq_len))


@pytest.mark.parametrize("hq,hkv,d,bs,lens", [
    (24, 2, 256, 784, [32768]),        # 12 query heads per KV head
    (32, 2, 128, 16, [5000, 17, 0]),   # 16 per KV head
    (128, 1, 128, 832, [3000]),        # 128 per KV head: the MFMA kernel's limit
])
def test_large_groups_run_on_the_mfma_kernel(hq, hkv, d, bs, lens):
    import paged_kv_cache_08_amd as P
    log(f"case: q_len 1, {hq}/{hkv}/{d}, page {bs}, lengths {lens}")
    case = W.make_case(90 + hq + hkv, lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       interleave=True, boost_frac=0.05)
    got = run_gpu(case)
    assert P.last_variant().startswith("verify_mfma")
    assert_matches_oracle(got, oracle_out(case), f"q1 {hq}/{hkv}/{d} B{bs}")
