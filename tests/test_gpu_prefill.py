"""Packed prefill on the GPU (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import (assert_parity, prefill_dev, say, sample_rows, to_dev, to_dev_i32,
                      to_host_bits, to_host_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run(case):
    q, k, v, cu = prefill_dev(case)
    out = K.kev_packed_attn_prefill(q, k, v, cu)
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    return out


def check_full(case, orc, what):
    say(f"prefill {what}: T={case.total_tokens} heads={case.heads}/{case.kv_heads} d={case.head_dim} {case.dtype}")
    got = to_host_f64(run(case))
    ref = orc.prefill_case(case)
    assert_parity(got, ref, case.dtype, what)
    return got


def test_tiny_config(orc):
    check_full(W.prefill_case("tiny"), orc, "tiny fp32 4/4 d16 [37,64,11,128]")


def test_qwen25_shape_full(orc):
    check_full(W.prefill_case("qwen25_7b"), orc, "qwen2.5-7b-shaped full")


def test_qwen3_shape_reduced_heads_full(orc):
    # same 32 lengths (fix-total to 24576), 8 q / 2 kv heads: every row checked
    check_full(W.prefill_case("qwen3_8b", heads=8, kv_heads=2), orc, "qwen3-8b lengths, 8/2 heads")


def test_qwen3_shape_full_size_sampled(orc):
    case = W.prefill_case("qwen3_8b")
    say(f"prefill qwen3-8b full size sampled T={case.total_tokens}")
    got = to_host_f64(run(case))
    rows, heads = sample_rows(case, 600, seed=1)
    ref = orc.prefill_rows(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads,
                           case.head_dim, case.dtype, rows, heads)
    assert_parity(got[rows, heads], ref, case.dtype, "qwen3-8b full size, sampled rows")


def test_skewed_long_reduced_heads_every_row(orc):
    # the same 256 lengths (131072 tokens, questions up to 6967 rows: up to 218 key tiles per
    # query block), 8 q / 2 kv heads: every output element against the oracle
    check_full(W.prefill_case("skewed_long", heads=8, kv_heads=2), orc, "skewed long lengths, 8/2 heads")


def test_skewed_long_sampled(orc):
    case = W.prefill_case("skewed_long")
    say(f"prefill skewed long T={case.total_tokens}")
    got = to_host_f64(run(case))
    rows, heads = sample_rows(case, 300, seed=2)
    ref = orc.prefill_rows(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads,
                           case.head_dim, case.dtype, rows, heads)
    assert_parity(got[rows, heads], ref, case.dtype, "skewed long, sampled rows")


@pytest.mark.parametrize("hq,hk", [(28, 4), (32, 8), (7, 1), (4, 1), (8, 8), (16, 2), (12, 4),
                                   (5, 1), (6, 1), (2, 1), (64, 8), (3, 3), (32, 2), (32, 1), (24, 4)])
def test_head_layouts(orc, hq, hk):
    case = W.make_prefill([1, 95, 31, 160, 64, 33, 0, 200], hq, hk, 128, W.BF16, seed=hq * 100 + hk)
    check_full(case, orc, f"bf16 {hq}/{hk} d128 ragged")


@pytest.mark.parametrize("hq,hk", [(8, 2), (7, 1), (4, 4), (6, 2)])
def test_wave_row_block_boundaries(orc, hq, hk):
    # head_dim 128: a wavefront owns 48 query rows, and an item 48*R rows (R = 1, 4, 4, 4 for
    # these groupings); lengths on both sides of those edges, every row checked
    lens = [47, 48, 49, 95, 96, 97, 143, 144, 145, 191, 192, 193, 383, 385]
    case = W.make_prefill(lens, hq, hk, 128, W.BF16, seed=hq * 7 + hk)
    check_full(case, orc, f"bf16 {hq}/{hk} d128, 48-row block edges")


def test_one_long_question_sampled(orc):
    # 32768 rows in one question: the last items walk 1024 key tiles
    case = W.make_prefill([32768], 8, 2, 128, W.BF16, seed=327)
    say(f"prefill one question of {case.total_tokens} rows, 8/2 heads, sampled")
    got = to_host_f64(run(case))
    rows, heads = sample_rows(case, 300, seed=3)
    rows = np.concatenate([rows, [0, 47, 48, 32767]]).astype(rows.dtype)
    heads = np.concatenate([heads, [0, 7, 3, 5]]).astype(heads.dtype)
    ref = orc.prefill_rows(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads,
                           case.head_dim, case.dtype, rows, heads)
    assert_parity(got[rows, heads], ref, case.dtype, "one 32768-row question, sampled rows")


def test_head_dim_64(orc):
    check_full(W.make_prefill([300, 1, 77, 129], 8, 2, 64, W.BF16, seed=64), orc, "bf16 d64")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_fp32_head_dims(orc, d):
    check_full(W.make_prefill([70, 1, 130, 0, 33], 4, 2, d, W.F32, seed=d), orc, f"fp32 d{d}")


@pytest.mark.parametrize("lens", [[1], [1] * 50, [2048], [33, 31, 32, 65, 63, 64, 127, 129],
                                  [0, 0, 5, 0], [4097, 3],
                                  # 64 questions (items derived in the attention kernel) and 65
                                  # (scheduling pass first), equal and mixed lengths
                                  [3] * 64, [3] * 65, [(i * 37) % 90 for i in range(64)],
                                  [(i * 37) % 90 for i in range(65)]])
def test_segment_edge_cases(orc, lens):
    check_full(W.make_prefill(lens, 8, 2, 128, W.BF16, seed=len(lens)), orc, f"bf16 lens={lens[:8]}")


def test_worked_example_values():
    """Primer section 2.4: scores 1..4 against values 10..40 give 34.926527 for the full row."""
    d = 16
    q = np.zeros((4, 1, d), np.float32)
    q[:, 0, 0] = 4.0                         # q.k_j / sqrt(16) = j
    k = np.zeros((4, 1, d), np.float32)
    k[:, 0, 0] = [1, 2, 3, 4]
    v = np.zeros((4, 1, d), np.float32)
    v[:, 0, :] = np.array([10, 20, 30, 40], np.float32)[:, None]
    say("prefill worked example fp32 d16")
    out = K.kev_packed_attn_prefill(to_dev(q, W.F32), to_dev(k, W.F32), to_dev(v, W.F32),
                                    to_dev_i32([0, 4])).cpu().numpy()
    assert abs(out[3, 0, 0] - 34.926527) < 5e-5
    assert abs(out[1, 0, 0] - (10 + 20 * np.e) / (1 + np.e)) < 5e-5
    assert out[0, 0, 0] == 10.0
    # the same in bf16 at head dim 128, values scaled to 0.1..0.4
    d = 128
    qb = np.zeros((4, 1, d), np.float32)
    qb[:, 0, 0] = np.sqrt(d)
    kb = np.zeros((4, 1, d), np.float32)
    kb[:, 0, 0] = [1, 2, 3, 4]
    vb = np.zeros((4, 1, d), np.float32)
    vb[:, 0, :] = np.array([0.1, 0.2, 0.3, 0.4], np.float32)[:, None]
    say("prefill worked example bf16 d128")
    outb = K.kev_packed_attn_prefill(*(to_dev(W.round_to_bf16_bits(x), W.BF16) for x in (qb, kb, vb)),
                                     to_dev_i32([0, 4])).float().cpu().numpy()
    assert abs(outb[3, 0, 0] - 0.34926527) < 2e-3


def test_length_one_rows_equal_v_exactly():
    case = W.make_prefill([1, 1, 5, 1], 8, 4, 128, W.BF16, seed=11)
    say("prefill length-1 rows")
    out = to_host_bits(run(case))
    for row in (0, 1, 7):
        assert np.array_equal(out[row], np.repeat(case.v[row], 2, axis=0))


def test_packed_equals_each_segment_alone_bitwise():
    case = W.make_prefill([100, 1, 257, 64, 31], 8, 2, 128, W.BF16, seed=5)
    say("prefill packed vs alone")
    packed = to_host_bits(run(case))
    cu = case.cu_seqlens
    for s in range(case.n_seg):
        a, b = int(cu[s]), int(cu[s + 1])
        alone = W.PrefillCase("alone", W.BF16, 8, 2, 128, np.array([b - a]), 0,
                              case.q[a:b].copy(), case.k[a:b].copy(), case.v[a:b].copy())
        assert np.array_equal(to_host_bits(run(alone)), packed[a:b]), s


def test_neighbour_nan_poison_leaves_segment_bitwise_unchanged():
    case = W.make_prefill([90, 200, 45], 8, 2, 128, W.BF16, seed=6)
    say("prefill NaN poison of neighbours")
    base = to_host_bits(run(case))
    a, b = int(case.cu_seqlens[1]), int(case.cu_seqlens[2])
    nan = np.uint16(0x7FC0)
    for arr in (case.q, case.k, case.v):
        arr[:a] = nan
        arr[b:] = nan
    poisoned = to_host_bits(run(case))
    assert np.array_equal(poisoned[a:b], base[a:b])


def test_future_in_segment_values_do_not_leak():
    case = W.make_prefill([150, 70], 4, 1, 128, W.BF16, seed=8)
    say("prefill large future keys/values")
    base = to_host_bits(run(case))
    big = W.round_to_bf16_bits(np.full((1, 128), 3.0e38, np.float32))
    case.k[149] = big
    case.v[149] = big
    changed = to_host_bits(run(case))
    assert np.array_equal(changed[:149], base[:149])
    assert np.array_equal(changed[150:], base[150:])


def test_repeat_runs_bitwise_identical():
    case = W.prefill_case("qwen25_7b", heads=7, kv_heads=1)
    say("prefill determinism")
    q, k, v, cu = prefill_dev(case)
    o1 = to_host_bits(K.kev_packed_attn_prefill(q, k, v, cu))
    o2 = to_host_bits(K.kev_packed_attn_prefill(q, k, v, cu))
    assert np.array_equal(o1, o2)


def test_device_schedule_matches_host_schedule():
    for name in ("tiny", "qwen25_7b", "qwen3_8b", "skewed_long"):
        lens = W.prefill_lengths(name)
        cu = W.cu_from_lengths(lens)
        for br in (32, 48, 64, 96, 128, 192):
            for order in (K.KEV_ORDER_QUESTION, K.KEV_ORDER_LEVEL):
                say(f"schedule {name} block_rows={br} order={order}")
                dev = K.kev_schedule_device(to_dev_i32(cu), int(cu[-1]), br, order)
                host = K.kev_schedule_host(cu, br, order)
                assert len(dev) == len(host)
                # questions of equal block count may come in another order on the device:
                # the (block count, query block) sequence and the item set must match
                nb = -(-np.diff(cu) // br)
                assert np.array_equal(nb[dev[:, 0]], nb[host[:, 0]])
                assert np.array_equal(dev[:, 1], host[:, 1])
                assert sorted(map(tuple, dev.tolist())) == sorted(map(tuple, host.tolist()))


def test_bad_cu_seqlens_flagged_and_nothing_written(monkeypatch):
    q = torch.zeros(10, 4, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(10, 1, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    cu = to_dev_i32([0, 6, 4, 10])        # decreasing
    say("prefill bad cu_seqlens (device check)")
    K.kev_packed_attn_prefill(q, k, k, cu, out=out)
    assert K.kev_get_device_errors() & K.KEV_DEVERR_SEQLENS
    assert bool((out == 7.0).all())
    monkeypatch.setenv("KEV_CHECK", "1")
    with pytest.raises(K.KevError) as e:
        K.kev_packed_attn_prefill(q, k, k, cu, out=out)
    assert e.value.code == K.KEV_ERR_BAD_SEQLENS
    with pytest.raises(K.KevError) as e:
        K.kev_packed_attn_prefill(q, k, k, to_dev_i32([0, 4, 9]), out=out)   # ends short of T
    assert e.value.code == K.KEV_ERR_BAD_SEQLENS
    monkeypatch.delenv("KEV_CHECK")
    for bad in ([0, 4, 9], [1, 4, 10], [0] + [5] * 35 + [3] * 35 + [10]):   # short end, nonzero start, 71 segs
        say(f"prefill bad cu_seqlens {bad[:4]}.. (device check, {len(bad) - 1} segments)")
        K.kev_packed_attn_prefill(q, k, k, to_dev_i32(bad), out=out)
        assert K.kev_get_device_errors() & K.KEV_DEVERR_SEQLENS
        assert bool((out == 7.0).all())
