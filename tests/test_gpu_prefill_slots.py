"""Prefill-to-slot handoff on the GPU (through the C ABI) against the CPU oracle.

kev_packed_attn_prefill_slots computes the packed prefill and stores every question's K/V
rows as rows 0..len-1 of its slot; a following decode continues each question there.
"""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import assert_parity, prefill_dev, say, to_dev, to_dev_i32, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def make(lens, hq, hk, d, n_slots, cap, seed):
    case = W.make_prefill(lens, hq, hk, d, W.BF16, seed=seed)
    rng = np.random.default_rng(seed + 1)
    slots = rng.permutation(n_slots)[:len(lens)].astype(np.int32)
    pool = W.round_to_bf16_bits(rng.standard_normal((n_slots, 2, hk, cap, d)).astype(np.float32))
    return case, slots, pool


def run(case, slots, pool):
    q, k, v, cu = prefill_dev(case)
    dpool = to_dev(pool, W.BF16)
    out = K.kev_packed_attn_prefill_slots(q, k, v, cu, dpool, to_dev_i32(slots))
    torch.cuda.synchronize()
    return out, dpool


@pytest.mark.parametrize("lens,hq,hk,d", [([7, 0, 1, 64, 33, 96], 8, 2, 128, ),
                                          ([96, 1, 50], 32, 8, 64),
                                          ([31, 32, 33, 0, 5], 28, 4, 128)])
def test_store_and_prefill_match_oracle(orc, lens, hq, hk, d):
    case, slots, pool = make(lens, hq, hk, d, n_slots=len(lens) + 3, cap=96, seed=len(lens) + hq)
    say(f"prefill_slots lens={lens} {hq}/{hk} d{d}")
    out, dpool = run(case, slots, pool)
    assert K.kev_get_device_errors() == 0
    assert np.array_equal(to_host_bits(dpool), orc.store_kv(case.k, case.v, case.cu_seqlens, slots, pool, W.BF16))
    assert_parity(to_host_f64(out), orc.prefill_case(case), W.BF16, f"prefill_slots {lens}")


def test_handoff_then_decode_continues_each_question(orc):
    lens = [40, 1, 0, 77, 12]
    hq, hk, d = 32, 8, 128
    case, slots, pool = make(lens, hq, hk, d, n_slots=9, cap=80, seed=31)
    say("prefill_slots then decode")
    _, dpool = run(case, slots, pool)
    assert K.kev_get_device_errors() == 0
    stored = orc.store_kv(case.k, case.v, case.cu_seqlens, slots, pool, W.BF16)
    keep = [s for s in range(len(lens)) if lens[s] > 0]
    rng = np.random.default_rng(32)
    qn = W.round_to_bf16_bits(rng.standard_normal((len(keep), hq, d)).astype(np.float32))
    kn = W.round_to_bf16_bits(rng.standard_normal((len(keep), hk, d)).astype(np.float32))
    vn = W.round_to_bf16_bits(rng.standard_normal((len(keep), hk, d)).astype(np.float32))
    ids = slots[keep]
    cl = np.array([lens[s] + 1 for s in keep], np.int32)
    out = K.kev_slot_attn_decode(to_dev(qn, W.BF16), dpool, to_dev_i32(ids), to_dev_i32(cl),
                                 to_dev(kn, W.BF16), to_dev(vn, W.BF16))
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.decode(qn, stored, ids, cl, kn, vn, hq, W.BF16, want_pool=True)
    assert_parity(to_host_f64(out), ref, W.BF16, "decode after handoff")
    assert np.array_equal(to_host_bits(dpool), ref_pool)


def test_qwen25_shape_store(orc):
    case = W.prefill_case("qwen25_7b")
    rng = np.random.default_rng(5)
    n_slots, cap = 12, 2458
    slots = rng.permutation(n_slots)[:case.n_seg].astype(np.int32)
    pool = np.zeros((n_slots, 2, case.kv_heads, cap, case.head_dim), np.uint16)
    say("prefill_slots qwen2.5-7b-shaped store")
    _, dpool = run(case, slots, pool)
    assert K.kev_get_device_errors() == 0
    assert np.array_equal(to_host_bits(dpool), orc.store_kv(case.k, case.v, case.cu_seqlens, slots, pool, W.BF16))


def test_invalid_slot_or_overflow_skips_that_question(orc, monkeypatch):
    lens = [10, 20, 30]
    case, _, pool = make(lens, 8, 2, 128, n_slots=5, cap=25, seed=41)
    say("prefill_slots bad slot id / overflow (device guards)")
    slots = np.array([3, 9, 1], np.int32)        # question 1: slot out of range; question 2: 30 > 25
    _, dpool = run(case, slots, pool)
    flags = K.kev_get_device_errors()
    assert flags & K.KEV_DEVERR_SLOT and flags & K.KEV_DEVERR_CACHE_LEN
    got = to_host_bits(dpool)
    # only question 0 was stored
    expect = orc.store_kv(case.k[:10], case.v[:10], [0, 10], [3], pool, W.BF16)
    assert np.array_equal(got, expect)
    monkeypatch.setenv("KEV_CHECK", "1")
    for ids, code in (([3, 9, 1], K.KEV_ERR_BAD_SLOT), ([3, 3, 1], K.KEV_ERR_BAD_SLOT),
                      ([3, 0, 1], K.KEV_ERR_SLOT_OVERFLOW)):
        q, k, v, cu = prefill_dev(case)
        with pytest.raises(K.KevError) as e:
            K.kev_packed_attn_prefill_slots(q, k, v, cu, to_dev(pool, W.BF16), to_dev_i32(ids))
        assert e.value.code == code
