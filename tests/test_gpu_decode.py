"""Slot-pool decode on the GPU (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import (assert_parity, decode_dev, prefill_dev, say, to_dev, to_dev_i32, to_host_bits,
                      to_host_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module")
def full_case():
    return W.make_decode()


def run(dc, **over):
    t = decode_dev(dc)
    t.update(over)
    out = K.kev_slot_attn_decode(**t)
    torch.cuda.synchronize()
    return out, t["kv_pool"]


def test_slot_decode_config(orc, full_case):
    dc = full_case
    say(f"decode full config n_req={dc.n_req} cap={dc.capacity} slots={dc.n_slots}")
    out, pool = run(dc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    assert_parity(to_host_f64(out), ref, dc.dtype, "slot decode 64 req, cap 2458")
    # the pool differs from before only in the appended rows, which hold k_new / v_new
    assert np.array_equal(to_host_bits(pool), ref_pool)


@pytest.mark.parametrize("hq,hk,d", [(32, 8, 128), (8, 8, 128), (16, 8, 128), (64, 8, 128), (256, 8, 128),
                                     (28, 4, 128), (8, 2, 64), (4, 1, 64), (32, 2, 128), (32, 1, 64),
                                     (24, 8, 128)])
def test_head_layouts_and_edges(orc, hq, hk, d):
    lens = [1, 2, 255, 256, 257, 511, 512, 513, 1000, 1023, 1024, 1025]
    dc = W.make_decode(n_req=len(lens), n_slots=20, capacity=1025, heads=hq, kv_heads=hk,
                       head_dim=d, seed=hq + hk + d, cache_lens=lens)
    say(f"decode {hq}/{hk} d{d} lens={lens}")
    out, pool = run(dc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    assert_parity(to_host_f64(out), ref, dc.dtype, f"decode {hq}/{hk} d{d}")
    assert np.array_equal(to_host_bits(pool), ref_pool)


@pytest.mark.parametrize("n_req,hq,hk,d", [(48, 32, 16, 64), (80, 16, 8, 128)])
def test_many_units_grid_orders(orc, n_req, hq, hk, d):
    # more (request, KV head) units than two per CU: 48 requests are issued longest first,
    # 80 requests (over 64) in index order
    dc = W.make_decode(n_req=n_req, n_slots=n_req + 3, capacity=300, heads=hq, kv_heads=hk,
                       head_dim=d, seed=n_req + hk)
    say(f"decode {n_req} req {hq}/{hk} d{d}")
    out, pool = run(dc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    assert_parity(to_host_f64(out), ref, dc.dtype, f"decode {n_req} req {hq}/{hk} d{d}")
    assert np.array_equal(to_host_bits(pool), ref_pool)


def test_length_one_returns_v_new_exactly():
    dc = W.make_decode(n_req=3, n_slots=4, capacity=64, heads=8, kv_heads=2, head_dim=128,
                       seed=3, cache_lens=[1, 1, 1])
    say("decode L=1")
    out, _ = run(dc)
    got = to_host_bits(out)
    for r in range(3):
        assert np.array_equal(got[r], np.repeat(dc.v_new[r], 4, axis=0))


def test_rows_past_length_and_other_slots_never_read(full_case):
    dc = full_case
    say("decode NaN-poisoned stale rows / unused slots")
    base, _ = run(dc)
    pool = dc.pool.copy()
    nan = np.uint16(0x7FC0)
    used = set(int(s) for s in dc.slot_ids)
    for s in range(dc.n_slots):
        if s not in used:
            pool[s] = nan
    for r in range(dc.n_req):
        pool[int(dc.slot_ids[r]), :, :, int(dc.cache_lens[r]) - 1:] = nan
    poisoned = W.DecodeCase(**{**dc.__dict__, "pool": pool})
    out, _ = run(poisoned)
    assert np.array_equal(to_host_bits(out), to_host_bits(base))


def test_repeat_calls_identical_and_counters_reset():
    dc = W.make_decode(n_req=16, n_slots=20, capacity=2458, heads=32, kv_heads=8, head_dim=128,
                       seed=9)
    t = decode_dev(dc)
    say("decode repeat calls")
    o1 = to_host_bits(K.kev_slot_attn_decode(**t))
    o2 = to_host_bits(K.kev_slot_attn_decode(**t))
    o3 = to_host_bits(K.kev_slot_attn_decode(**t))
    assert np.array_equal(o1, o2) and np.array_equal(o2, o3)


def test_decode_matches_prefill_last_row(orc):
    """Primer section 2.2: decode over the cache equals the last row of a full recompute."""
    L = 700
    pc = W.make_prefill([L], 32, 8, 128, W.BF16, seed=77)
    pool = np.zeros((2, 2, 8, 1024, 128), np.uint16)
    pool[1, 0, :, :L - 1] = pc.k[:L - 1].transpose(1, 0, 2)
    pool[1, 1, :, :L - 1] = pc.v[:L - 1].transpose(1, 0, 2)
    dc = W.DecodeCase("from-prefill", W.BF16, 32, 8, 128, 2, 1024, 0,
                      np.array([1], np.int32), np.array([L], np.int32), pc.q[L - 1:L].copy(),
                      pc.k[L - 1:L].copy(), pc.v[L - 1:L].copy(), pool)
    say("decode vs prefill last row")
    dec, _ = run(dc)
    q, k, v, cu = prefill_dev(pc)
    pre = K.kev_packed_attn_prefill(q, k, v, cu)
    ref = orc.prefill_rows(pc.q, pc.k, pc.v, pc.cu_seqlens, 32, 8, 128, W.BF16,
                           np.full(32, L - 1, np.int32), np.arange(32, dtype=np.int32))
    assert_parity(to_host_f64(dec)[0], ref, W.BF16, "decode row")
    assert_parity(to_host_f64(pre)[L - 1], ref, W.BF16, "prefill last row")


def test_invalid_slot_and_length_are_flagged_and_skipped(monkeypatch):
    dc = W.make_decode(n_req=3, n_slots=4, capacity=64, heads=8, kv_heads=2, head_dim=128,
                       seed=5, cache_lens=[10, 20, 30])
    t = decode_dev(dc)
    out = torch.full_like(t["q"], 5.0)
    say("decode invalid slot id / cache length (device guards)")
    K.kev_slot_attn_decode(**{**t, "slot_ids": to_dev_i32([0, 9, 2]), "out": out})
    assert K.kev_get_device_errors() & K.KEV_DEVERR_SLOT
    assert bool((out[1] == 5.0).all()) and not bool((out[0] == 5.0).all())
    out.fill_(5.0)
    K.kev_slot_attn_decode(**{**t, "cache_lens": to_dev_i32([10, 65, 0]), "out": out})
    flags = K.kev_get_device_errors()
    assert flags & K.KEV_DEVERR_CACHE_LEN
    assert bool((out[1:] == 5.0).all())
    monkeypatch.setenv("KEV_CHECK", "1")
    for ids, lens, code in (([0, 9, 2], [10, 20, 30], K.KEV_ERR_BAD_SLOT),
                            ([0, 0, 2], [10, 20, 30], K.KEV_ERR_BAD_SLOT),
                            ([0, 1, 2], [10, 65, 30], K.KEV_ERR_SLOT_OVERFLOW)):
        with pytest.raises(K.KevError) as e:
            K.kev_slot_attn_decode(**{**t, "slot_ids": to_dev_i32(ids), "cache_lens": to_dev_i32(lens)})
        assert e.value.code == code


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 32])
@pytest.mark.parametrize("paged", [False, True])
def test_split_units_match_oracle(orc, monkeypatch, splits, paged):
    """Each unit's tiles cut over `splits` workgroups (more splits than tiles for the short
    requests) and merged: the oracle's values and the same appended rows."""
    lens = [1, 31, 32, 33, 100, 2458]
    dc = W.make_decode(n_req=len(lens), n_slots=8, capacity=2458, seed=70 + splits, cache_lens=lens)
    monkeypatch.setenv("KEV_DECODE_SPLITS", str(splits))
    say(f"decode split={splits} paged={paged} lens={lens}")
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    if paged:
        pc = W.paged_from_slots(dc, 16, spare_blocks=4)
        t = dict(q=to_dev(pc.q, W.BF16), kv_pool=to_dev(pc.pool, W.BF16), block_tables=to_dev_i32(pc.block_tables),
                 cache_lens=to_dev_i32(pc.cache_lens), k_new=to_dev(pc.k_new, W.BF16), v_new=to_dev(pc.v_new, W.BF16))
        out = K.kev_paged_attn_decode(**t)
        torch.cuda.synchronize()
        assert K.kev_get_device_errors() == 0
        back = W.slots_from_paged_pool(pc, to_host_bits(t["kv_pool"]), dc)
        for r in range(dc.n_req):
            s, L = int(dc.slot_ids[r]), int(dc.cache_lens[r])
            assert np.array_equal(back[s, :, :, :L], ref_pool[s, :, :, :L])
    else:
        out, pool = run(dc)
        assert K.kev_get_device_errors() == 0
        assert np.array_equal(to_host_bits(pool), ref_pool)
    assert_parity(to_host_f64(out), ref, dc.dtype, f"decode split={splits} paged={paged}")


@pytest.mark.parametrize("hq,hk,d", [(32, 1, 128), (32, 2, 64), (28, 4, 128)])
@pytest.mark.parametrize("paged", [False, True])
def test_split_merge_wide_groups(orc, monkeypatch, hq, hk, d, paged):
    """Split units whose group has 7, 16 or 32 query heads: the merge combines every head's
    ranges (32 heads x 128 d is more output than one merge workgroup covers in one pass)."""
    lens = [3, 64, 700, 1025]
    dc = W.make_decode(n_req=len(lens), n_slots=6, capacity=1025, heads=hq, kv_heads=hk, head_dim=d,
                       seed=90 + hq + hk, cache_lens=lens)
    monkeypatch.setenv("KEV_DECODE_SPLITS", "5")
    say(f"decode split=5 {hq}/{hk} d{d} paged={paged}")
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    if paged:
        pc = W.paged_from_slots(dc, 32, spare_blocks=3)
        t = dict(q=to_dev(pc.q, W.BF16), kv_pool=to_dev(pc.pool, W.BF16), block_tables=to_dev_i32(pc.block_tables),
                 cache_lens=to_dev_i32(pc.cache_lens), k_new=to_dev(pc.k_new, W.BF16), v_new=to_dev(pc.v_new, W.BF16))
        out = K.kev_paged_attn_decode(**t)
        torch.cuda.synchronize()
    else:
        out, pool = run(dc)
        assert np.array_equal(to_host_bits(pool), ref_pool)
    assert K.kev_get_device_errors() == 0
    assert_parity(to_host_f64(out), ref, dc.dtype, f"decode split=5 {hq}/{hk} d{d} paged={paged}")


@pytest.mark.parametrize("n_req", [1, 2, 5])
def test_low_occupancy_batches(orc, n_req):
    """A batch that has shrunk to a few requests (automatic split count)."""
    dc = W.make_decode(n_req=n_req, n_slots=8, seed=80 + n_req)
    say(f"decode low occupancy n_req={n_req} lens={list(dc.cache_lens)}")
    out, pool = run(dc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    assert_parity(to_host_f64(out), ref, dc.dtype, f"decode n_req={n_req}")
    assert np.array_equal(to_host_bits(pool), ref_pool)


def test_full_config_split_and_unsplit_agree(orc, full_case, monkeypatch):
    ref = orc.decode_case(full_case)
    for splits in (1, 4):
        monkeypatch.setenv("KEV_DECODE_SPLITS", str(splits))
        say(f"decode full config split={splits}")
        out, _ = run(full_case)
        assert K.kev_get_device_errors() == 0
        assert_parity(to_host_f64(out), ref, full_case.dtype, f"decode full config split={splits}")
