"""Seeded random small cases for every entry point, each checked against the CPU oracle.

The shapes, lengths, prefixes, block sizes and batch sizes are drawn from a fixed seed per case,
so a failure names a reproducible case.  Every case is small enough for the oracle to run in a
fraction of a second.
"""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import assert_parity, prefill_dev, say, to_dev, to_dev_i32, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

# (heads, kv_heads) pairs: MHA, GQA groups 2..8 and the TP-shard shapes
HEADS = [(8, 8), (8, 2), (16, 8), (28, 4), (32, 8), (4, 1), (7, 1), (12, 3), (40, 8)]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def lengths(rng, n, hi):
    """Question lengths with the edge values mixed in: 0, 1, tile and block boundaries."""
    edges = np.array([0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129])
    out = rng.integers(0, hi + 1, n)
    pick = rng.random(n) < 0.4
    out[pick] = rng.choice(edges[edges <= hi], pick.sum())
    return out


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(orc, seed):
    rng = np.random.default_rng(1000 + seed)
    hq, hk = HEADS[seed % len(HEADS)]
    d = 64 if seed % 3 == 0 else 128
    lens = lengths(rng, int(rng.integers(1, 12)), 300)
    case = W.make_prefill(lens, hq, hk, d, W.BF16, seed=2000 + seed)
    say(f"random prefill seed={seed} {hq}/{hk} d{d} lens={list(lens)}")
    out = K.kev_packed_attn_prefill(*prefill_dev(case))
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    assert_parity(to_host_f64(out), orc.prefill_case(case), W.BF16, f"random prefill {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_chunked_prefill(orc, seed):
    rng = np.random.default_rng(3000 + seed)
    hq, hk = HEADS[(seed * 5) % len(HEADS)]
    d = 128 if seed % 4 else 64
    n = int(rng.integers(1, 9))
    lens = lengths(rng, n, 200)
    pre = lengths(rng, n, 250)
    cap = int((lens + pre).max()) + int(rng.integers(0, 40)) + 1
    case = W.make_chunked(lens, pre, hq, hk, d, cap, n_slots=n + int(rng.integers(0, 4)), seed=4000 + seed)
    say(f"random chunked seed={seed} {hq}/{hk} d{d} lens={list(lens)} pre={list(pre)} cap={cap}")
    dq, dk, dv, dpool = (to_dev(x, W.BF16) for x in (case.q, case.k, case.v, case.pool))
    out = K.kev_chunked_prefill_slots(dq, dk, dv, to_dev_i32(case.cu_seqlens), dpool, to_dev_i32(case.slot_ids),
                                      to_dev_i32(case.prefix_lens))
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.chunked_prefill(case.q, case.k, case.v, case.cu_seqlens, hq, case.slot_ids,
                                        case.prefix_lens, case.pool, W.BF16)
    assert_parity(to_host_f64(out), ref, W.BF16, f"random chunked {seed}")
    assert np.array_equal(to_host_bits(dpool), ref_pool)


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(orc, seed, monkeypatch):
    """Slot and paged decode of the same random requests, with a random split count."""
    rng = np.random.default_rng(5000 + seed)
    hq, hk = HEADS[(seed * 7) % len(HEADS)]
    d = 64 if seed % 3 == 1 else 128
    n_req = int(rng.integers(1, 40))
    cap = int(rng.integers(1, 700))
    lens = np.minimum(lengths(rng, n_req, cap), cap)
    lens = np.maximum(lens, 1)
    dc = W.make_decode(n_req=n_req, n_slots=n_req + int(rng.integers(0, 5)), capacity=cap, heads=hq,
                       kv_heads=hk, head_dim=d, seed=6000 + seed, cache_lens=lens)
    splits = [0, 1, 2, 5, 8, 32][seed % 6]
    if splits:
        monkeypatch.setenv("KEV_DECODE_SPLITS", str(splits))
    B = [1, 4, 16, 32, 64, 128][(seed * 5) % 6]
    pc = W.paged_from_slots(dc, B, spare_blocks=int(rng.integers(0, 6)), seed=7000 + seed)
    say(f"random decode seed={seed} {hq}/{hk} d{d} n_req={n_req} cap={cap} splits={splits} B={B}")
    ref, ref_pool = orc.decode_case(dc, want_pool=True)
    dpool = to_dev(dc.pool, W.BF16)
    out = K.kev_slot_attn_decode(to_dev(dc.q, W.BF16), dpool, to_dev_i32(dc.slot_ids), to_dev_i32(dc.cache_lens),
                                 to_dev(dc.k_new, W.BF16), to_dev(dc.v_new, W.BF16))
    ppool = to_dev(pc.pool, W.BF16)
    pout = K.kev_paged_attn_decode(to_dev(pc.q, W.BF16), ppool, to_dev_i32(pc.block_tables),
                                   to_dev_i32(pc.cache_lens), to_dev(pc.k_new, W.BF16), to_dev(pc.v_new, W.BF16))
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    assert_parity(to_host_f64(out), ref, W.BF16, f"random slot decode {seed}")
    assert np.array_equal(to_host_bits(dpool), ref_pool)
    assert torch.equal(out.view(torch.int16), pout.view(torch.int16))   # same rows, same arithmetic
    pref_pool = orc.paged_decode(pc.q, pc.pool, pc.block_tables, pc.cache_lens, pc.k_new, pc.v_new, hq, W.BF16,
                                 want_pool=True)[1]
    assert np.array_equal(to_host_bits(ppool), pref_pool)
