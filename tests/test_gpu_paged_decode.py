"""Decode against a paged (block-table) KV pool on the GPU (through the C ABI).

kev_paged_attn_decode reads request r's position p from block block_tables[r, p // B],
row p % B, appends the new K/V row in place and attends over positions 0..L-1.  Checked
against the CPU oracle, and against the slot decode on the same rows (same tiles and
arithmetic, so the outputs must agree bit for bit).
"""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import assert_parity, decode_dev, say, to_dev, to_dev_i32, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module")
def decode_case():
    return W.make_decode()


def paged_dev(pc):
    return dict(q=to_dev(pc.q, W.BF16), kv_pool=to_dev(pc.pool, W.BF16),
                block_tables=to_dev_i32(pc.block_tables), cache_lens=to_dev_i32(pc.cache_lens),
                k_new=to_dev(pc.k_new, W.BF16), v_new=to_dev(pc.v_new, W.BF16))


def run_paged(pc):
    a = paged_dev(pc)
    out = K.kev_paged_attn_decode(**a)
    torch.cuda.synchronize()
    return out, a["kv_pool"]


@pytest.mark.parametrize("n_req,hq,hk,d,cap,B", [
    (10, 32, 8, 128, 300, 16),
    (10, 32, 8, 128, 300, 32),
    (7, 8, 2, 64, 200, 64),
    (9, 28, 4, 128, 150, 8),      # Qwen2.5-7B group of 7, blocks smaller than a 32-row tile
    (5, 16, 16, 64, 40, 1),       # one position per block
])
def test_paged_matches_oracle(orc, n_req, hq, hk, d, cap, B):
    lens = np.random.default_rng(n_req + B).integers(1, cap + 1, n_req)
    lens[:3] = [1, min(B, cap), min(B + 1, cap)]            # first row, block edges
    dc = W.make_decode(n_req=n_req, n_slots=n_req + 2, capacity=cap, heads=hq, kv_heads=hk, head_dim=d,
                       seed=60 + B, cache_lens=lens)
    pc = W.paged_from_slots(dc, B, spare_blocks=5, seed=61)
    say(f"paged decode n_req={n_req} {hq}/{hk} d{d} B={B} lens={list(lens)}")
    out, dpool = run_paged(pc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.paged_decode(pc.q, pc.pool, pc.block_tables, pc.cache_lens, pc.k_new, pc.v_new, hq,
                                     W.BF16, want_pool=True)
    assert_parity(to_host_f64(out), ref, W.BF16, f"paged decode B={B}")
    assert np.array_equal(to_host_bits(dpool), ref_pool)


@pytest.mark.parametrize("B", [16, 64])
def test_full_size_paged_equals_slot_decode(orc, decode_case, B):
    """The decode workload (64 requests, lengths up to 2458) over a paged pool: bit for bit the
    slot decode's output, the same rows after the append, and the oracle's values."""
    dc = decode_case
    pc = W.paged_from_slots(dc, B, spare_blocks=32)
    say(f"paged decode full size B={B} blocks={pc.n_blocks}")
    out, dpool = run_paged(pc)
    a = decode_dev(dc)
    out_slot = K.kev_slot_attn_decode(**a)
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    assert torch.equal(out.view(torch.int16), out_slot.view(torch.int16))
    back = W.slots_from_paged_pool(pc, to_host_bits(dpool), dc)
    slot_after = to_host_bits(a["kv_pool"])
    for r in range(dc.n_req):
        s, L = int(dc.slot_ids[r]), int(dc.cache_lens[r])
        assert np.array_equal(back[s, :, :, :L], slot_after[s, :, :, :L])
    ref = orc.paged_decode(pc.q, pc.pool, pc.block_tables, pc.cache_lens, pc.k_new, pc.v_new, dc.heads, W.BF16)
    assert_parity(to_host_f64(out), ref, W.BF16, f"paged decode full size B={B}")


def test_shared_prefix_blocks(orc):
    """Two requests read the same prefix blocks and append into blocks of their own."""
    rng = np.random.default_rng(62)
    B, hq, hk, d = 16, 32, 8, 128
    pool = W.round_to_bf16_bits(rng.standard_normal((12, 2, hk, B, d)).astype(np.float32))
    tables = np.array([[3, 7, 1, -1], [3, 7, 9, 4], [5, -1, -1, -1]], np.int32)
    lens = np.array([40, 60, 16], np.int32)                 # both share blocks 3 and 7 (32 rows)
    q, kn, vn = (W.round_to_bf16_bits(rng.standard_normal((3, h, d)).astype(np.float32)) for h in (hq, hk, hk))
    pc = W.PagedDecodeCase("shared", hq, hk, d, B, 62, tables, lens, q, kn, vn, pool)
    say("paged decode with shared prefix blocks")
    out, dpool = run_paged(pc)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.paged_decode(q, pool, tables, lens, kn, vn, hq, W.BF16, want_pool=True)
    assert_parity(to_host_f64(out), ref, W.BF16, "shared prefix blocks")
    assert np.array_equal(to_host_bits(dpool), ref_pool)


def test_invalid_blocks_and_lengths(orc, monkeypatch):
    rng = np.random.default_rng(63)
    B, hq, hk, d = 16, 8, 2, 64
    pool = W.round_to_bf16_bits(rng.standard_normal((6, 2, hk, B, d)).astype(np.float32))
    tables = np.array([[0, 1], [2, 9], [3, -1], [4, 5]], np.int32)
    lens = np.array([20, 30, 40, 0], np.int32)   # 1: block 9 outside; 2: 40 > 2 blocks; 3: length 0
    q, kn, vn = (W.round_to_bf16_bits(rng.standard_normal((4, h, d)).astype(np.float32)) for h in (hq, hk, hk))
    pc = W.PagedDecodeCase("bad", hq, hk, d, B, 63, tables, lens, q, kn, vn, pool)
    say("paged decode bad block id / lengths (device guards)")
    a = paged_dev(pc)
    out0 = torch.zeros((4, hq, d), dtype=torch.bfloat16, device="cuda")
    out = K.kev_paged_attn_decode(**a, out=out0)
    flags = K.kev_get_device_errors()
    assert flags & K.KEV_DEVERR_BLOCK and flags & K.KEV_DEVERR_CACHE_LEN
    got = to_host_f64(out)
    assert (got[1:] == 0).all()
    ref, ref_pool = orc.paged_decode(q[:1], pool, tables[:1], lens[:1], kn[:1], vn[:1], hq, W.BF16, want_pool=True)
    assert_parity(got[:1], ref, W.BF16, "valid request beside invalid ones")
    assert np.array_equal(to_host_bits(a["kv_pool"]), ref_pool)
    monkeypatch.setenv("KEV_CHECK", "1")
    good = np.array([20, 30, 10, 5], np.int32)
    for tb, ln, code in ((tables, good, K.KEV_ERR_BAD_SLOT),                              # block 9
                         (np.array([[0, 1], [2, 3], [4, -1], [5, -1]]), np.array([20, 30, 40, 5]),
                          K.KEV_ERR_SLOT_OVERFLOW),                                         # 40 > 32
                         (np.array([[0, 1], [0, 1], [4, -1], [5, -1]]), np.array([20, 20, 3, 5]),
                          K.KEV_ERR_BAD_SLOT),                                              # same append row
                         (np.array([[0, 1], [1, -1], [4, -1], [5, -1]]), np.array([20, 2, 3, 5]),
                          K.KEV_ERR_BAD_SLOT)):                                             # appends into a row 0 reads
        b = dict(paged_dev(pc), block_tables=to_dev_i32(tb), cache_lens=to_dev_i32(ln))
        with pytest.raises(K.KevError) as e:
            K.kev_paged_attn_decode(**b)
        assert e.value.code == code


def test_block_table_limit(orc):
    """One position per block and a request spanning KEV_PAGED_MAX_BLOCKS blocks: the whole
    block-id table of that request is staged on chip.  A request one position longer, with a
    table row wide enough to hold it, is past the limit and is flagged and skipped."""
    lim = K.KEV_PAGED_MAX_BLOCKS
    rng = np.random.default_rng(64)
    hq, hk, d = 8, 2, 64
    lens = np.array([lim, 1000, 1, lim + 1], np.int32)
    used = int(lens[:3].sum())
    n_blocks = used + 3
    pool = W.round_to_bf16_bits(rng.standard_normal((n_blocks, 2, hk, 1, d)).astype(np.float32))
    perm = rng.permutation(n_blocks).astype(np.int32)
    tables = np.full((4, lim + 1), -1, np.int32)
    off = 0
    for r in range(3):
        tables[r, :lens[r]] = perm[off:off + lens[r]]
        off += int(lens[r])
    tables[3, :] = 0                           # never read: the request is past the limit
    q, kn, vn = (W.round_to_bf16_bits(rng.standard_normal((4, h, d)).astype(np.float32)) for h in (hq, hk, hk))
    pc = W.PagedDecodeCase("table_limit", hq, hk, d, 1, 64, tables, lens, q, kn, vn, pool)
    say(f"paged decode B=1, table limit {lim}, lens={list(lens)}")
    out0 = torch.zeros((4, hq, d), dtype=torch.bfloat16, device="cuda")
    a = paged_dev(pc)
    out = K.kev_paged_attn_decode(**a, out=out0)
    assert K.kev_get_device_errors() == K.KEV_DEVERR_CACHE_LEN
    got = to_host_f64(out)
    assert (got[3] == 0).all()
    ref, ref_pool = orc.paged_decode(q[:3], pool, tables[:3], lens[:3], kn[:3], vn[:3], hq, W.BF16,
                                     want_pool=True)
    assert_parity(got[:3], ref, W.BF16, "paged decode at the block-table limit")
    assert np.array_equal(to_host_bits(a["kv_pool"]), ref_pool)
