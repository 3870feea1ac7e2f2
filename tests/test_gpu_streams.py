"""The boundary's stream contract on the GPU: every call's workspace is stream-ordered (calls on
several streams in flight at once, and calls whose workspace grows, need no synchronisation and
do not disturb each other), and the device error word is per stream (kev_get_device_errors(s)
reports the units of stream s only).  A slot pool is passed in explicitly and the library keeps
no hidden state between calls (KV-cache isolation article, hnwysp.cn, sections 3.3 and 4.3)."""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import assert_parity, decode_dev, prefill_dev, say, to_dev_i32, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def test_error_words_are_per_stream():
    dc = W.make_decode(n_req=3, n_slots=4, capacity=64, heads=8, kv_heads=2, head_dim=128,
                       seed=11, cache_lens=[10, 20, 30])
    t = decode_dev(dc)
    bad_ids = to_dev_i32([0, 9, 2])
    out_a, out_b = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say("decode with an out-of-range slot id on stream A, a valid decode on stream B")
    K.kev_slot_attn_decode(**{**t, "slot_ids": bad_ids, "out": out_a}, stream=sa)
    K.kev_slot_attn_decode(**{**t, "out": out_b}, stream=sb)
    assert K.kev_get_device_errors(stream=sb) == 0
    assert K.kev_get_device_errors(stream=sa) & K.KEV_DEVERR_SLOT
    assert K.kev_get_device_errors(stream=sa) == 0           # read and cleared
    # the default stream's word is separate as well
    K.kev_slot_attn_decode(**{**t, "slot_ids": bad_ids, "out": out_a}, stream=sa)
    assert K.kev_get_device_errors() == 0
    assert K.kev_get_device_errors(stream=sa) & K.KEV_DEVERR_SLOT


def test_prefills_and_split_decodes_in_flight_on_several_streams(orc):
    cases = [W.make_prefill([300, 1, 77, 129, 512], 28, 4, 128, W.BF16, seed=21),
             W.make_prefill([17, 900, 64], 32, 8, 128, W.BF16, seed=22)]
    devs = [prefill_dev(c) for c in cases]
    outs = [[torch.empty_like(d[0]) for _ in range(3)] for d in devs]
    dc = W.make_decode(n_req=2, n_slots=6, capacity=900, heads=32, kv_heads=8, head_dim=128, seed=23)
    dd = decode_dev(dc)
    douts = [torch.empty_like(dd["q"]) for _ in range(3)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    say("three rounds of two prefills and a split decode on three streams, no synchronisation between")
    for rnd in range(3):
        for i, s in enumerate(streams):
            if i < 2:
                q, k, v, cu = devs[i]
                K.kev_packed_attn_prefill(q, k, v, cu, out=outs[i][rnd], stream=s)
            else:
                # a 2-request batch splits its units over workgroups: the split states live in
                # the call's workspace; the append rewrites the same rows with the same values
                K.kev_slot_attn_decode(**{**dd, "out": douts[rnd]}, stream=s)
    torch.cuda.synchronize()
    for s in streams:
        assert K.kev_get_device_errors(stream=s) == 0
    for i, c in enumerate(cases):
        ref = orc.prefill_case(c)
        for rnd in range(3):
            assert_parity(to_host_f64(outs[i][rnd]), ref, c.dtype, f"stream {i} round {rnd}")
    ref = orc.decode_case(dc)
    for rnd in range(3):
        assert_parity(to_host_f64(douts[rnd]), ref, W.BF16, f"split decode round {rnd}")


def test_workspace_grows_and_shrinks_without_synchronisation(orc):
    sizes = [[5, 40], [3000, 2000, 1, 4000], [64], [8000, 7000]]
    cases = [W.make_prefill(s, 32, 8, 128, W.BF16, seed=30 + i) for i, s in enumerate(sizes)]
    devs = [prefill_dev(c) for c in cases]
    torch.cuda.synchronize()
    say("prefills of growing and shrinking work lists back to back on one stream")
    outs = [K.kev_packed_attn_prefill(*d) for d in devs]
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    for c, o in zip(cases, outs):
        rows = np.array([0, c.total_tokens - 1, c.total_tokens // 2], np.int32)
        heads = np.array([0, 31, 17], np.int32)
        ref = orc.prefill_rows(c.q, c.k, c.v, c.cu_seqlens, c.heads, c.kv_heads, c.head_dim, c.dtype,
                               rows, heads)
        assert_parity(to_host_f64(o)[rows, heads], ref, c.dtype, f"T={c.total_tokens}")
