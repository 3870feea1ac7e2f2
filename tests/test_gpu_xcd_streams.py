"""XCD-aware item streams (fewer KV heads than XCDs, 8 to 64 questions): every item is computed
the same way wherever it runs, so the outputs and the stored K/V are bit for bit those of the
plain question-major launch (KEV_XCD_STREAMS=0), for packed and chunked prefill, with empty and
one-row questions in the batch."""
import numpy as np
import pytest
import torch

import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import prefill_dev, say, to_dev, to_dev_i32, to_host_bits

pytestmark = pytest.mark.gpu


def both_ways(monkeypatch, fn):
    monkeypatch.setenv("KEV_XCD_STREAMS", "0")
    plain = fn()
    monkeypatch.delenv("KEV_XCD_STREAMS")
    streamed = fn()
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    return plain, streamed


@pytest.mark.parametrize("lens,hq", [([700, 1, 0, 2048, 129, 64, 1500, 33], 28),
                                     ([5, 300, 2000, 17, 0, 900, 1, 1, 4000, 250, 64, 640], 16),
                                     ([1024] * 8, 32)])
def test_packed_prefill_streams_bitwise(monkeypatch, lens, hq):
    case = W.make_prefill(lens, hq, 4, 128, W.BF16, seed=len(lens) * 7 + hq)
    q, k, v, cu = prefill_dev(case)
    say(f"prefill streams vs plain: {len(lens)} questions, {hq}/4 heads")
    plain, streamed = both_ways(monkeypatch, lambda: to_host_bits(K.kev_packed_attn_prefill(q, k, v, cu)))
    assert np.array_equal(plain, streamed)


def test_chunked_prefill_streams_bitwise(monkeypatch):
    cc = W.make_chunked([512, 700, 1, 300, 64, 1000, 128, 0, 2048], [0, 300, 900, 1500, 0, 64, 3000, 10, 1024],
                        28, 4, 128, capacity=4096, n_slots=11, seed=81)
    args = [to_dev(x, W.BF16) for x in (cc.q, cc.k, cc.v)]
    cu, ids, pre = (to_dev_i32(x) for x in (cc.cu_seqlens, cc.slot_ids, cc.prefix_lens))
    say("chunked prefill streams vs plain: 9 questions, 28/4 heads")

    def run():
        pool = to_dev(cc.pool, W.BF16)
        out = K.kev_chunked_prefill_slots(*args, cu, pool, ids, pre)
        return to_host_bits(out), to_host_bits(pool)

    (po, pp), (so, sp) = both_ways(monkeypatch, run)
    assert np.array_equal(po, so) and np.array_equal(pp, sp)
