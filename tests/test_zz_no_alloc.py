"""The no-allocation prefill (kev_packed_attn_prefill_noalloc) through the C ABI: the same
results as kev_packed_attn_prefill, bit for bit, on two calls in a row (the second smaller, so
it runs over what the first left in the shared device scratch), device-array errors reported
by kev_get_device_errors, and work lists past the scratch refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import prefill_dev, say, to_dev_i32, to_host_bits

pytestmark = pytest.mark.gpu


def test_noalloc_matches_the_allocating_prefill_on_two_calls_in_a_row():
    cases = [W.make_prefill([300, 1, 77, 129, 2048, 0, 513], 32, 8, 128, W.BF16, seed=71),
             W.make_prefill([40, 9], 28, 4, 128, W.BF16, seed=72)]
    for i, c in enumerate(cases):
        q, k, v, cu = prefill_dev(c)
        say(f"noalloc prefill call {i}: T={c.total_tokens} heads={c.heads}/{c.kv_heads}")
        ref = K.kev_packed_attn_prefill(q, k, v, cu)
        got = torch.full_like(q, float("nan"))
        K.kev_packed_attn_prefill_noalloc(q, k, v, cu, out=got)
        torch.cuda.synchronize()
        assert K.kev_get_device_errors() == 0
        assert np.array_equal(to_host_bits(got), to_host_bits(ref)), f"call {i} differs"


def test_noalloc_fp32_and_head_dim_64():
    for c in (W.prefill_case("tiny"), W.make_prefill([300, 1, 77], 8, 2, 64, W.BF16, seed=73)):
        q, k, v, cu = prefill_dev(c)
        say(f"noalloc prefill {c.dtype} d={c.head_dim}")
        ref = K.kev_packed_attn_prefill(q, k, v, cu)
        got = torch.empty_like(q)
        K.kev_packed_attn_prefill_noalloc(q, k, v, cu, out=got)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(got), to_host_bits(ref))


def test_noalloc_device_errors_and_scratch_limit():
    c = W.make_prefill([30, 50], 8, 2, 128, W.BF16, seed=74)
    q, k, v, _ = prefill_dev(c)
    out = torch.zeros_like(q)
    say("noalloc prefill with cu_seqlens that do not end at total_tokens (device guard)")
    K.kev_packed_attn_prefill_noalloc(q, k, v, to_dev_i32([0, 30, 70]), out=out)
    assert K.kev_get_device_errors() & K.KEV_DEVERR_SEQLENS
    assert K.kev_get_device_errors() == 0           # read and cleared
    assert bool((out == 0).all())                   # nothing computed
    L = K.load_library()
    p = ctypes.c_void_p(16)
    rc = L.kev_packed_attn_prefill_noalloc(p, p, p, p, 1, 32, 8, 128, p, 8 << 20, K.KEV_BF16, None)
    assert rc == K.KEV_ERR_SCRATCH_LIMIT
