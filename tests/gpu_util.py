"""Helpers shared by the GPU tests: host<->device copies of generator output and the parity gate."""
from __future__ import annotations

import sys

import numpy as np
import torch

from segment_isolated_packed_amd import workloads as W

# Parity gate (assert_close style, both bounds must hold):
#   max abs err = max |g - r|                          <= atol
#   max rel err = max |g - r| / max(|r|, atol / rtol)  <= rtol
TOL = {W.BF16: (2e-2, 1e-2), W.F32: (1e-5, 1e-5)}


def say(msg: str):
    """Name the case before each GPU step, flushed, so a lost box still says what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.cuda()


def to_dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def parity(got: np.ndarray, ref: np.ndarray, dtype: str) -> tuple[float, float]:
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), atol / rtol)).max()) if err.size else 0.0
    return max_abs, max_rel


def assert_parity(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    atol, rtol = TOL[dtype]
    max_abs, max_rel = parity(got, ref, dtype)
    print(f"[parity] {what}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} (atol={atol}, rtol={rtol})",
          flush=True)
    assert max_abs <= atol and max_rel <= rtol, (what, max_abs, max_rel)


def prefill_dev(case):
    return (to_dev(case.q, case.dtype), to_dev(case.k, case.dtype), to_dev(case.v, case.dtype),
            to_dev_i32(case.cu_seqlens))


def decode_dev(dc):
    return dict(q=to_dev(dc.q, dc.dtype), kv_pool=to_dev(dc.pool, dc.dtype),
                slot_ids=to_dev_i32(dc.slot_ids), cache_lens=to_dev_i32(dc.cache_lens),
                k_new=to_dev(dc.k_new, dc.dtype), v_new=to_dev(dc.v_new, dc.dtype))


def sample_rows(case, n: int, seed: int = 0):
    """Rows to check one by one: the first and last row of every question plus random rows."""
    rng = np.random.default_rng(seed)
    cu = case.cu_seqlens
    rows = []
    for s in range(case.n_seg):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            rows += [a, b - 1]
    rows += list(rng.integers(0, case.total_tokens, n))
    rows = np.array(rows, dtype=np.int32)
    heads = rng.integers(0, case.heads, len(rows)).astype(np.int32)
    return rows, heads
