"""Seeded synthetic inputs for packed prefill and slot-pool decode.

Both the HIP path (tests, bench) and the oracle's tests draw their inputs
here, so that the two sides see the same bits.  The module holds no
attention arithmetic: it draws random numbers, applies the segment-length
recipes, rounds the drawn fp32 values to bf16 (round to nearest even), and
counts the work and bytes used for reporting.

Workload shapes follow the pages: questions packed back to back into one
token stream with their intervals recorded (Kev article, icman.com.cn, §2.2
and §5.3), the KV slot pool with one fixed-capacity slot per question whose
capacity is 1.2x the P95 length plus 20% reserve slots (Kev part 2,
gsyq.cn, §2.2), and Qwen-shaped head counts (inference-engine primer,
sakurs2.com, §2.1 follows one Qwen3-8B call).

bf16 tensors are carried as ``uint16`` arrays of raw bits; fp32 as float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

BF16 = "bf16"
F32 = "f32"


# ----------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ----------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if dtype != BF16:
        return rng.standard_normal(shape, dtype=np.float32)
    out = np.empty(shape, dtype=np.uint16)   # same draws as one call, in cache-sized pieces
    _normal_into(rng, out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(-1, 1))
    return out


def _normal_into(rng: np.random.Generator, out: np.ndarray, chunk_rows: int = 1 << 12) -> None:
    """Fill a bf16-bits array with N(0,1) draws, chunked along axis 0 to cap host memory."""
    flat = out.reshape(out.shape[0], -1)
    for lo in range(0, flat.shape[0], chunk_rows):
        hi = min(flat.shape[0], lo + chunk_rows)
        flat[lo:hi] = round_to_bf16_bits(rng.standard_normal((hi - lo, flat.shape[1]), dtype=np.float32))


# ----------------------------------------------------------------------------
# segment-length recipes
# ----------------------------------------------------------------------------

def fix_total(x: np.ndarray, total: int, lo: int, hi: int) -> np.ndarray:
    """Scale raw lengths so they sum to exactly ``total`` inside [lo, hi].

    Scale by total/sum, round half to even, clip, then hand out the remaining
    +1/-1 tokens one at a time, cycling over segments in descending-length
    order (stable) and skipping segments already at the bound.
    """
    x = np.asarray(x, dtype=np.float64)
    n = len(x)
    if not (n * lo <= total <= n * hi):
        raise ValueError("total not reachable inside [lo, hi]")
    y = np.clip(np.rint(x * (total / x.sum())), lo, hi).astype(np.int64)
    order = np.argsort(-y, kind="stable")
    diff = int(total - y.sum())
    step = 1 if diff > 0 else -1
    bound = hi if diff > 0 else lo
    pos = 0
    while diff != 0:
        s = order[pos % n]
        pos += 1
        if y[s] == bound:
            continue
        y[s] += step
        diff -= step
    return y


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("too many tokens for int32 cu_seqlens")
    return cu.astype(np.int32)


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------

@dataclass
class PrefillCase:
    name: str
    dtype: str
    heads: int
    kv_heads: int
    head_dim: int
    seqlens: np.ndarray
    seed: int
    q: np.ndarray            # [T, heads, d]     (uint16 bf16 bits or float32)
    k: np.ndarray            # [T, kv_heads, d]
    v: np.ndarray            # [T, kv_heads, d]
    cu_seqlens: np.ndarray = field(init=False)

    def __post_init__(self):
        self.cu_seqlens = cu_from_lengths(self.seqlens)

    @property
    def n_seg(self) -> int:
        return len(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def effective_flops(self) -> int:
        """Unmasked score entries only: 2 FLOP per MAC for QK^T and again for PV."""
        L = self.seqlens.astype(np.int64)
        return int(4 * self.head_dim * self.heads * int((L * (L + 1) // 2).sum()))

    def algorithmic_bytes(self) -> int:
        """Compulsory HBM traffic: read q, k, v once and write out once."""
        T = self.total_tokens
        return int(T * self.head_dim * self.elem_bytes * (2 * self.heads + 2 * self.kv_heads))


@dataclass
class DecodeCase:
    name: str
    dtype: str
    heads: int
    kv_heads: int
    head_dim: int
    n_slots: int
    capacity: int
    seed: int
    slot_ids: np.ndarray     # int32 [n_req], distinct
    cache_lens: np.ndarray   # int32 [n_req], tokens in the slot after the append (1..capacity)
    q: np.ndarray            # [n_req, heads, d]
    k_new: np.ndarray        # [n_req, kv_heads, d]
    v_new: np.ndarray        # [n_req, kv_heads, d]
    pool: np.ndarray         # [n_slots, 2, kv_heads, capacity, d]  (K plane then V plane)

    @property
    def n_req(self) -> int:
        return len(self.slot_ids)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def algorithmic_bytes(self) -> int:
        """Cached K/V rows read + new K/V read and appended + q read + out written."""
        e, d, hk, hq = self.elem_bytes, self.head_dim, self.kv_heads, self.heads
        cached = int((self.cache_lens.astype(np.int64) - 1).sum()) * hk * d * e * 2
        newkv = self.n_req * hk * d * e * 2 * 2
        qo = self.n_req * hq * d * e * 2
        return cached + newkv + qo

    def flops(self) -> int:
        return int(4 * self.head_dim * self.heads * int(self.cache_lens.astype(np.int64).sum()))


def make_prefill(seqlens, heads: int, kv_heads: int, head_dim: int, dtype: str,
                 seed: int, name: str = "custom") -> PrefillCase:
    """Q/K/V ~ N(0,1), drawn in the order q, k, v from ``default_rng(seed)``."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    rng = np.random.default_rng(seed)
    T = int(seqlens.sum())
    q = _normal(rng, (T, heads, head_dim), dtype)
    k = _normal(rng, (T, kv_heads, head_dim), dtype)
    v = _normal(rng, (T, kv_heads, head_dim), dtype)
    return PrefillCase(name, dtype, heads, kv_heads, head_dim, seqlens, seed, q, k, v)


def qwen25_lengths(rng: np.random.Generator, n: int = 8) -> np.ndarray:
    return rng.integers(256, 2049, size=n).astype(np.int64)


def qwen3_lengths(rng: np.random.Generator, n: int = 32, total: int = 24576) -> np.ndarray:
    raw = np.exp(rng.normal(math.log(512.0), 0.8, size=n))
    return fix_total(raw, total, 16, 4096)


def skewed_lengths(rng: np.random.Generator, n: int = 256, total: int = 131072) -> np.ndarray:
    n_long = int(round(0.1 * n))
    n_short = n - n_long
    short = rng.integers(16, 129, size=n_short).astype(np.int64)
    long_raw = rng.integers(2048, 8193, size=n_long).astype(np.float64)
    long = fix_total(long_raw, total - int(short.sum()), 2048, 8192)
    lengths = np.concatenate([short, long])
    return lengths[rng.permutation(n)]


PREFILL_CONFIGS = {
    # name: (dtype, heads, kv_heads, head_dim, lengths recipe, seed)
    "tiny": (F32, 4, 4, 16, lambda rng: np.array([37, 64, 11, 128], dtype=np.int64), 7),
    "qwen25_7b": (BF16, 28, 4, 128, qwen25_lengths, 42),
    "qwen3_8b": (BF16, 32, 8, 128, qwen3_lengths, 43),
    "skewed_long": (BF16, 32, 8, 128, skewed_lengths, 45),
}

PREFILL_DESCRIPTIONS = {
    "tiny": "fp32, 4 heads (MHA), head_dim 16, segments [37,64,11,128]",
    "qwen25_7b": "bf16, 28 q / 4 kv heads, head_dim 128, 8 segments uniform in [256,2048]",
    "qwen3_8b": "bf16, 32 q / 8 kv heads, head_dim 128, 32 lognormal segments (median 512, sigma 0.8) fixed to 24576 tokens within [16,4096]",
    "skewed_long": "bf16, 32 q / 8 kv heads, head_dim 128, 131072 tokens over 256 segments (90% in [16,128], 10% in [2048,8192])",
}


def prefill_lengths(name: str, seed: int | None = None) -> np.ndarray:
    dtype, hq, hk, d, recipe, default_seed = PREFILL_CONFIGS[name]
    rng = np.random.default_rng(default_seed if seed is None else seed)
    return recipe(rng)


def prefill_case(name: str, seed: int | None = None, heads: int | None = None,
                 kv_heads: int | None = None) -> PrefillCase:
    """One of the named prefill workloads; lengths come first from the rng, then q, k, v.

    ``heads``/``kv_heads`` override the head counts (same lengths and draw order),
    which gives smaller cases with the same segment structure.
    """
    dtype, hq, hk, d, recipe, default_seed = PREFILL_CONFIGS[name]
    seed = default_seed if seed is None else seed
    hq = hq if heads is None else heads
    hk = hk if kv_heads is None else kv_heads
    rng = np.random.default_rng(seed)
    lengths = recipe(rng)
    T = int(lengths.sum())
    q = _normal(rng, (T, hq, d), dtype)
    k = _normal(rng, (T, hk, d), dtype)
    v = _normal(rng, (T, hk, d), dtype)
    return PrefillCase(name, dtype, hq, hk, d, lengths, seed, q, k, v)


DECODE_DESCRIPTION = ("bf16, 32 q / 8 kv heads, head_dim 128, 64 requests, slot capacity 2458, "
                      "80-slot pool, cache lengths uniform in [1,2458], new K/V appended in-kernel")


def make_decode(n_req: int = 64, n_slots: int = 80, capacity: int = 2458, heads: int = 32,
                kv_heads: int = 8, head_dim: int = 128, seed: int = 44, dtype: str = BF16,
                cache_lens=None, name: str = "slot_decode") -> DecodeCase:
    """Slot-pool decode inputs.

    Draw order: slot ids (first n_req of a permutation of the pool), cache
    lengths (uniform in [1, capacity], counting the appended token), the whole
    pool (every slot and position filled, so stale rows exist), q, k_new, v_new.
    """
    rng = np.random.default_rng(seed)
    slot_ids = rng.permutation(n_slots)[:n_req].astype(np.int32)
    drawn = rng.integers(1, capacity + 1, size=n_req).astype(np.int32)
    lens = drawn if cache_lens is None else np.asarray(cache_lens, dtype=np.int32)
    shape = (n_slots, 2, kv_heads, capacity, head_dim)
    if dtype == BF16:
        pool = np.empty(shape, dtype=np.uint16)
        _normal_into(rng, pool.reshape(n_slots * 2 * kv_heads * capacity, head_dim))
    else:
        pool = rng.standard_normal(shape, dtype=np.float32)
    q = _normal(rng, (n_req, heads, head_dim), dtype)
    k_new = _normal(rng, (n_req, kv_heads, head_dim), dtype)
    v_new = _normal(rng, (n_req, kv_heads, head_dim), dtype)
    return DecodeCase(name, dtype, heads, kv_heads, head_dim, n_slots, capacity, seed,
                      slot_ids, lens, q, k_new, v_new, pool)


@dataclass
class ChunkedCase:
    """A packed batch of prompt chunks, each continuing the rows already cached in its slot."""
    name: str
    heads: int
    kv_heads: int
    head_dim: int
    n_slots: int
    capacity: int
    seed: int
    seqlens: np.ndarray      # chunk lengths
    prefix_lens: np.ndarray  # int32 [n_seg], rows already in each slot
    slot_ids: np.ndarray     # int32 [n_seg], distinct
    q: np.ndarray            # [T, heads, d]     bf16 bits
    k: np.ndarray            # [T, kv_heads, d]
    v: np.ndarray            # [T, kv_heads, d]
    pool: np.ndarray         # [n_slots, 2, kv_heads, capacity, d]
    dtype: str = BF16
    cu_seqlens: np.ndarray = field(init=False)

    def __post_init__(self):
        self.cu_seqlens = cu_from_lengths(self.seqlens)

    @property
    def n_seg(self) -> int:
        return len(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def effective_flops(self) -> int:
        """Unmasked score entries only (chunk row i of a question with prefix P sees P + i + 1
        keys): 2 FLOP per MAC for QK^T and again for PV."""
        L = self.seqlens.astype(np.int64)
        P = self.prefix_lens.astype(np.int64)
        return int(4 * self.head_dim * self.heads * int((L * P + L * (L + 1) // 2).sum()))

    def algorithmic_bytes(self) -> int:
        """Compulsory HBM traffic: q, k, v and out of the chunk once, the prefix K/V rows
        once, and the chunk's K/V rows written into the slots."""
        T, d = self.total_tokens, self.head_dim
        prefix = int(self.prefix_lens.astype(np.int64).sum())
        return int(2 * d * (T * (2 * self.heads + 2 * self.kv_heads) + 2 * self.kv_heads * (prefix + T)))


def make_chunked(seqlens, prefix_lens, heads: int, kv_heads: int, head_dim: int, capacity: int,
                 n_slots: int, seed: int, name: str = "chunked") -> ChunkedCase:
    """Chunked-prefill inputs (bf16).  Draw order: slot ids (first n_seg of a permutation of
    the pool), the whole pool (every row filled, so rows past each prefix hold stale values a
    correct kernel never reads), q, k, v of the chunks."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32)
    if len(seqlens) != len(prefix_lens) or (prefix_lens + seqlens > capacity).any():
        raise ValueError("every chunk must fit its slot after its prefix")
    rng = np.random.default_rng(seed)
    slot_ids = rng.permutation(n_slots)[:len(seqlens)].astype(np.int32)
    pool = np.empty((n_slots, 2, kv_heads, capacity, head_dim), dtype=np.uint16)
    _normal_into(rng, pool.reshape(-1, head_dim))
    T = int(seqlens.sum())
    q = _normal(rng, (T, heads, head_dim), BF16)
    k = _normal(rng, (T, kv_heads, head_dim), BF16)
    v = _normal(rng, (T, kv_heads, head_dim), BF16)
    return ChunkedCase(name, heads, kv_heads, head_dim, n_slots, capacity, seed, seqlens, prefix_lens,
                       slot_ids, q, k, v, pool)


CHUNKED_DESCRIPTION = ("bf16, 28 q / 4 kv heads, head_dim 128 (Qwen2.5-7B attention shape): 8 prompts of "
                       "8192 tokens prefilled in 2048-token chunks; the packed batch holds chunk s mod 4 of "
                       "prompt s, so prefixes are 0, 2048, 4096, 6144 (twice each); 12-slot pool of capacity 8192")


def chunked_case(seed: int = 46) -> ChunkedCase:
    """The chunked-prefill workload: the batch a chunked scheduler would run once 8 long
    prompts are spread over the four chunk phases (16384 new tokens against 24576 cached)."""
    prefix = np.array([(s % 4) * 2048 for s in range(8)], np.int32)
    return make_chunked([2048] * 8, prefix, 28, 4, 128, capacity=8192, n_slots=12, seed=seed,
                        name="chunked_qwen25_7b")



@dataclass
class PagedDecodeCase:
    """Decode inputs over a paged pool: request r's position p lives in block
    block_tables[r, p // block_size], row p % block_size."""
    name: str
    heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    seed: int
    block_tables: np.ndarray  # int32 [n_req, max_blocks]; unused entries -1
    cache_lens: np.ndarray    # int32 [n_req], positions after the append
    q: np.ndarray             # [n_req, heads, d]
    k_new: np.ndarray         # [n_req, kv_heads, d]
    v_new: np.ndarray
    pool: np.ndarray          # [n_blocks, 2, kv_heads, block_size, d]
    dtype: str = BF16

    @property
    def n_req(self) -> int:
        return len(self.cache_lens)

    @property
    def n_blocks(self) -> int:
        return self.pool.shape[0]

    def blocks_in_use(self) -> int:
        return int(((self.cache_lens.astype(np.int64) + self.block_size - 1) // self.block_size).sum())

    def algorithmic_bytes(self) -> int:
        """As for the slot decode, plus the block ids each request reads."""
        d, hk, hq = self.head_dim, self.kv_heads, self.heads
        cached = int((self.cache_lens.astype(np.int64) - 1).sum()) * hk * d * 2 * 2
        return cached + self.n_req * (hk * d * 2 * 2 * 2 + hq * d * 2 * 2) + 4 * self.blocks_in_use()


def paged_from_slots(dc: DecodeCase, block_size: int, spare_blocks: int = 0, seed: int = 47) -> PagedDecodeCase:
    """The same decode step over a paged pool: each request's cached rows are cut into blocks
    of `block_size` positions (only as many as its length needs, as an on-demand allocator
    would hand out; a block past the slot's capacity is zero-padded) and scattered over a pool
    of shuffled blocks, plus `spare_blocks` unused ones.  Decoding it must give the slot decode's output, and the pools after the append
    hold the same rows."""
    rng = np.random.default_rng(seed)
    B = block_size
    need = (dc.cache_lens.astype(np.int64) + B - 1) // B
    n_blocks = int(need.sum()) + spare_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    max_blocks = max(int(need.max()), 1)
    tables = np.full((dc.n_req, max_blocks), -1, np.int32)
    pool = np.zeros((n_blocks, 2, dc.kv_heads, B, dc.head_dim), dtype=dc.pool.dtype)
    if spare_blocks > 0:
        spare = np.empty((spare_blocks,) + pool.shape[1:], dtype=pool.dtype)
        _normal_into(rng, spare.reshape(-1, dc.head_dim))
        pool[perm[n_blocks - spare_blocks:]] = spare
    nxt = 0
    for r in range(dc.n_req):
        s, L = int(dc.slot_ids[r]), int(dc.cache_lens[r])
        for j in range(int(need[r])):
            b = int(perm[nxt])
            nxt += 1
            tables[r, j] = b
            rows = dc.pool[s, :, :, j * B:min((j + 1) * B, dc.capacity)]
            pool[b, :, :, :rows.shape[2]] = rows
    return PagedDecodeCase(f"{dc.name}_paged{B}", dc.heads, dc.kv_heads, dc.head_dim, B, seed, tables,
                           dc.cache_lens.copy(), dc.q, dc.k_new, dc.v_new, pool)


def slots_from_paged_pool(pc: PagedDecodeCase, pool: np.ndarray, dc: DecodeCase) -> np.ndarray:
    """Rows 0..L-1 of every request gathered back from a paged pool into dc's slot layout
    (a copy of dc.pool with those rows replaced)."""
    out = dc.pool.copy()
    B = pc.block_size
    for r in range(pc.n_req):
        s, L = int(dc.slot_ids[r]), int(pc.cache_lens[r])
        for j in range((L + B - 1) // B):
            n = min(B, L - j * B)
            out[s, :, :, j * B:j * B + n] = pool[pc.block_tables[r, j], :, :, :n]
    return out
