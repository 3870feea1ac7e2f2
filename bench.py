"""Benchmark of the packed-prefill + slot-decode hot path on one MI355X.

One step = one packed prefill over the skewed long workload (bf16, 32 q / 8 kv heads,
head_dim 128, 131072 tokens over 256 questions: 90% of lengths in [16,128], 10% in
[2048,8192], seed 45) followed by one slot-pool decode (bf16, 32 q / 8 kv heads, 64
requests, slot capacity 2458, 80-slot pool, new K/V appended in-kernel, seed 44).  Between
the two a 512 MiB buffer is read so the decode reads its KV rows from HBM rather than from
the 256 MB MALL.  ``--workload`` selects another prefill shape for the step.

Prints ONE JSON line.  `value` is the prefill's effective TFLOP/s (only unmasked score
entries counted: 4 * d * heads * sum L(L+1)/2 FLOPs per call) over the average duration of
the prefill call (work-list pass + attention kernel) measured with HIP events on the launch
stream (created without the system-scope fence, so that recording them adds no cache
write-back and invalidation between the calls); `roofline.achieved` divides the same FLOPs by the attention kernel's own average
duration, taken with events the library records around that launch on the call's stream.
The decode's achieved HBM GB/s (algorithmic bytes over event-timed duration) is reported
beside it, per call and per kernel.  More calls are timed the same way: the other prefill
shapes, the prefill that also stores every question's K/V into its slot, a chunked prefill
of 8 long prompts against their cached prefixes, the decode over a paged (block-table)
pool holding the same rows, the decode of batches cut to 1, 4 and 16 requests, and the
decode at scaled lengths (fixed cost and streaming rate per call).  The CPU oracle is
timed on the host cores on bounded samples of every prefill shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBPS = 8000.0        # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources whose change invalidates a kernel's recorded HBM traffic: the kernel itself and
# everything that decides its launch and item order (the work-list pass and the call).
PREFILL_SOURCES = ["kev_prefill_bf16.hip", "kev_mfma_core.h", "kev_internal.h", "kev_tiles.h",
                   "kev_schedule.hip", "kev_api.hip"]
DECODE_SOURCES = ["kev_decode.hip", "kev_mfma_core.h", "kev_internal.h", "kev_api.hip"]
STORE_SOURCES = ["kev_store_kv.hip", "kev_internal.h", "kev_api.hip"]
PREFILL_NAMES = ("qwen25_7b", "qwen3_8b", "skewed_long")


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "segment_isolated_packed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of
    `kernel` on `workload`, or None if there is none or the sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{kernel}/{workload}")
    if not e or e.get("source_sha256") != src_hash:
        return None
    return e.get("bytes_per_launch")


class TimingEvent:
    """A HIP event used only for timing: created with hipEventDisableSystemFence, so recording it
    adds no system-scope cache write-back and invalidation between the calls it brackets (HIP
    documents the flag for events that only measure time).  Same interface as the parts of
    torch.cuda.Event used here; `cuda_event` is the raw handle the library's kernel-event hook
    takes."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            import torch
            # the HIP runtime torch has loaded: its streams are the ones recorded on here
            with open("/proc/self/maps") as f:
                paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
            torch_dir = os.path.dirname(os.path.abspath(torch.__file__))
            paths.sort(key=lambda q: not q.startswith(torch_dir))
            if not paths:
                raise RuntimeError("no HIP runtime loaded in this process")
            h = ctypes.CDLL(paths[0])
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        h = self._runtime()
        e = ctypes.c_void_p()
        if h.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self._e = e
        self.cuda_event = e.value

    def record(self, stream):
        import ctypes
        if self._runtime().hipEventRecord(self._e, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        if self._runtime().hipEventElapsedTime(ctypes.byref(ms), self._e, end._e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def _sample_pairs(case, rng, n):
    """n (row, head) pairs drawn uniformly over the workload, with their effective FLOPs."""
    import numpy as np
    rows = rng.integers(0, case.total_tokens, n).astype(np.int32)
    heads = rng.integers(0, case.heads, n).astype(np.int32)
    seg = np.searchsorted(case.cu_seqlens, rows, side="right") - 1
    keys = rows - case.cu_seqlens[seg] + 1
    return rows, heads, int(4 * case.head_dim * int(keys.astype(np.int64).sum()))


def time_oracle_rows(orc, case, budget_s: float, n_threads: int, chunk: int = 4096) -> dict:
    """The oracle on (row, head) pairs sampled uniformly from the workload, chunk by chunk
    until about budget_s seconds of compute have passed."""
    import numpy as np
    rng = np.random.default_rng(1234)
    flops = pairs = 0
    dt = 0.0
    while dt < budget_s:
        rows, heads, f = _sample_pairs(case, rng, chunk)
        t0 = time.perf_counter()
        orc.prefill_rows(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads,
                         case.head_dim, case.dtype, rows, heads, n_threads=n_threads)
        dt += time.perf_counter() - t0
        flops += f
        pairs += chunk
    return {"tflops": flops / dt / 1e12, "seconds": dt, "threads": n_threads,
            "sample": f"{pairs} (row, query head) outputs drawn uniformly over the workload, "
                      f"{flops / 1e9:.1f} GFLOP effective"}


def time_oracle_full(orc, case, n_threads: int) -> dict:
    t0 = time.perf_counter()
    orc.prefill(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads, case.head_dim,
                case.dtype, n_threads=n_threads)
    dt = time.perf_counter() - t0
    return {"tflops": case.effective_flops() / dt / 1e12, "seconds": dt, "threads": n_threads,
            "sample": f"whole workload ({case.n_seg} questions, {case.heads} heads, "
                      f"{case.effective_flops() / 1e9:.2f} GFLOP effective)"}


def oracle_timing(headline: str, budget_s: float) -> tuple[dict, dict]:
    """The oracle as it stands, on the host cores: threaded over all cores on every prefill
    shape (whole workload where it takes seconds, uniform row samples otherwise) and
    single-threaded on the tiny and Qwen2.5-7B shapes.  Returns (cpu_baseline of the
    headline workload, every timing)."""
    import oracle
    from segment_isolated_packed_amd import workloads as W
    orc = oracle.get()
    cores = orc.max_threads()          # read before any single-threaded call changes it
    res = {"cores": cores}
    tiny = W.prefill_case("tiny")
    res["tiny"] = {"threaded": time_oracle_full(orc, tiny, cores),
                   "single_thread": time_oracle_full(orc, tiny, 1)}
    for name in PREFILL_NAMES:
        log(f"oracle timing: {name}")
        c = W.prefill_case(name)
        entry = {}
        if name == "skewed_long":
            entry["threaded"] = time_oracle_rows(orc, c, budget_s, cores)
        else:
            entry["threaded"] = time_oracle_full(orc, c, cores)
        if name == "qwen25_7b":
            entry["single_thread"] = time_oracle_rows(orc, c, budget_s / 3, 1, chunk=256)
        res[name] = entry
        del c
    h = res[headline]["threaded"]
    base = {"value": h["tflops"], "unit": "TFLOP/s", "cores": h["threads"], "kind": "oracle",
            "sample": f"fp64 oracle ({W.PREFILL_DESCRIPTIONS[headline]}): {h['sample']}, "
                      f"{h['seconds']:.1f} s on {h['threads']} threads"}
    return base, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skewed_long", choices=list(PREFILL_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-budget", type=float, default=20.0,
                    help="seconds of oracle compute per sampled leg")
    ap.add_argument("--back-to-back", action="store_true",
                    help="also time 100 prefill calls per event pair (throughput of calls issued "
                         "one after another; off by default so that profiler averages of the "
                         "attention kernel cover the timed and roofline calls only)")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="time only the prefill and decode calls of the step (profiling runs whose "
                         "per-kernel averages must not mix in the other legs' launches)")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="how the 256 MB MALL is evicted before each decode: read a 512 MiB "
                         "buffer (default), write it, or not at all")
    ap.add_argument("--only", choices=["prefill", "decode", "chunked", "copy"], default=None,
                    help="run one half of the step, or a 1 GiB device copy that calibrates "
                         "the HBM byte counters (profiling runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU; the path shards by question or KV head "
              "with no exchange step, and multi-GPU runs are not part of it (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import segment_isolated_packed_amd as K
    from segment_isolated_packed_amd import workloads as W

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")

    def to_dev(a, dtype):
        if dtype == W.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def new_events(n, k):
        """n groups of k timing events (TimingEvent: no system-scope fence when recorded)."""
        torch.cuda.synchronize()
        return [[TimingEvent() for _ in range(k)] for _ in range(n)]

    if args.only == "copy":
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 2 * src.numel(), "launches": args.warmup + args.steps}))
        return

    do_pre = args.only in (None, "prefill")
    do_dec = args.only in (None, "decode")
    pc = dc = None
    if do_pre:
        log(f"generating {args.workload} prefill inputs")
        pc = W.prefill_case(args.workload)
        q, k, v = (to_dev(x, pc.dtype) for x in (pc.q, pc.k, pc.v))
        cu = torch.from_numpy(pc.cu_seqlens).to(dev)
        out = torch.empty_like(q)
    flush_buf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    flush_rows = flush_buf.view(torch.int32).view(512, 1 << 18)   # summed in place: read only
    flush_sink = torch.zeros(512, dtype=torch.int32, device=dev)

    def flush():
        if args.flush == "read":
            torch.sum(flush_rows, dim=1, dtype=torch.int32, out=flush_sink)
        elif args.flush == "write":
            flush_buf.fill_(1)

    if do_dec:
        log("generating slot-decode inputs")
        dc = W.make_decode()
        dq, dpool, dkn, dvn = (to_dev(x, dc.dtype) for x in (dc.q, dc.pool, dc.k_new, dc.v_new))
        dids = torch.from_numpy(dc.slot_ids).to(dev)
        dlens = torch.from_numpy(dc.cache_lens).to(dev)
        dout = torch.empty_like(dq)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if do_pre:
            if ev: ev[0].record(stream)
            K.kev_packed_attn_prefill(q, k, v, cu, out=out)
            if ev: ev[1].record(stream)
        if do_dec:
            flush()
            if ev: ev[2].record(stream)
            K.kev_slot_attn_decode(dq, dpool, dids, dlens, dkn, dvn, out=dout)
            if ev: ev[3].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    errs = K.kev_get_device_errors()
    if errs:
        raise RuntimeError(f"device error flags {errs}")

    events = new_events(args.steps, 4)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")

    # The main kernels alone (roofline): the same calls again, with events that the library
    # records around that kernel's launch on the call's stream (kept out of the timed steps,
    # whose call times they would lengthen).
    pre_kernel_ms = dec_kernel_ms = dec_fenced_ms = float("nan")
    pre_b2b_ms = None
    if do_pre:
        kev = new_events(args.steps, 2)
        for e in kev:
            K.kev_set_kernel_events(e[0], e[1])
            K.kev_packed_attn_prefill(q, k, v, cu, out=out)
            K.kev_set_kernel_events(None, None)
        torch.cuda.synchronize()
        pre_kernel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
        # Back-to-back calls (one event pair around 100 launches, 5 repeats, median): the
        # throughput a caller issuing prefills one after another sees.
        b2b = []
        for _ in range(5 if args.back_to_back else 0):
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(stream)
            for _ in range(100):
                K.kev_packed_attn_prefill(q, k, v, cu, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            b2b.append(e0.elapsed_time(e1) / 100)
        pre_b2b_ms = float(np.median(b2b)) if b2b else None
    if do_dec:
        kev = new_events(args.steps, 2)
        for e in kev:
            flush()
            K.kev_set_kernel_events(e[0], e[1])
            K.kev_slot_attn_decode(dq, dpool, dids, dlens, dkn, dvn, out=dout)
            K.kev_set_kernel_events(None, None)
        torch.cuda.synchronize()
        dec_kernel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
        # The same call between torch's default events, whose recording also writes back and
        # invalidates the caches at system scope (reported beside the call rate, not as it).
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e in fev:
            flush()
            e[0].record(stream)
            K.kev_slot_attn_decode(dq, dpool, dids, dlens, dkn, dvn, out=dout)
            e[1].record(stream)
        torch.cuda.synchronize()
        dec_fenced_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
    if K.kev_get_device_errors():
        raise RuntimeError("device error flags in the kernel-timing pass")

    extra = not args.no_extra_legs

    # Prefill-to-slot handoff (kev_packed_attn_prefill_slots) on the step's prefill workload:
    # every question's K/V rows stored into its own slot of a pool sized for its longest
    # question.  The store kernel's own duration comes from the profiler trace, not from here.
    slots_res = None
    if extra and do_pre and pc.dtype == W.BF16:
        cap = int(max(pc.seqlens.max(), 1))
        spool = torch.zeros((pc.n_seg + 4, 2, pc.kv_heads, cap, pc.head_dim), dtype=torch.bfloat16, device=dev)
        sids = torch.arange(pc.n_seg, dtype=torch.int32, device=dev)
        for _ in range(2):
            K.kev_packed_attn_prefill_slots(q, k, v, cu, spool, sids, out=out)
        sev = new_events(args.steps, 2)
        for e in sev:
            e[0].record(stream)
            K.kev_packed_attn_prefill_slots(q, k, v, cu, spool, sids, out=out)
            e[1].record(stream)
        torch.cuda.synchronize()
        if K.kev_get_device_errors():
            raise RuntimeError("device error flags in the prefill-to-slot leg")
        s_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
        slots_res = {"ms": s_ms, "store_bytes": 2 * 2 * pc.total_tokens * pc.kv_heads * pc.head_dim * 2,
                     "slot_capacity": cap,
                     "call": "kev_packed_attn_prefill_slots: prefill + every question's K/V stored "
                             "into its slot (store_kv_kernel, timed in the profiler trace)"}
        del spool

    # The decode over a paged pool (kev_paged_attn_decode): the same requests and rows cut into
    # blocks of B positions scattered over a pool of only the blocks the lengths need.
    paged_res = []
    if extra and do_dec:
        for B in (16, 64):
            log(f"paged decode, block size {B}")
            pg = W.paged_from_slots(dc, B)
            ppool, pq, pkn, pvn = (to_dev(x, W.BF16) for x in (pg.pool, pg.q, pg.k_new, pg.v_new))
            ptab, plen = (torch.from_numpy(x).to(dev) for x in (pg.block_tables, pg.cache_lens))
            pout = torch.empty_like(pq)
            pev = new_events(args.steps, 2)
            for i in range(max(args.warmup, 1) + args.steps):
                flush()
                e = pev[i - max(args.warmup, 1)] if i >= max(args.warmup, 1) else None
                if e: e[0].record(stream)
                K.kev_paged_attn_decode(pq, ppool, ptab, plen, pkn, pvn, out=pout)
                if e: e[1].record(stream)
            torch.cuda.synchronize()
            if K.kev_get_device_errors():
                raise RuntimeError("device error flags in the paged-decode leg")
            ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))
            paged_res.append({
                "block_size": B, "ms": ms, "gbps": pg.algorithmic_bytes() / (ms * 1e-3) / 1e9,
                "algorithmic_mb": pg.algorithmic_bytes() / 1e6, "blocks": pg.n_blocks,
                "pool_mb": pg.pool.nbytes / 1e6, "slot_pool_mb": dc.pool.nbytes / 1e6,
                "rows_used": int(dc.cache_lens.sum()), "rows_reserved_paged": pg.n_blocks * B,
                "rows_reserved_slots": dc.n_slots * dc.capacity})
            del ppool, pq, pkn, pvn, pout

    # A batch that has shrunk as requests finished: the first n requests of the decode workload
    # (same pool), with the automatic split of units over workgroups and with splitting off.
    low_res = []
    if extra and do_dec:
        for n in (1, 4, 16):
            lq, lkn, lvn = dq[:n].contiguous(), dkn[:n].contiguous(), dvn[:n].contiguous()
            lids, llens = dids[:n].contiguous(), dlens[:n].contiguous()
            lout = torch.empty_like(lq)
            L = dc.cache_lens[:n].astype(np.int64)
            lbytes = int((L - 1).sum()) * dc.kv_heads * dc.head_dim * 2 * 2 + \
                n * (dc.kv_heads * dc.head_dim * 2 * 2 * 2 + dc.heads * dc.head_dim * 2 * 2)
            row = {"n_req": n, "algorithmic_mb": lbytes / 1e6, "max_len": int(L.max())}
            prev = os.environ.pop("KEV_DECODE_SPLITS", None)
            for mode in ("auto", "unsplit"):
                if mode == "unsplit":
                    os.environ["KEV_DECODE_SPLITS"] = "1"
                lev = new_events(args.steps, 2)
                for i in range(max(args.warmup, 1) + args.steps):
                    flush()
                    e = lev[i - max(args.warmup, 1)] if i >= max(args.warmup, 1) else None
                    if e: e[0].record(stream)
                    K.kev_slot_attn_decode(lq, dpool, lids, llens, lkn, lvn, out=lout)
                    if e: e[1].record(stream)
                torch.cuda.synchronize()
                os.environ.pop("KEV_DECODE_SPLITS", None)
                if prev is not None:
                    os.environ["KEV_DECODE_SPLITS"] = prev
                ms = float(np.mean([e[0].elapsed_time(e[1]) for e in lev]))
                row[mode] = {"us": ms * 1e3, "gbps": lbytes / (ms * 1e-3) / 1e9}
            low_res.append(row)
        if K.kev_get_device_errors():
            raise RuntimeError("device error flags in the low-occupancy decode leg")

    # Decode time against bytes: the decode workload with every length scaled by f (the appends
    # land at the scaled rows, after every other decode leg has run).  A line through the
    # points splits a call into a fixed cost and a steady streaming rate.
    scale_res = None
    if extra and do_dec:
        log("decode time vs bytes")
        pts = []
        for f in (0.125, 0.25, 0.5, 0.75, 1.0):
            L = np.maximum(1, np.round(dc.cache_lens * f)).astype(np.int32)
            slens = torch.from_numpy(L).to(dev)
            sbytes = int((L.astype(np.int64) - 1).sum()) * dc.kv_heads * dc.head_dim * 2 * 2 + \
                dc.n_req * (dc.kv_heads * dc.head_dim * 2 * 2 * 2 + dc.heads * dc.head_dim * 2 * 2)
            sev = new_events(args.steps, 2)
            for i in range(max(args.warmup, 1) + args.steps):
                flush()
                e = sev[i - max(args.warmup, 1)] if i >= max(args.warmup, 1) else None
                if e: e[0].record(stream)
                K.kev_slot_attn_decode(dq, dpool, dids, slens, dkn, dvn, out=dout)
                if e: e[1].record(stream)
            torch.cuda.synchronize()
            pts.append((f, sbytes, float(np.mean([e[0].elapsed_time(e[1]) for e in sev])) * 1e3))
        if K.kev_get_device_errors():
            raise RuntimeError("device error flags in the decode scaling leg")
        slope, icpt = np.polyfit([p[1] for p in pts], [p[2] for p in pts], 1)
        scale_res = {"length_scales": [p[0] for p in pts], "algorithmic_mb": [p[1] / 1e6 for p in pts],
                     "us": [p[2] for p in pts], "fixed_us": float(icpt),
                     "steady_gbps": float(1e-3 / slope) if slope > 0 else None,
                     "note": "least-squares line: call time = fixed_us + bytes / steady rate (MALL flushed)"}

    # The other prefill shapes (parity-test cases; reported beside `value`, not as it).
    other_res = {}
    if extra and do_pre:
        for name in PREFILL_NAMES:
            if name == args.workload:
                continue
            log(f"prefill {name}")
            oc = W.prefill_case(name)
            oq, ok_, ov = (to_dev(x, oc.dtype) for x in (oc.q, oc.k, oc.v))
            ocu = torch.from_numpy(oc.cu_seqlens).to(dev)
            oout = torch.empty_like(oq)
            for _ in range(2):
                K.kev_packed_attn_prefill(oq, ok_, ov, ocu, out=oout)
            oev = new_events(args.steps, 4)
            for e in oev:
                e[0].record(stream)
                K.kev_set_kernel_events(e[2], e[3])
                K.kev_packed_attn_prefill(oq, ok_, ov, ocu, out=oout)
                K.kev_set_kernel_events(None, None)
                e[1].record(stream)
            torch.cuda.synchronize()
            if K.kev_get_device_errors():
                raise RuntimeError(f"device error flags in the {name} prefill leg")
            cms = float(np.mean([e[0].elapsed_time(e[1]) for e in oev]))
            kms = float(np.mean([e[2].elapsed_time(e[3]) for e in oev]))
            ktf = oc.effective_flops() / (kms * 1e-3) / 1e12
            other_res[name] = {"tokens": oc.total_tokens, "effective_gflop": oc.effective_flops() / 1e9,
                               "call_ms": cms, "call_tflops": oc.effective_flops() / (cms * 1e-3) / 1e12,
                               "kernel_ms": kms, "kernel_tflops": ktf, "kernel_frac": ktf / PEAK_BF16_TFLOPS,
                               "kernel_hbm_bytes_per_launch": traffic_for("prefill_r48_kernel", name,
                                                                          source_hash(PREFILL_SOURCES)),
                               "workload": W.PREFILL_DESCRIPTIONS[name]}
            del oq, ok_, ov, oout

    # Chunked prefill against slot prefixes (kev_chunked_prefill_slots) on its own workload:
    # 8 long prompts at four different chunk phases, packed into one call.
    chunk_res = None
    if (extra and args.only is None) or args.only == "chunked":
        log("generating chunked-prefill inputs")
        cc = W.chunked_case()
        cq, ck, cv, cpool = (to_dev(x, W.BF16) for x in (cc.q, cc.k, cc.v, cc.pool))
        ccu, cids, cpre = (torch.from_numpy(x).to(dev) for x in (cc.cu_seqlens, cc.slot_ids, cc.prefix_lens))
        cout = torch.empty_like(cq)
        for _ in range(max(args.warmup, 1)):
            K.kev_chunked_prefill_slots(cq, ck, cv, ccu, cpool, cids, cpre, out=cout)
        cev = new_events(args.steps, 4)
        for e in cev:
            e[0].record(stream)
            K.kev_set_kernel_events(e[2], e[3])
            K.kev_chunked_prefill_slots(cq, ck, cv, ccu, cpool, cids, cpre, out=cout)
            K.kev_set_kernel_events(None, None)
            e[1].record(stream)
        torch.cuda.synchronize()
        if K.kev_get_device_errors():
            raise RuntimeError("device error flags in the chunked-prefill leg")
        c_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in cev]))
        ck_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in cev]))
        c_tf = cc.effective_flops() / (c_ms * 1e-3) / 1e12
        chunk_res = {
            "ms": c_ms, "effective_tflops": c_tf, "pct_peak": c_tf / PEAK_BF16_TFLOPS * 100,
            "kernel_ms": ck_ms, "kernel_tflops": cc.effective_flops() / (ck_ms * 1e-3) / 1e12,
            "effective_gflop": cc.effective_flops() / 1e9, "algorithmic_mb": cc.algorithmic_bytes() / 1e6,
            "workload": W.CHUNKED_DESCRIPTION, "seed": cc.seed,
            "kernel_hbm_bytes_per_launch": traffic_for("prefill_r48_kernel_prefix", "chunked_qwen25_7b",
                                                       source_hash(PREFILL_SOURCES)),
            "call": "kev_chunked_prefill_slots: scheduler + prefill_r48_kernel<true> (prefix) + K/V append"}
        del cq, ck, cv, cpool, cout

    pre_ms = [e[0].elapsed_time(e[1]) for e in events] if do_pre else [float("nan")]
    dec_ms = [e[2].elapsed_time(e[3]) for e in events] if do_dec else [float("nan")]
    pre_avg = float(np.mean(pre_ms))
    dec_avg = float(np.mean(dec_ms))
    flops = pc.effective_flops() if do_pre else 0
    dbytes = dc.algorithmic_bytes() if do_dec else 0
    tflops = flops / (pre_avg * 1e-3) / 1e12 if do_pre else None
    kernel_tflops = flops / (pre_kernel_ms * 1e-3) / 1e12 if do_pre else None
    gbps = dbytes / (dec_avg * 1e-3) / 1e9 if do_dec else None
    dec_kernel_gbps = dbytes / (dec_kernel_ms * 1e-3) / 1e9 if do_dec else None

    result = {
        "metric": "effective TFLOP/s packed prefill (% MFMA peak); decode HBM GB/s (% peak)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, lengths per the workload recipe)",
        "config": {
            "workload": f"{args.workload} packed prefill + slot-pool decode",
            "prefill": W.PREFILL_DESCRIPTIONS[args.workload],
            "prefill_seed": pc.seed if pc else None,
            "prefill_tokens": pc.total_tokens if pc else None,
            "prefill_effective_gflop": flops / 1e9,
            "decode": W.DECODE_DESCRIPTION,
            "decode_seed": dc.seed if dc else None,
            "decode_algorithmic_mb": dbytes / 1e6,
            "step": f"prefill call (scheduler + attention kernel), 512 MiB MALL flush ({args.flush}), decode call",
            "timing": "HIP events created with hipEventDisableSystemFence around each call and, for the "
                      "roofline, around each kernel launch (no system-scope cache write-back and "
                      "invalidation at the events)",
        },
        "prefill_ms": pre_avg,
        "prefill_pct_peak": tflops / PEAK_BF16_TFLOPS * 100 if tflops else None,
        "roofline": {
            "bound": "mfma", "achieved": kernel_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": kernel_tflops / PEAK_BF16_TFLOPS if kernel_tflops else None,
            "traffic": traffic_for("prefill_r48_kernel", args.workload, source_hash(PREFILL_SOURCES)),
            "kernel": "kev prefill_r48_kernel<false> (the head_dim-128 attention kernel; events recorded "
                      "by the library around its launch on the call's stream)",
            "kernel_ms": pre_kernel_ms,
            "algorithmic_flops_per_launch": flops,
            "call_ms": pre_avg,
            "call_tflops": tflops,
            "call_frac": tflops / PEAK_BF16_TFLOPS if tflops else None,
            "back_to_back_call_ms": pre_b2b_ms,
            "back_to_back_tflops": flops / (pre_b2b_ms * 1e-3) / 1e12 if pre_b2b_ms else None,
        },
        "decode": {
            "value": gbps, "unit": "GB/s", "ms": dec_avg,
            "roofline": {"bound": "hbm", "achieved": dec_kernel_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": dec_kernel_gbps / PEAK_HBM_GBPS if dec_kernel_gbps else None,
                         "kernel_ms": dec_kernel_ms,
                         "call_gbps": gbps, "call_frac": gbps / PEAK_HBM_GBPS if gbps else None,
                         "call_gbps_fenced_events": dbytes / (dec_fenced_ms * 1e6) if dec_fenced_ms == dec_fenced_ms else None,
                         "traffic": traffic_for("decode_bf16_kernel", "slot_decode", source_hash(DECODE_SOURCES)),
                         "kernel": "kev decode_bf16_kernel<128> (the only kernel of the call; kernel "
                                   "events recorded by the library, MALL flushed before each call)",
                         "algorithmic_bytes_per_launch": dbytes},
        },
        "prefill_slots": None if slots_res is None else dict(slots_res, extra_ms_vs_prefill=slots_res["ms"] - pre_avg),
        "prefill_other_configs": other_res or None,
        "chunked_prefill": chunk_res,
        "paged_decode": paged_res or None,
        "decode_low_occupancy": low_res or None,
        "decode_time_vs_bytes": scale_res,
        "cpu_baseline": None,
        "oracle_timing": None,
    }
    if not args.no_cpu_baseline and do_pre:
        log("timing the CPU oracle on bounded samples")
        del q, k, v, out
        result["cpu_baseline"], result["oracle_timing"] = oracle_timing(args.workload, args.oracle_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
