"""Build the HIP library ``libkev.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m segment_isolated_packed_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkev.so")
SOURCES = ["kev_api.hip", "kev_host.cpp", "kev_schedule.hip", "kev_prefill_bf16.hip", "kev_prefill_f32.hip",
           "kev_decode.hip", "kev_store_kv.hip"]
ARCH = os.environ.get("KEV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
            "-Wno-unused-result", "-munsafe-fp-atomics",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def scratch_users(remarks: str) -> list[tuple[str, int]]:
    """Kernels whose compiler resource-usage remarks report private (scratch) memory per lane.

    No kernel of the library may spill: a spill reload inside the prefill loop waits for every
    outstanding vector-memory operation, including the direct-to-LDS loads in flight, and a
    register that a spill copies while an inline-asm load is still filling it would be stored
    before the data lands.
    """
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def _vregs(operand: str) -> set[int]:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", operand)
    return {int(m.group(1))} if m else set()


def early_load_reads(asm: str) -> list[tuple[str, str]]:
    """(kernel, instruction) pairs where a VGPR written by a plain ``global_load_dwordx4`` is read
    before the first ``s_waitcnt`` on vmcnt that follows it.

    The prefill kernels load their query rows with inline asm, so the compiler adds no wait for
    them; the counted wait after the K/V prologue covers them.  A copy of one of those registers
    placed earlier by register allocation would read a load still in flight.
    """
    bad, name, pending, done = [], None, set(), False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, pending, done = m.group(1), set(), False
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")) or name is None or done:
            continue
        ops = [x.strip(",") for x in t.split()[1:]]
        if t.startswith("global_load_dwordx4"):
            pending |= _vregs(ops[0]) if ops else set()
        elif pending and t.startswith("s_waitcnt") and "vmcnt" in t:
            done = True
        elif pending:
            srcs = set()
            for o in (ops if t.startswith("s_") else ops[1:]):
                srcs |= _vregs(o)
            if srcs & pending:
                bad.append((name, t))
    return bad


def _check_prefill_asm() -> None:
    """Compiles the bf16 prefill to device assembly and applies early_load_reads."""
    asm = os.path.join(OBJ, "kev_prefill_bf16.s")
    cmd = [hipcc()] + compile_flags() + ["--cuda-device-only", "-S", os.path.join(CSRC, "kev_prefill_bf16.hip"),
                                         "-o", asm]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for kev_prefill_bf16.hip:\n{p.stderr}")
    with open(asm) as f:
        bad = early_load_reads(f.read())
    if bad:
        raise RuntimeError(f"kev_prefill_bf16.hip: query-load registers read before their wait: {bad[:4]}")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                         os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    bad = scratch_users(p.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {bad}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        check = ex.submit(_check_prefill_asm)
        objs = list(ex.map(_compile, SOURCES))
        check.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
