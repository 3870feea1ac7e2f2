"""The build's checks on the compiled HIP code: scratch use reported by the compiler's
resource-usage remarks, and reads of an inline-asm load's registers before the wait that
covers the load.  Each check is exercised on planted text here, and on the real prefill
assembly when hipcc is available."""
import os
import shutil
import subprocess

import pytest

from segment_isolated_packed_amd import build as B


def test_scratch_users_reports_only_kernels_with_scratch():
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: _Zk1 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark: Function Name: _Zk2 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert B.scratch_users(remarks) == [("_Zk2", 36)]


def test_early_load_reads_planted():
    load = "_Zk:\n\tglobal_load_dwordx4 v[4:7], v[0:1], off\n"
    # a copy of a loaded register before the wait is reported, with its kernel
    assert B.early_load_reads(load + "\tv_mov_b32_e32 v9, v5\n\ts_waitcnt vmcnt(0)\n") == \
        [("_Zk", "v_mov_b32_e32 v9, v5")]
    # the same copy after the wait, writes to the registers, and reads of other registers are fine
    assert B.early_load_reads(load + "\ts_waitcnt vmcnt(2)\n\tv_mov_b32_e32 v9, v5\n") == []
    assert B.early_load_reads(load + "\tv_mov_b32_e32 v9, v3\n\ts_waitcnt vmcnt(0)\n") == []
    # an lgkmcnt-only wait does not cover the load
    assert B.early_load_reads(load + "\ts_waitcnt lgkmcnt(0)\n\tv_add_u32_e32 v1, v7, v2\n") == \
        [("_Zk", "v_add_u32_e32 v1, v7, v2")]
    # the direct-to-LDS loads are not query loads and the scan restarts at each kernel
    assert B.early_load_reads("_Zk:\n\tglobal_load_lds_dwordx4 v[4:5], off\n\tv_mov_b32_e32 v9, v4\n") == []
    assert B.early_load_reads(load + "_Zk2:\n\tv_mov_b32_e32 v9, v5\n") == []


@pytest.mark.skipif(not os.path.exists(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"))
                    and shutil.which("hipcc") is None, reason="needs hipcc")
def test_prefill_assembly_reads_no_query_register_before_its_wait(tmp_path):
    asm = str(tmp_path / "prefill.s")
    cmd = [B.hipcc()] + B.compile_flags() + ["--cuda-device-only", "-S",
                                             os.path.join(B.CSRC, "kev_prefill_bf16.hip"), "-o", asm]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(asm).read()
    assert text.count("global_load_dwordx4 ") >= 4 * 2 + 12 * 2   # query loads of all four kernels
    assert B.early_load_reads(text) == []
