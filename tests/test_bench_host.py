"""bench.py's host side, on the CPU: its command-line contract for runs it
cannot measure, and the translation-unit hashes that keep HBM-traffic
figures tied to the kernel sources they were counted on."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_several_gpus_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_bad_step_counts_refused():
    r = _run("--steps", "0")
    assert r.returncode == 2
    assert "--steps" in r.stderr


def test_tu_hashes_cover_every_kernel_source():
    import bench
    hashes = bench.tu_source_hashes()
    csrc = os.path.join(ROOT, "gemv_prefill_decode_amd", "csrc")
    assert set(hashes) == {f for f in os.listdir(csrc) if f.endswith(".hip")}
    assert all(len(h) == 16 for h in hashes.values())
    # a kernel's unit is the .hip file that defines it
    assert bench.kernel_tu("qmm::gemm_lds_kernel<4, 16, 128, 2, false>") == "gemm_lds.hip"
    assert bench.kernel_tu("qmm::gemv_mfma_kernel<3, 2, 2, 2, 1, 8>@131072") == "gemv.hip"
    assert bench.kernel_tu("qmm::moe_kernel<5, 2, 2, false, 0, 0>") == "moe.hip"
