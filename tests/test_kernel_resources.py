"""Compile-time resource check of the chunk kernel (CPU, no GPU needed).

The chunk kernel uses all the registers two waves per SIMD allow.  A spill to
scratch inside its step loop waits on the vector-memory counter, which also
counts the step's output stores, and has cost a fifth of the kernel's time, so
every instantiation must compile without scratch.
"""
import os
import re
import subprocess

import pytest

import linear_attention_state_amd.build as build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_chunk_kernel_has_no_scratch(tmp_path):
    src = os.path.join(ROOT, "linear_attention_state_amd", "csrc", "gdn_chunk.hip")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC, *flags, "--offload-device-only", "-c", "-I", os.path.join(ROOT, "include"), src,
           "-o", str(tmp_path / "chunk.o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    kernel, seen = None, {}
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and kernel and "chunk_scan_kernel" in kernel:
            seen[kernel] = int(m.group(1))
    assert len(seen) == 3, seen  # host-planned, device-planned and streaming instantiations
    assert all(v == 0 for v in seen.values()), seen


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_mamba2_scan_kernel_fits_two_waves_per_simd(tmp_path):
    """The Mamba2 scan kernel holds its state in registers: no scratch, and at
    most 256 VGPRs so that two workgroups share a CU."""
    src = os.path.join(ROOT, "linear_attention_state_amd", "csrc", "ssd_scan.hip")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC, *flags, "--offload-device-only", "-c", "-I", os.path.join(ROOT, "include"), src,
           "-o", str(tmp_path / "ssd.o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    text = res.stderr
    assert "ssd_chunk_kernel" in text
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    occ = [int(v) for v in re.findall(r"Occupancy \[waves/SIMD\]: (\d+)", text)]
    assert scratch and all(v == 0 for v in scratch), scratch
    assert occ and min(occ) >= 2, occ


def _resources(src_name, tmp_path):
    src = os.path.join(ROOT, "linear_attention_state_amd", "csrc", src_name)
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC, *flags, "--offload-device-only", "-c", "-I", os.path.join(ROOT, "include"), src,
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    kernel, seen = None, {}
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and kernel:
            seen[kernel] = int(m.group(1))
    return seen


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_fp32_chunk_kernel_has_no_scratch(tmp_path):
    """Every instantiation (d_k, d_v in 16..128, bf16 and fp32 activations) keeps
    its state tiles in registers without scratch, the fp32-activation 128 x 128
    one included, although it holds the next chunk's q/k rows in registers over
    the chunk: its operand reads are 16-byte LDS loads (the LDS struct is
    16-byte aligned), which leaves room for them."""
    seen = {k: v for k, v in _resources("gdn_chunk_generic.hip", tmp_path).items() if "chunk_generic_kernel" in k}
    assert len(seen) == 32, seen
    assert all(v == 0 for v in seen.values()), seen


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_kda_chunk_kernel_spills_only_outside_its_loops(tmp_path):
    """The KDA chunk kernel spills a few values that live across the whole
    sequence loop (stored before it, reloaded after it: at most 64 bytes per
    lane); a larger scratch size means a spill inside a step."""
    seen = {k: v for k, v in _resources("kda_chunk.hip", tmp_path).items() if "kda_chunk_kernel" in k}
    assert len(seen) == 1, seen
    assert all(v <= 64 for v in seen.values()), seen
