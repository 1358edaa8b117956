"""The source keys of the committed HBM-traffic lines (CPU, no GPU needed).

bench.py uses a measured traffic line only while the kernel's source files hash
to the prefix the line was taken with; a header the kernel includes but the hash
leaves out would let a changed kernel keep a stale line.
"""
import os
import re

import bench

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "linear_attention_state_amd", "csrc")


def _local_includes(name, seen=None):
    seen = set() if seen is None else seen
    with open(os.path.join(CSRC, name)) as f:
        for inc in re.findall(r'^\s*#include\s+"([^"]+)"', f.read(), flags=re.M):
            if inc not in seen and os.path.exists(os.path.join(CSRC, inc)):
                seen.add(inc)
                _local_includes(inc, seen)
    return seen


def test_every_included_header_is_hashed():
    for kernel, files in bench.KERNEL_SOURCES.items():
        assert files[0].endswith(".hip"), (kernel, files)
        assert set(files[1:]) == _local_includes(files[0]), (kernel, files, sorted(_local_includes(files[0])))


def test_traffic_lines_name_known_kernels():
    path = os.path.join(os.path.dirname(CSRC), "..", "profiles", "hbm_traffic.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        kernel, sha = line.split()[:2]
        assert kernel in bench.KERNEL_SOURCES, line
        assert re.fullmatch(r"[0-9a-f]{16}", sha), line
