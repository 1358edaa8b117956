"""Benchmark of the packed-batch gated-delta-net layer forward on one MI355X.

One step = one gdn_varlen_forward call over one batch of the workload: conv +
SiLU + q/k normalisation, the gated delta rule with state read from and written
to the pools, outputs written.  Inputs (x, weights, g, beta, offsets, indices,
state pools) are generated once, copied to HBM before timing, and stay there.

Primary line: the prefill workload (8 sequences, lengths uniform in [256, 4096],
H_k=16, H_v=32, d_k=d_v=128, W=4, bf16 activations, fp32 state), tokens/s.
The same JSON line carries, as nested objects, the decode workload (256
sequences of one token, 1024-block pool), the mixed continuous-batching step
(64 decode tokens beside 4 prefill chunks of 512 tokens), the long prefill (4
sequences of 32768 tokens), the prefill step planned on the device and
replayed from a HIP graph, the standalone varlen conv layer (gdn_varlen_conv on
the prefill rows), the fork copy (gdn_state_copy of 256 blocks), the fp32
chunk kernel on the prefill lengths for the all-fp32 layer and for a bf16 layer
with 64-wide heads, the KDA layer (a decay per key channel) on the prefill and
decode workloads, and the Mamba2 scan, each with the roofline of its dominant kernel and the
per-kernel event timings.  Every gated-delta-net entry also carries the fp64
CPU oracle timed on the host cores on the same workload (`cpu_baseline`), and
the parity of its first call (from fresh pools) against that oracle run: max
relative L2 error over (sequence, value head) slabs and the bit-exact verdicts.

    python bench.py [--gpus 1] [--steps 50] [--warmup 50] [--no-cpu-baseline]

The line also carries `measured_peaks` (the MFMA rate of back-to-back
products from gdn_mfma_peak_probe, bf16 and fp32, and the HBM rate of the
library's 1 GiB streaming copy, gdn_hbm_copy_probe, with torch's copy beside it)
and every roofline its `frac_of_measured` beside `frac`; a roofline whose
kernel has a measured traffic line in profiles/hbm_traffic.txt also carries
`traffic_gbs` (those bytes over the kernel's duration) and its fraction of the
measured copy rate.

Warm-up runs at least `--warmup` steps and at least 60 ms of back-to-back GPU
work, so the clocks have settled (the first few dozen steps after the inputs
are uploaded run up to 10% slower) whatever count is asked for; the line
reports the count run.  The K timed steps run twice: once end to end for
`value` and `ms_per_step`, once more with the library's event pair around every
kernel for `kernels` and `roofline` (those events add a few percent to a step,
so they stay out of the first pass).

On the prefill workload the chunk kernel also runs the conv of the rows (its
workgroups convert rows before their scans), so its duration covers both; the
roofline's `frac` prices only the chunk flops over it, and `step_frac` prices
the same flops over the whole step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_MFMA = 2.5e15  # dense bf16 MFMA, MI355X
PEAK_HBM = 8.0e12        # HBM3E, MI355X
PEAK_F32_MFMA = 157.3e12  # dense fp32 MFMA, MI355X
METRIC = "GDN layer tokens/s (prefill, decode) at 1 GPU; % MFMA / HBM peak"


def chunk_flops(layer, lengths, c: int = 64) -> float:
    """Algorithmic flops of the chunked (WY / UT) form: per chunk of c rows,
    H_k Gram pairs (Q K^T, K K^T: 4 c^2 d_k) and per value head the dense
    products W, U~ (2 c^2 (d_k + d_v)), P U (2 c^2 d_v), W S, Q S, K^T U
    (6 c d_k d_v) and the triangular inverse (2/3 c^3)."""
    Hk, Hv, dk, dv = layer.num_k_heads, layer.num_v_heads, layer.head_k_dim, layer.head_v_dim
    total = 0.0
    for L in lengths:
        if L < 2:
            continue
        full, rem = divmod(L, c)
        for cc in [c] * full + ([rem] if rem else []):
            total += Hk * 4 * cc * cc * dk + Hv * (2 * cc * cc * (dk + dv) + 2 * cc * cc * dv
                                                   + 6 * cc * dk * dv + (2.0 / 3.0) * cc ** 3)
    return total


def token_path_bytes(layer, n_tokens: int) -> float:
    """Algorithmic HBM bytes of the one-token path per launch: per token the
    fp32 state of every value head read and written, the token's x row, the
    conv state read, the output row, g and beta."""
    C = layer.conv_channels
    s = 2 if layer.act_dtype == "bf16" else 4
    state = layer.num_v_heads * layer.head_k_dim * layer.head_v_dim * 4
    per_tok = 2 * state + C * s + (layer.conv_width - 1) * C * s + layer.num_v_heads * layer.head_v_dim * s \
        + 2 * layer.num_v_heads * 4
    return n_tokens * per_tok + C * layer.conv_width * s


# The source files of each profiled kernel: its own file, and for the two chunk
# kernels the header holding the conv tasks they run.
# each kernel's .hip followed by every local header it includes, directly or not
KERNEL_SOURCES = {"chunk_scan": ("gdn_chunk.hip", "gdn_device.h", "gdn_mfma.h", "gdn_convtask.h"),
                  "token_recurrent": ("gdn_recurrent.hip", "gdn_device.h"),
                  "kda_chunk": ("kda_chunk.hip", "gdn_device.h", "gdn_mfma.h", "gdn_convtask.h"),
                  "chunk_generic": ("gdn_chunk_generic.hip", "gdn_device.h", "gdn_mfma.h"),
                  "conv_silu_norm": ("gdn_conv.hip", "gdn_device.h"), "ssd_scan": ("ssd_scan.hip", "gdn_device.h"),
                  "ssd_token": ("ssd_scan.hip", "gdn_device.h"), "state_copy": ("gdn_conv.hip", "gdn_device.h")}


def kernel_source_sha(kernel: str):
    """sha256[:16] of the kernel's source files, concatenated in order (the key
    of its lines in profiles/hbm_traffic.txt), or None for an unknown kernel."""
    import hashlib

    files = KERNEL_SOURCES.get(kernel)
    if files is None:
        return None
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "linear_attention_state_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if a summary for
    this kernel's current source on this workload is committed under profiles/."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha(kernel)
    if sha is None:
        return None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if (len(parts) >= 5 and not line.startswith("#") and parts[0] == kernel and parts[1] == sha
                    and parts[4] == workload):
                return float(parts[2]) + float(parts[3])
    return None


def add_traffic(roof: dict, kernel: str, workload: str, kernel_ms: float) -> None:
    """Records in a roofline the kernel's average duration, its measured HBM
    bytes per launch (profiles/hbm_traffic.txt, null when no line matches the
    current source), and the rate those bytes make over the duration."""
    roof["kernel_ms"] = kernel_ms
    roof["traffic"] = load_traffic(kernel, workload)
    if roof["traffic"] is not None:
        roof["traffic_gbs"] = roof["traffic"] / (kernel_ms * 1e-3) / 1e9


def step_bytes(layer, lengths) -> float:
    """Algorithmic HBM bytes of one whole step of the layer: per token the x row
    read, the output row written, g and beta read; per sequence its recurrent
    state and conv state read and written; the conv taps once."""
    C = layer.conv_channels
    s = 2 if layer.act_dtype == "bf16" else 4
    per_tok = C * s + layer.num_v_heads * layer.head_v_dim * s + 2 * layer.num_v_heads * 4
    per_seq = 2 * (layer.num_v_heads * layer.head_k_dim * layer.head_v_dim * 4 + (layer.conv_width - 1) * C * s)
    return sum(lengths) * per_tok + len(lengths) * per_seq + C * layer.conv_width * s


def warm(step, sync, min_steps: int, min_ms: float = 60.0) -> int:
    """Runs `step` at least min_steps times and until min_ms of wall time (the
    GPU busy all along) has passed, so the clocks have settled whatever warm-up
    count was asked for.  Returns the number of steps run."""
    n = 0
    t0 = time.perf_counter()
    while n < min_steps or (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(5):
            step()
        n += 5
        sync()
    return n


def run(cfg_id: int, steps: int, warmup: int, placements=()):
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.config(cfg_id)
    L = b.layer
    dev = torch.device("cuda", 0)
    d = {k: getattr(b, k).to(dev).contiguous() for k in
         ("x", "conv_weight", "g", "beta", "cu_seqlens", "read_idx", "write_idx", "conv_pool", "ssm_pool")}
    T = b.total_tokens
    out = torch.empty(T, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device=dev)
    ws = torch.empty(max(gdn.gdn_workspace_size(L, T, len(b.lengths)), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    cu_host = b.cu_seqlens.clone()

    def step():
        gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], cu_host,
                               d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out,
                               workspace=ws, stream=stream.cuda_stream)

    # the first call, from the fresh pools: its results are what the oracle leg
    # checks (later steps run on the pools this one wrote)
    gdn.gdn_device_status(clear=True)
    step()
    first = (out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu())
    status = gdn.gdn_device_status(clear=True)
    warm_steps = warm(step, torch.cuda.synchronize, warmup)

    def timed_steps():
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0

    # Two timed passes of `steps` steps: the first end to end (the reported
    # rate), the second with the library's event pair around every kernel (the
    # per-kernel durations and the roofline).  Those events cost a few percent
    # of the step, so they stay out of the first pass.
    ms, wall = timed_steps()
    gdn.gdn_kernel_timing(True)
    ms_events, _ = timed_steps()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    status |= gdn.gdn_device_status(clear=True)
    kernels = {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}
    # the dominant kernel of the layer's own work: the chunk kernel or the token kernel
    dom = max((k for k in kernels if k in ("chunk_scan", "token_recurrent")),
              key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    dom_s = kernels[dom]["avg_ms"] * 1e-3
    flops = chunk_flops(L, b.lengths)
    if dom == "chunk_scan":
        work = flops
        roof = {"bound": "mfma", "achieved": work / dom_s / 1e12, "peak": PEAK_BF16_MFMA / 1e12,
                "unit": "TFLOP/s"}
    else:
        n_short = sum(1 for v in b.lengths if v <= 1)
        work = token_path_bytes(L, n_short)
        roof = {"bound": "hbm", "achieved": work / dom_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the same work over the whole step (every kernel of the path, and the gaps)
    roof["step_frac"] = roof["achieved"] * dom_s / (ms * 1e-3) / roof["peak"]
    if dom == "chunk_scan" and "conv_silu_norm" not in kernels:
        roof["note"] = "chunk_scan also ran the conv of the rows (no separate conv kernel)"
    add_traffic(roof, dom, {1: "prefill", 2: "decode", 3: "mixed", 4: "long"}.get(cfg_id, ""), dom_s * 1e3)
    roof["kernel"] = dom
    res = {
        "batch": b, "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_events, "wall_s": wall, "tokens": T,
        "value": T * steps / (ms * steps * 1e-3), "kernels": kernels, "roofline": roof, "first": first,
        "warmup_steps_run": warm_steps, "device_status": status,
        # the whole step against both roofs: every algorithmic byte and chunk flop over the step time
        "step_hbm_frac": step_bytes(L, b.lengths) / (ms * 1e-3) / PEAK_HBM,
        "step_mfma_frac": flops / (ms * 1e-3) / PEAK_BF16_MFMA,
    }
    # the same steps with the conv placement forced (GDN_CONV_IN_SCAN), for comparison
    if placements:
        old = os.environ.get("GDN_CONV_IN_SCAN")
        res["ms_per_step_forced"] = {}
        try:
            for mode in placements:
                os.environ["GDN_CONV_IN_SCAN"] = mode
                for _ in range(3):
                    step()
                res["ms_per_step_forced"][mode] = timed_steps()[0]
        finally:
            if old is None:
                os.environ.pop("GDN_CONV_IN_SCAN", None)
            else:
                os.environ["GDN_CONV_IN_SCAN"] = old
    return res


def run_graph(steps: int, warmup: int):
    """The prefill step planned on the device (cu_seqlens_host = NULL), captured
    once in a HIP graph and replayed."""
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.config(1)
    L = b.layer
    dev = torch.device("cuda", 0)
    d = {k: getattr(b, k).to(dev).contiguous() for k in
         ("x", "conv_weight", "g", "beta", "cu_seqlens", "read_idx", "write_idx", "conv_pool", "ssm_pool")}
    T = b.total_tokens
    out = torch.empty(T, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device=dev)
    ws = torch.empty(gdn.gdn_workspace_size(L, T, len(b.lengths)), dtype=torch.uint8, device=dev)

    def step():
        gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], None,
                               d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    return {"workload": "the prefill workload planned on the device, one HIP graph replay per step",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms}


def run_conv(steps: int, warmup: int):
    """The standalone varlen conv layer (gdn_varlen_conv, SiLU) on the prefill
    workload's rows: x [T][8192] bf16, W = 4, every sequence from the trash block."""
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.config(1)
    dev = torch.device("cuda", 0)
    x = b.x.to(dev).contiguous()
    w = b.conv_weight.to(dev).contiguous()
    cu = b.cu_seqlens.to(dev)
    ri, wi = b.read_idx.to(dev), b.write_idx.to(dev)
    pool = b.conv_pool.to(dev).contiguous()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    cu_host = b.cu_seqlens.clone()

    def step():
        gdn.gdn_varlen_conv(x, w, cu, cu_host, ri, wi, pool, y, silu=True, stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gdn.gdn_kernel_timing(True)
    for _ in range(steps):
        step()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    T, C, W = b.total_tokens, b.layer.conv_channels, b.layer.conv_width
    n = len(b.lengths)
    # algorithmic bytes: x read, y written, each sequence's state read and written, the taps
    work = 2 * T * C * 2 + 2 * n * (W - 1) * C * 2 + C * W * 2
    conv_ms = kt["conv_silu_norm"][0] / kt["conv_silu_norm"][1]
    roof = {"bound": "hbm", "achieved": work / (conv_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "kernel": "conv_silu_norm"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    add_traffic(roof, "conv_silu_norm", "conv", conv_ms)
    return {"workload": "standalone varlen conv + SiLU: the prefill rows (T=%d, C=%d, W=%d, bf16), "
                        "%d sequences from the trash block" % (T, C, W, n),
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "roofline": roof,
            "kernels": {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}}


def ssd_bytes(layer, lengths) -> float:
    """Algorithmic HBM bytes of one Mamba2 scan launch: per token the head
    inputs x (H*P bf16), B and C (2*G*N bf16), dt (H fp32) and the output y
    (H*P bf16); per sequence its state (H*P*N fp32) read and written."""
    H, P, G, N = layer.num_heads, layer.head_dim, layer.num_groups, layer.state_dim
    T = sum(lengths)
    return T * (H * P * 2 + 2 * G * N * 2 + H * 4 + H * P * 2) + len(lengths) * H * P * N * 4 * 2


def ssd_flops(layer, lengths, chunk: int = 64) -> float:
    """Flops of the dense products the chunked dual form defines: per chunk of
    c rows and head, C B^T on and below the diagonal (c(c+1)N), its product
    with X (c(c+1)P), C S and B^T X (2cNP each)."""
    H, P, N = layer.num_heads, layer.head_dim, layer.state_dim
    total = 0.0
    for L in lengths:
        for c0 in range(0, L, chunk):
            cc = min(chunk, L - c0)
            total += H * (cc * (cc + 1) * (N + P) + 4 * cc * N * P)
    return total


def run_ssd(cfg: int, steps: int, warmup: int):
    """The Mamba2 scan (ssd_varlen_scan) on a Mamba2 workload: 0 prefill, 1 decode."""
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.ssd_config(cfg)
    L = b.layer
    dev = torch.device("cuda", 0)
    xbc = b.xbc.to(dev).contiguous()
    x, B, C = b.views(xbc)
    t = {k: getattr(b, k).to(dev).contiguous() for k in ("dt", "A", "D", "dt_bias", "cu_seqlens", "read_idx",
                                                          "write_idx", "ssm_pool")}
    y = torch.empty(b.total_tokens, L.num_heads, L.head_dim, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    cu_host = b.cu_seqlens.clone()

    def step():
        gdn.ssd_varlen_scan(L, x, B, C, t["dt"], t["A"], t["cu_seqlens"], cu_host, t["read_idx"], t["write_idx"],
                            t["ssm_pool"], y, dt_bias=t["dt_bias"], D=t["D"], stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gdn.gdn_kernel_timing(True)
    for _ in range(steps):
        step()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    dom = max(kt, key=lambda k: kt[k][0])
    k_ms = kt[dom][0] / kt[dom][1]
    byt, fl = ssd_bytes(L, b.lengths), ssd_flops(L, b.lengths)
    # arithmetic intensity below the machine balance (2.5e15 / 8e12 = 312 flop/B): priced against HBM
    roof = {"bound": "hbm", "achieved": byt / (k_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "kernel": dom, "mfma_tflops": fl / (k_ms * 1e-3) / 1e12,
            "flop_per_byte": fl / byt}
    roof["frac"] = roof["achieved"] / roof["peak"]
    add_traffic(roof, dom, "mamba2_prefill" if cfg == 0 else "mamba2_decode", k_ms)
    n = len(b.lengths)
    what = ("prefill: %d sequences, lengths %s, T=%d, from the trash block" % (n, b.lengths, b.total_tokens)
            if cfg == 0 else "decode: %d sequences of 1 token, %d-block pool" % (n, b.ssm_pool.shape[0]))
    return {"workload": "Mamba2 scan, H=%d heads of %d, G=%d, N=%d; %s" % (L.num_heads, L.head_dim, L.num_groups,
                                                                           L.state_dim, what),
            "value": b.total_tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "roofline": roof,
            "kernels": {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}}


def kda_flops(layer, lengths, c: int = 64) -> float:
    """Algorithmic flops of the chunked KDA form: the decay differs per value
    head and key channel, so every value head has its own decayed Gram pair
    (4 c^2 d_k) beside the same dense products as the gated delta rule
    (2 c^2 (d_k + d_v) + 2 c^2 d_v + 6 c d_k d_v + 2/3 c^3)."""
    Hv, dk, dv = layer.num_v_heads, layer.head_k_dim, layer.head_v_dim
    total = 0.0
    for L in lengths:
        if L < 2:
            continue
        full, rem = divmod(L, c)
        for cc in [c] * full + ([rem] if rem else []):
            total += Hv * (4 * cc * cc * dk + 2 * cc * cc * (dk + dv) + 2 * cc * cc * dv + 6 * cc * dk * dv
                           + (2.0 / 3.0) * cc ** 3)
    return total


def kda_chunk_bytes(layer, lengths) -> float:
    """Algorithmic HBM bytes of the KDA chunk kernel: per row of a chunked
    sequence its conv output row (q, k, v), its decays g (fp32, one per value
    head and key channel), b and its output row; per sequence the fp32 state
    read and written."""
    s = 2 if layer.act_dtype == "bf16" else 4
    Hv, dk, dv = layer.num_v_heads, layer.head_k_dim, layer.head_v_dim
    rows = sum(L for L in lengths if L >= 2)
    seqs = sum(1 for L in lengths if L >= 2)
    return rows * (layer.conv_channels * s + Hv * dk * 4 + Hv * 4 + Hv * dv * s) + seqs * 2 * Hv * dk * dv * 4


def run_kda(cfg_id: int, steps: int, warmup: int):
    """The KDA layer (kda_varlen_forward: the gated delta rule with a decay per
    key channel) on the gated-delta-net prefill (cfg_id 1: chunk kernel on
    MFMA) or decode (cfg_id 2: token kernel, HBM bound) workload."""
    import numpy as np
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.config(cfg_id)
    L = b.layer
    dev = torch.device("cuda", 0)
    d = {k: getattr(b, k).to(dev).contiguous() for k in
         ("x", "conv_weight", "beta", "cu_seqlens", "read_idx", "write_idx", "conv_pool", "ssm_pool")}
    rng = np.random.default_rng(7)
    g = torch.tensor(-np.logaddexp(0.0, rng.standard_normal((b.total_tokens, L.num_v_heads, L.head_k_dim))),
                     dtype=torch.float32, device=dev)
    out = torch.empty(b.total_tokens, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device=dev)
    stream = torch.cuda.current_stream(dev)
    cu_host = b.cu_seqlens.clone()
    ws = torch.empty(max(gdn.gdn_workspace_size(L, b.total_tokens, len(b.lengths)), 1), dtype=torch.uint8,
                     device=dev)

    def step():
        gdn.kda_varlen_forward(L, d["x"], d["conv_weight"], g, d["beta"], d["cu_seqlens"], cu_host, d["read_idx"],
                               d["write_idx"], d["conv_pool"], d["ssm_pool"], out, stream=stream.cuda_stream,
                               workspace=ws)

    warmed = warm(step, torch.cuda.synchronize, warmup)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gdn.gdn_kernel_timing(True)
    for _ in range(steps):
        step()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    status = gdn.gdn_device_status(clear=True)
    if cfg_id == 2:
        k_ms = kt["token_recurrent"][0] / kt["token_recurrent"][1]
        # the gated-delta-net decode bytes, with g per key channel instead of per head
        work = token_path_bytes(L, b.total_tokens) + b.total_tokens * L.num_v_heads * (L.head_k_dim - 1) * 4
        roof = {"bound": "hbm", "achieved": work / (k_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "kernel": "token_recurrent"}
        add_traffic(roof, "token_recurrent", "kda_decode", k_ms)
        what = "KDA decode: 256 sequences of 1 token"
    else:
        k_ms = kt["kda_chunk"][0] / kt["kda_chunk"][1]
        roof = {"bound": "mfma", "achieved": kda_flops(L, b.lengths) / (k_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_MFMA / 1e12, "unit": "TFLOP/s", "kernel": "kda_chunk"}
        add_traffic(roof, "kda_chunk", "kda_prefill", k_ms)
        # about 117 flop per algorithmic byte, below the chip's 312: the bytes bound it first
        kb = kda_chunk_bytes(L, b.lengths)
        roof["hbm_bytes"] = kb
        roof["hbm_frac"] = kb / (k_ms * 1e-3) / PEAK_HBM
        what = "KDA prefill: %d sequences, lengths %s, T=%d" % (len(b.lengths), b.lengths, b.total_tokens)
    roof["frac"] = roof["achieved"] / roof["peak"]
    return {"workload": what + "; H_k=16, H_v=32, d=128, W=4, bf16, g per key channel, %d-block pool"
                        % b.ssm_pool.shape[0],
            "value": b.total_tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "roofline": roof,
            "warmup_steps_run": warmed, "device_status": status,
            "kernels": {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}}


def run_generic(act: str, d: int, steps: int, warmup: int):
    """The chunk kernel for other head sizes and the all-fp32 layer
    (chunk_generic, fp32 MFMA) on the prefill lengths: H_k=16, H_v=32, head
    size d, activations in `act`, all sequences from the trash block."""
    import numpy as np
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b1 = workloads.config(1)
    L = workloads.Layer(16, 32, d, d, 4, act)
    b = workloads.make_batch(L, b1.lengths, [0] * len(b1.lengths), b1.write_idx.tolist(), 16, [],
                             np.random.default_rng(1101), "prefill-%s-d%d" % (act, d))
    dev = torch.device("cuda", 0)
    dd = {k: getattr(b, k).to(dev).contiguous() for k in
          ("x", "conv_weight", "g", "beta", "cu_seqlens", "read_idx", "write_idx", "conv_pool", "ssm_pool")}
    out = torch.empty(b.total_tokens, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device=dev)
    ws = torch.empty(max(gdn.gdn_workspace_size(L, b.total_tokens, len(b.lengths)), 1), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    cu_host = b.cu_seqlens.clone()

    def step():
        gdn.gdn_varlen_forward(L, dd["x"], dd["conv_weight"], dd["g"], dd["beta"], dd["cu_seqlens"], cu_host,
                               dd["read_idx"], dd["write_idx"], dd["conv_pool"], dd["ssm_pool"], out,
                               workspace=ws, stream=stream.cuda_stream)

    warmed = warm(step, torch.cuda.synchronize, warmup)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gdn.gdn_kernel_timing(True)
    for _ in range(steps):
        step()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    k_ms = kt["chunk_generic"][0] / kt["chunk_generic"][1]
    # the operands are fp32 whatever the activations: priced against the fp32 MFMA peak
    roof = {"bound": "mfma", "achieved": chunk_flops(L, b.lengths) / (k_ms * 1e-3) / 1e12,
            "peak": PEAK_F32_MFMA / 1e12, "unit": "TFLOP/s", "kernel": "chunk_generic"}
    add_traffic(roof, "chunk_generic", "prefill_fp32" if act == "f32" else "prefill_d64", k_ms)
    roof["frac"] = roof["achieved"] / roof["peak"]
    return {"workload": "prefill lengths %s, T=%d; H_k=16, H_v=32, d_k=d_v=%d, W=4, %s activations, fp32 "
                        "arithmetic" % (b.lengths, b.total_tokens, d, act),
            "value": b.total_tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "roofline": roof,
            "warmup_steps_run": warmed, "device_status": gdn.gdn_device_status(clear=True),
            "kernels": {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}}


def run_state_copy(steps: int, warmup: int):
    """The fork copy (gdn_state_copy) of 256 blocks of the decode workload's
    1024-block pool into 256 other blocks."""
    import torch

    import linear_attention_state_amd as gdn
    import workloads

    b = workloads.config(2)
    dev = torch.device("cuda", 0)
    cp = b.conv_pool.to(dev).contiguous()
    sp = b.ssm_pool.to(dev).contiguous()
    P = sp.shape[0]
    perm = torch.randperm(P - 1, generator=torch.Generator().manual_seed(5)) + 1
    src = perm[:256].to(torch.int32).to(dev)
    dst = perm[256:512].to(torch.int32).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_state_copy(b.layer, cp, sp, src, dst, stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gdn.gdn_kernel_timing(True)
    for _ in range(steps):
        step()
    kt = gdn.gdn_kernel_times()
    gdn.gdn_kernel_timing(False)
    per_block = sp[0].numel() * 4 + cp[0].numel() * cp.element_size()
    work = 2 * 256 * per_block  # each block read once and written once
    k_ms = kt["state_copy"][0] / kt["state_copy"][1]
    roof = {"bound": "hbm", "achieved": work / (k_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "kernel": "state_copy"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    add_traffic(roof, "state_copy", "copy", k_ms)
    return {"workload": "fork copy of 256 blocks (2 MiB recurrent + 48 KiB conv state each) within a 1024-block pool",
            "value": 256 / (ms * 1e-3), "unit": "blocks/s", "ms_per_step": ms, "roofline": roof,
            "kernels": {k: {"avg_ms": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items()}}


def first_call_parity(batch, first, ref) -> dict:
    """The first call's results (from fresh pools) against the oracle's: max
    relative L2 error over (sequence, value head) slabs of outputs and final
    states, and the bit-exact verdicts (conv pool, blocks no sequence writes,
    the trash block)."""
    import numpy as np
    import torch

    out_g, cp_g, sp_g = first
    out_r, fin_r, cp_r, _ = ref
    cu = batch.cu_seqlens.tolist()
    worst_o = worst_s = 0.0
    for s in range(len(cu) - 1):
        wb = int(batch.write_idx[s])
        if wb < 0:
            continue
        og = out_g[cu[s]:cu[s + 1]].double().numpy()
        for m in range(batch.layer.num_v_heads):
            if cu[s + 1] > cu[s]:
                r = out_r[cu[s]:cu[s + 1], m]
                worst_o = max(worst_o, float(np.linalg.norm(og[:, m] - r) / max(np.linalg.norm(r), 1e-300)))
            r = fin_r[s, m]
            e = sp_g[wb, m].double().numpy() - r
            worst_s = max(worst_s, float(np.linalg.norm(e) / max(np.linalg.norm(r), 1e-300)))
    written = set(int(v) for v in batch.write_idx.tolist() if v >= 0)
    idx = torch.tensor([b for b in range(batch.ssm_pool.shape[0]) if b not in written], dtype=torch.long)
    conv_exact = bool(torch.equal(cp_g.view(torch.uint8) if cp_g.numel() else cp_g,
                                  cp_r.view(torch.uint8) if cp_r.numel() else cp_r))
    return {"out_max_rel_l2": worst_o, "state_max_rel_l2": worst_s,
            "tolerance": 1e-2 if batch.layer.act_dtype == "bf16" else 1e-4,
            "conv_pool_bit_exact": conv_exact,
            "unwritten_blocks_bit_exact": bool(torch.equal(sp_g[idx], batch.ssm_pool[idx])),
            "trash_block_zero": not bool(sp_g[0].any())}


def cpu_baseline(batch, first=None):
    """The fp64 oracle on the host cores, on the same workload (all of it: it
    takes from under a second to about 15 s), tokens/s.  With the first GPU
    call's results, the same oracle run also gives that call's parity."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    t0 = time.perf_counter()
    ref = oracle.forward(batch.layer, batch.x, batch.conv_weight, batch.g, batch.beta, batch.cu_seqlens,
                         batch.read_idx, batch.write_idx, batch.conv_pool, batch.ssm_pool, threads=threads)
    dt = time.perf_counter() - t0
    res = {"value": batch.total_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "the whole workload (%d tokens, %d sequences), %.1f s" % (batch.total_tokens,
                                                                             len(batch.lengths), dt)}
    if first is not None:
        res["first_call_parity"] = first_call_parity(batch, first, ref)
    return res


def measured_peaks() -> dict:
    """What this device reaches on plain work, to quote kernel rates against:
    dense MFMA on back-to-back independent products (gdn_mfma_peak_probe, bf16
    and fp32) and HBM on a 1 GiB streaming copy (gdn_hbm_copy_probe: bytes read
    plus bytes written), with torch's own device copy of the same buffer beside
    it."""
    import torch

    import linear_attention_state_amd as gdn

    bf = gdn.gdn_mfma_peak_probe("bf16", 4096)
    f32 = gdn.gdn_mfma_peak_probe("f32", 4096)
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy = gdn.gdn_hbm_copy_probe(src, dst, reps=10)
    for _ in range(3):
        dst.copy_(src)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(10):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    torch_gbs = 2.0 * 4 * n * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": bf, "mfma_f32_tflops": f32, "hbm_copy_gbs": copy, "torch_copy_gbs": torch_gbs}


def annotate(obj, peaks: dict) -> None:
    """Adds to every roofline in the line its fraction of the measured peak of
    the same resource (`frac_of_measured`), and where its measured HBM traffic
    is known, that traffic's rate over the measured streaming-copy rate
    (`traffic_frac_of_measured_copy`)."""
    if isinstance(obj, dict):
        roof = obj.get("roofline")
        if isinstance(roof, dict) and "achieved" in roof:
            if roof["bound"] == "hbm":
                ref = peaks["hbm_copy_gbs"]
            elif roof["peak"] == PEAK_F32_MFMA / 1e12:
                ref = peaks["mfma_f32_tflops"]
            else:
                ref = peaks["mfma_bf16_tflops"]
            roof["frac_of_measured"] = roof["achieved"] / ref
            if roof.get("traffic_gbs") is not None:
                roof["traffic_frac_of_measured_copy"] = roof["traffic_gbs"] / peaks["hbm_copy_gbs"]
        for v in obj.values():
            annotate(v, peaks)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true", help="skip the standalone conv layer and fork copy entries")
    ap.add_argument("--no-long", action="store_true", help="skip the long-prefill entry (4 x 32768 tokens)")
    ap.add_argument("--no-mamba2", action="store_true", help="skip the Mamba2 scan entries")
    ap.add_argument("--only", choices=["prefill", "decode", "mixed", "conv", "copy", "graph", "long", "mamba2_prefill",
                                       "mamba2_decode", "kda_prefill", "kda_decode", "prefill_fp32", "prefill_d64", "peaks"],
                    default=None,
                    help="run one workload alone and print its numbers (profiling runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run only a device-to-device copy of this many bytes (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer's path runs on a single MI355X "
              "(--gpus %d was asked for)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_bytes:
        import torch
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.warmup + args.steps}), flush=True)
        return
    if args.only == "conv":
        print(json.dumps(run_conv(args.steps, args.warmup)), flush=True)
        return
    if args.only == "copy":
        print(json.dumps(run_state_copy(args.steps, args.warmup)), flush=True)
        return
    if args.only in ("prefill_fp32", "prefill_d64"):
        r = run_generic("f32", 128, args.steps, args.warmup) if args.only == "prefill_fp32" else \
            run_generic("bf16", 64, args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return
    if args.only in ("kda_prefill", "kda_decode"):
        print(json.dumps(run_kda(1 if args.only == "kda_prefill" else 2, args.steps, args.warmup)), flush=True)
        return
    if args.only in ("mamba2_prefill", "mamba2_decode"):
        print(json.dumps(run_ssd(0 if args.only == "mamba2_prefill" else 1, args.steps, args.warmup)), flush=True)
        return
    if args.only == "graph":
        print(json.dumps(run_graph(args.steps, args.warmup)), flush=True)
        return
    if args.only == "peaks":
        print(json.dumps(measured_peaks()), flush=True)
        return
    if args.only in ("prefill", "decode", "mixed", "long"):
        r = run({"prefill": 1, "decode": 2, "mixed": 3, "long": 4}[args.only], args.steps, args.warmup)
        print(json.dumps({"workload": args.only, "value": r["value"], "ms_per_step": r["ms_per_step"],
                          "roofline": r["roofline"], "kernels": r["kernels"]}), flush=True)
        return

    def entry(r, what, cpu=True):
        """A nested entry of the line for one GDN workload run by `run`."""
        e = {"workload": what, "value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
             "roofline": r["roofline"], "step_hbm_frac": r["step_hbm_frac"], "step_mfma_frac": r["step_mfma_frac"],
             "kernels": r["kernels"], "warmup_steps_run": r["warmup_steps_run"],
             "device_status": r["device_status"]}
        if cpu and not args.no_cpu_baseline:
            e["cpu_baseline"] = cpu_baseline(r["batch"], r["first"])
        return e

    pre = run(1, args.steps, args.warmup)
    b = pre["batch"]
    line = {
        "metric": METRIC, "value": pre["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pre["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill: %d sequences, lengths %s, T=%d; H_k=16, H_v=32, d_k=d_v=128, W=4, "
                               "C=8192; bf16 activations, fp32 state; all from the trash block"
                               % (len(b.lengths), b.lengths, b.total_tokens),
                   "global_batch": len(b.lengths), "seq_len": max(b.lengths), "tokens": b.total_tokens},
        "roofline": pre["roofline"], "kernels": pre["kernels"], "warmup_steps_run": pre["warmup_steps_run"],
        "step_hbm_frac": pre["step_hbm_frac"], "device_status": pre["device_status"],
    }
    if not args.no_decode:
        dec = run(2, args.steps, args.warmup)
        line["decode"] = entry(dec, "decode: 256 sequences of 1 token, 1024-block pool of 2 MiB fp32 states")
        del dec
        mix = run(3, args.steps, args.warmup)
        line["mixed"] = entry(mix, "mixed continuous-batching step: 64 decode tokens and 4 prefill chunks of 512 "
                                   "tokens (2 continuing, 2 from the trash block) in seeded order, T=2112, "
                                   "512-block pool; same layer")
        del mix
    if not args.no_long:
        lp = run(4, args.steps, args.warmup, placements=("never", "always"))
        lp_note = ("conv streamed by helper workgroups inside chunk_scan"
                   if "conv_silu_norm" not in lp["kernels"] else "separate conv kernel")
        line["long_prefill"] = entry(
            lp, "long prefill: 4 sequences of 32768 tokens, all continuing from their blocks; same layer")
        line["long_prefill"]["placement"] = lp_note
        line["long_prefill"]["ms_per_step_conv_kernel_first"] = lp["ms_per_step_forced"]["never"]
        line["long_prefill"]["ms_per_step_phased"] = lp["ms_per_step_forced"]["always"]
        del lp
    if not args.no_conv:
        line["prefill_graph"] = run_graph(args.steps, args.warmup)
        line["conv"] = run_conv(args.steps, args.warmup)
        line["state_copy"] = run_state_copy(args.steps, args.warmup)
    if not args.no_mamba2:
        line["prefill_fp32"] = run_generic("f32", 128, args.steps, args.warmup)
        line["prefill_d64"] = run_generic("bf16", 64, args.steps, args.warmup)
        line["kda_prefill"] = run_kda(1, args.steps, args.warmup)
        line["kda_decode"] = run_kda(2, args.steps, args.warmup)
        line["mamba2_prefill"] = run_ssd(0, args.steps, args.warmup)
        line["mamba2_decode"] = run_ssd(1, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(b, pre["first"])
    line["measured_peaks"] = measured_peaks()
    annotate(line, line["measured_peaks"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
