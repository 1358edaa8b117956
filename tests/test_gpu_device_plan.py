"""GPU: launches planned on the device (cu_seqlens_host = NULL).

The device plan must give bitwise the same results as the host plan, and a
HIP graph captured with one batch must replay correctly for other batches of
the same sequence count and token count (other lengths, indices and data),
each replay checked against an eager run and the fp64 oracle, with eager work
between the replays.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_state_amd as gdn
import workloads
from gpu_util import compare, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _run(batch, host_plan: bool):
    d = to_device(batch)
    L = batch.layer
    out = torch.full((batch.total_tokens, L.num_v_heads, L.head_v_dim), 3.0, dtype=L.torch_act, device="cuda")
    gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"],
                           batch.cu_seqlens if host_plan else None, d["read_idx"], d["write_idx"],
                           d["conv_pool"], d["ssm_pool"], out)
    torch.cuda.synchronize()
    return out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b):
    for u, v in zip(a, b):
        assert torch.equal(_bits(u), _bits(v))


CASES = {
    "prefill": lambda: workloads.config(1),
    "decode": lambda: workloads.config(2),
    "mixed": lambda: workloads.config(3),
    "ragged": lambda: workloads.random_batch(workloads.BIG, [2, 3, 17, 63, 1, 130, 0, 16], seed=91),
    "fp32": lambda: workloads.random_batch(workloads.Layer(2, 4, 64, 32, 4, "f32"), [30, 1, 7], seed=92),
    "W2": lambda: workloads.random_batch(workloads.Layer(16, 32, 128, 128, 2, "bf16"), [5, 90, 1], seed=93),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_device_plan_equals_host_plan_bitwise(name):
    b = CASES[name]()
    print("case %s: %d sequences, T=%d" % (name, len(b.lengths), b.total_tokens), flush=True)
    _same(_run(b, True), _run(b, False))


@pytest.mark.parametrize("mode", ["always", "never"])
def test_device_plan_with_forced_placement(mode):
    b = workloads.random_batch(workloads.BIG, [40, 200, 3, 77], seed=94)
    old = os.environ.get("GDN_CONV_IN_SCAN")
    os.environ["GDN_CONV_IN_SCAN"] = mode
    try:
        dev = _run(b, False)
        host = _run(b, True)
    finally:
        if old is None:
            del os.environ["GDN_CONV_IN_SCAN"]
        else:
            os.environ["GDN_CONV_IN_SCAN"] = old
    _same(dev, host)
    errs = compare(b, dev, run_oracle(b))
    print("forced %s: out %.3e state %.3e" % (mode, errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)


def _same_shape_batch(lengths, seed, P=12):
    rng = np.random.default_rng(seed)
    n = len(lengths)
    blocks = rng.choice(np.arange(1, P), size=n, replace=False).tolist()
    fresh = rng.random(n) < 0.3
    reads = [0 if f else b_ for f, b_ in zip(fresh, blocks)]
    priors = [b_ for f, b_ in zip(fresh, blocks) if not f]
    return workloads.make_batch(workloads.BIG, lengths, reads, blocks, P, priors, rng, "graph")


def test_graph_replays_for_other_offsets_and_indices():
    """Captured with one batch of 6 sequences and 600 tokens; replayed for three
    others of the same counts (decode tokens, long and short sequences, other
    blocks), each replay against an eager run (bitwise) and the oracle."""
    batches = [_same_shape_batch(l, seed=95 + i) for i, l in enumerate(
        [[100, 100, 100, 100, 100, 100], [1, 300, 2, 250, 1, 46], [595, 1, 1, 1, 1, 1], [64, 64, 200, 136, 72, 64]])]
    a = batches[0]
    d = to_device(a)
    L = a.layer
    T = a.total_tokens
    out = torch.zeros(T, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device="cuda")
    ws = torch.empty(gdn.gdn_workspace_size(L, T, len(a.lengths)), dtype=torch.uint8, device="cuda")

    def fwd():
        gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], None,
                               d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    torch.cuda.synchronize()
    for rep, b in enumerate(batches[1:] + batches[:1] + batches[1:2]):
        src = to_device(b)
        for k in d:
            d[k].copy_(src[k])
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = (out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu())
        _same(got, _run(b, False))
        errs = compare(b, got, run_oracle(b))
        print("replay %d lengths %s: out %.3e state %.3e (%.1f)" % (rep, b.lengths, errs["out_rel_l2"],
                                                                    errs["state_rel_l2"], float(junk)), flush=True)
