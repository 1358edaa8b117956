"""GPU: the conv of the chunked rows run inside the chunk kernel ("fused")
against the conv kernel, forced both ways with GDN_CONV_IN_SCAN.

Both placements must give the same outputs, conv states and recurrent states
bit for bit (same arithmetic in the same order), and the fused one must also
meet the oracle bar.  The kernel timing of each call shows which placement ran.
"""
import os

import pytest
import torch

import linear_attention_state_amd as gdn
import workloads
from gpu_util import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _run(batch, mode):
    old = os.environ.get("GDN_CONV_IN_SCAN")
    os.environ["GDN_CONV_IN_SCAN"] = mode
    try:
        gdn.gdn_kernel_timing(True)
        res = run_gpu(batch)
        kernels = gdn.gdn_kernel_times()
    finally:
        gdn.gdn_kernel_timing(False)
        if old is None:
            del os.environ["GDN_CONV_IN_SCAN"]
        else:
            os.environ["GDN_CONV_IN_SCAN"] = old
    return res, kernels


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _both_ways(batch, name):
    print("case %s: lengths %s" % (name, batch.lengths), flush=True)
    (out_f, cp_f, sp_f), k_f = _run(batch, "always")
    (out_s, cp_s, sp_s), k_s = _run(batch, "never")
    assert "conv_silu_norm" not in k_f and "chunk_scan" in k_f, k_f
    assert "conv_silu_norm" in k_s, k_s
    assert torch.equal(_bits(out_f), _bits(out_s))
    assert torch.equal(_bits(cp_f), _bits(cp_s))
    assert torch.equal(sp_f, sp_s)
    errs = compare(batch, (out_f, cp_f, sp_f), run_oracle(batch))
    print("%s: out %.3e state %.3e" % (name, errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)
    return k_f


def test_ragged_lengths_with_priors():
    """Lengths around the 16-row task and 64-row chunk edges, and 2 and 3
    (shorter than the conv window), each continuing in place from its own block."""
    b = workloads.random_batch(workloads.BIG, [2, 3, 17, 63, 65, 130, 200, 16], seed=41)
    _both_ways(b, "ragged")


def test_fresh_and_continuing_sequences():
    b = workloads.random_batch(workloads.BIG, [90, 5, 300, 48], seed=42, fresh=[1, 0, 1, 0])
    _both_ways(b, "fresh")


def test_mixed_with_decode_tokens():
    """One-token sequences beside chunked ones: the conv-state commit kernel then
    runs for the one-token sequences only."""
    b = workloads.random_batch(workloads.BIG, [1, 70, 1, 33, 1], seed=43)
    k = _both_ways(b, "mixed")
    assert "token_recurrent" in k and "conv_state_commit" in k, k


def test_pure_prefill_skips_the_commit_kernel():
    b = workloads.random_batch(workloads.BIG, [40, 129], seed=44)
    k = _both_ways(b, "prefill")
    assert "conv_state_commit" not in k, k


def test_padding_sequence():
    b = workloads.random_batch(workloads.BIG, [64, 70, 9], seed=45)
    b.write_idx[1] = -2
    _both_ways(b, "padding")


@pytest.mark.parametrize("W", [2, 3])
def test_conv_widths(W):
    layer = workloads.Layer(16, 32, 128, 128, W, "bf16")
    b = workloads.random_batch(layer, [2, 31, 100], seed=46 + W)
    _both_ways(b, "W%d" % W)


def test_narrow_layer_partial_channel_slice():
    """C = 1024 < 4096 channels per task: most threads of a task have no channel."""
    layer = workloads.Layer(2, 4, 128, 128, 4, "bf16")
    b = workloads.random_batch(layer, [77, 3, 140], seed=49)
    _both_ways(b, "narrow")


def _stream_vs_separate(batch, name):
    print("case stream-%s: lengths %s" % (name, batch.lengths), flush=True)
    (out_f, cp_f, sp_f), k_f = _run(batch, "stream")
    (out_s, cp_s, sp_s), k_s = _run(batch, "never")
    assert "conv_silu_norm" not in k_f and "chunk_scan" in k_f, k_f
    assert "conv_silu_norm" in k_s, k_s
    assert torch.equal(_bits(out_f), _bits(out_s))
    assert torch.equal(_bits(cp_f), _bits(cp_s))
    assert torch.equal(sp_f, sp_s)
    errs = compare(batch, (out_f, cp_f, sp_f), run_oracle(batch))
    print("stream-%s: out %.3e state %.3e" % (name, errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)


STREAM_CASES = {
    "ragged": (workloads.BIG, [2, 3, 17, 63, 65, 130, 200], None),
    "fresh": (workloads.BIG, [700, 5, 300], [1, 0, 1]),
    "mixed": (workloads.BIG, [1, 300, 1, 70, 1], None),
    "single": (workloads.BIG, [1000], None),
    "W2": (workloads.Layer(16, 32, 128, 128, 2, "bf16"), [2, 31, 500], None),
    "W3": (workloads.Layer(16, 32, 128, 128, 3, "bf16"), [150, 31, 2], None),
    "narrow": (workloads.Layer(2, 4, 128, 128, 4, "bf16"), [77, 3, 640], None),
}


@pytest.mark.parametrize("name", sorted(STREAM_CASES))
def test_streamed_conv_equals_separate(name):
    """Streaming (helper workgroups convert rows while the scans wait chunk by
    chunk) against the conv kernel: bitwise, and within the oracle bar."""
    layer, lengths, fresh = STREAM_CASES[name]
    b = workloads.random_batch(layer, lengths, seed=51 + len(name), fresh=fresh)
    _stream_vs_separate(b, name)


def test_streamed_padding_sequence():
    b = workloads.random_batch(workloads.BIG, [64, 270, 9], seed=58)
    b.write_idx[1] = -2
    _stream_vs_separate(b, "padding")


def _call(batch, ws, mode):
    """One gdn_varlen_forward of a fresh device copy of `batch` on the given
    workspace, with the conv placement forced; no synchronisation."""
    from gpu_util import to_device
    d = to_device(batch)
    L = batch.layer
    out = torch.empty(batch.total_tokens, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device="cuda")
    old = os.environ.get("GDN_CONV_IN_SCAN")
    os.environ["GDN_CONV_IN_SCAN"] = mode
    try:
        gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], batch.cu_seqlens,
                               d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out, workspace=ws)
    finally:
        if old is None:
            del os.environ["GDN_CONV_IN_SCAN"]
        else:
            os.environ["GDN_CONV_IN_SCAN"] = old
    return out, d["conv_pool"], d["ssm_pool"]


@pytest.mark.parametrize("mode", ["always", "stream"])
def test_reused_workspace_reads_no_stale_rows(mode):
    """Two batches of the same lengths and different inputs run back to back on
    one workspace: the second call's scans must read the rows its own conv
    tasks wrote, never the first call's rows at the same addresses (the waits
    end with an acquire fence), so it equals the same call on a fresh
    workspace bit for bit."""
    lengths = [300, 70, 129, 64]
    first = workloads.random_batch(workloads.BIG, lengths, seed=60)
    second = workloads.random_batch(workloads.BIG, lengths, seed=61)
    print("case reuse-%s: lengths %s" % (mode, lengths), flush=True)
    nbytes = gdn.gdn_workspace_size(workloads.BIG, second.total_tokens, len(lengths))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fresh = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gdn.gdn_kernel_timing(True)
    try:
        _call(first, ws, mode)
        reused = _call(second, ws, mode)
        torch.cuda.synchronize()
        kernels = gdn.gdn_kernel_times()
    finally:
        gdn.gdn_kernel_timing(False)
    assert "conv_silu_norm" not in kernels and kernels["chunk_scan"][1] == 2, kernels
    ref = _call(second, fresh, mode)
    torch.cuda.synchronize()
    for a, b in zip(reused, ref):
        assert torch.equal(_bits(a), _bits(b))


def test_single_sequence_converts_all_its_own_rows():
    """One chunked sequence beside a decode token: its workgroups are the only
    claimers (the first rank is also the last), convert every task, and their
    scans then wait chunk by chunk."""
    b = workloads.random_batch(workloads.BIG, [700, 1], seed=62)
    _both_ways(b, "single")


def _run_claim(batch, rule):
    """The phased conv with its claim rule forced ("own", "budget") or chosen
    by the host (None)."""
    old = {k: os.environ.get(k) for k in ("GDN_CONV_IN_SCAN", "GDN_CONV_CLAIM")}
    os.environ["GDN_CONV_IN_SCAN"] = "always"
    if rule is None:
        os.environ.pop("GDN_CONV_CLAIM", None)
    else:
        os.environ["GDN_CONV_CLAIM"] = rule
    try:
        gdn.gdn_kernel_timing(True)
        res = run_gpu(batch)
        kernels = gdn.gdn_kernel_times()
    finally:
        gdn.gdn_kernel_timing(False)
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert "conv_silu_norm" not in kernels and "chunk_scan" in kernels, kernels
    return res


@pytest.mark.parametrize("name,lengths,fresh", [
    ("skewed", [2048, 64, 2048, 64, 2048, 64, 2048, 64], None),
    # (the two-token sequence continues from its block: started fresh, its
    # first output row is b (q.k) v, whose slab norm can nearly vanish, so a
    # relative error over that slab says nothing about the arithmetic)
    ("spread", [900, 700, 300, 130, 65, 3, 2], [1, 0, 0, 1, 0, 0, 0]),
    ("decode-beside", [1, 640, 1, 70, 1, 2], None),
])
def test_claim_rules_give_the_same_bits(name, lengths, fresh):
    """Chunk-major claiming by time budget alone (the shortest sequence's
    workgroups claim whatever is left) and sequence-major claiming of one's
    own tasks first convert the same rows with the same arithmetic: outputs
    and both states equal bit for bit, whichever rule the host picks, and
    within the oracle bar."""
    b = workloads.random_batch(workloads.BIG, lengths, seed=63, fresh=fresh)
    print("case claim-%s: lengths %s" % (name, lengths), flush=True)
    own = _run_claim(b, "own")
    for rule in ("budget", None):
        res = _run_claim(b, rule)
        for a, c in zip(res, own):
            assert torch.equal(_bits(a), _bits(c)), rule
    errs = compare(b, own, run_oracle(b))
    print("claim-%s: out %.3e state %.3e" % (name, errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)
