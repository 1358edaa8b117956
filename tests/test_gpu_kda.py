"""GPU parity of the KDA layer (kda_varlen_forward: the gated delta rule with a
decay per key channel) against the fp64 KDA oracle (oracle/kda_oracle.py),
through the C ABI.

Bar as for the gated-delta-net layer: outputs and final states per (sequence,
value head) within relative L2 error 1e-2 in bf16 and 1e-4 in fp32; conv
states bit-exact; blocks no sequence writes and the trash block untouched.  At
the decode workload's size the oracle runs on sampled value heads.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_state_amd as gdn
import workloads
from gpu_util import TOL, rel_l2, to_device
from oracle import kda_oracle

pytestmark = pytest.mark.gpu


def _g(batch, seed):
    rng = np.random.default_rng(seed)
    L = batch.layer
    raw = rng.standard_normal((batch.total_tokens, L.num_v_heads, L.head_k_dim))
    return torch.tensor(-np.logaddexp(0.0, raw), dtype=torch.float32)


def _run(batch, g):
    d = to_device(batch)
    L = batch.layer
    out = torch.full((batch.total_tokens, L.num_v_heads, L.head_v_dim), 7.0, dtype=L.torch_act, device="cuda")
    gdn.kda_varlen_forward(L, d["x"], d["conv_weight"], g.cuda().contiguous(), d["beta"], d["cu_seqlens"],
                           batch.cu_seqlens, d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out)
    torch.cuda.synchronize()
    return out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu()


def _check(name, batch, g, heads=None):
    L = batch.layer
    print("case %s: lengths %s" % (name, batch.lengths[:12]), flush=True)
    out, cp, sp = _run(batch, g)
    ro, rcp, rsp = kda_oracle.forward(L, batch.x, batch.conv_weight, g, batch.beta, batch.cu_seqlens,
                                      batch.read_idx, batch.write_idx, batch.conv_pool, batch.ssm_pool, heads=heads)
    heads = range(L.num_v_heads) if heads is None else heads
    cu = batch.cu_seqlens.tolist()
    worst_o = worst_s = 0.0
    written = set()
    for s in range(len(cu) - 1):
        wb = int(batch.write_idx[s])
        if wb < 0:
            assert bool((out[cu[s]:cu[s + 1]].float() == 7.0).all()), "padding rows written"
            continue
        written.add(wb)
        for m in heads:
            if cu[s + 1] > cu[s]:
                worst_o = max(worst_o, rel_l2(out[cu[s]:cu[s + 1], m].double().numpy(), ro[cu[s]:cu[s + 1], m]))
            worst_s = max(worst_s, rel_l2(sp[wb, m].double().numpy(), rsp[wb, m]))
    assert torch.equal(cp.view(torch.uint8), rcp.view(torch.uint8)), "conv pool differs"
    for blk in range(batch.ssm_pool.shape[0]):
        if blk not in written:
            assert torch.equal(sp[blk], batch.ssm_pool[blk]), "block %d written" % blk
    tol = TOL[L.act_dtype]
    print("%s: out %.3e state %.3e" % (name, worst_o, worst_s), flush=True)
    assert worst_o <= tol and worst_s <= tol, (worst_o, worst_s)


def test_bf16_ragged_with_decode_tokens():
    b = workloads.random_batch(workloads.BIG, [1, 40, 1, 3, 130, 1], seed=61, fresh=[0, 1, 0, 0, 0, 1])
    _check("bf16-ragged", b, _g(b, 62), heads=[0, 1, 13, 30, 31])


def test_fp32_small_layer_all_heads():
    layer = workloads.Layer(2, 4, 64, 32, 4, "f32")
    b = workloads.random_batch(layer, [17, 1, 0, 66], seed=63)
    _check("fp32", b, _g(b, 64))


def test_padding_sequence_and_width_two():
    layer = workloads.Layer(4, 8, 128, 128, 2, "bf16")
    b = workloads.random_batch(layer, [9, 20, 1], seed=65)
    b.write_idx[1] = -1
    _check("padding-W2", b, _g(b, 66))


def test_uniform_decay_matches_the_gated_delta_rule_kernels():
    """A decay equal on every channel gives the gated-delta-net layer: against
    gdn_varlen_forward (its token path for the decode tokens, the chunk kernel
    for the rest) within the bar."""
    from gpu_util import run_gpu

    b = workloads.random_batch(workloads.BIG, [1, 1, 70, 1], seed=67)
    out, cp, sp = _run(b, kda_oracle.with_scalar_decay(b.g, b.layer.head_k_dim))
    go, gcp, gsp = run_gpu(b)
    for s in range(4):
        rows = slice(int(b.cu_seqlens[s]), int(b.cu_seqlens[s + 1]))
        assert rel_l2(out[rows].double().numpy(), go[rows].double().numpy()) <= 1e-2
        wb = int(b.write_idx[s])
        assert rel_l2(sp[wb].double().numpy(), gsp[wb].double().numpy()) <= 1e-2
    assert torch.equal(cp.view(torch.uint8), gcp.view(torch.uint8))


def test_decode_workload_sampled_heads():
    b = workloads.config(2)
    _check("decode", b, _g(b, 68), heads=[0, 17, 31])


# ---- the chunked path (sequences of two or more tokens, bf16, d = 128)

def test_chunked_edge_lengths_around_64():
    """Lengths around the chunk size (2, 3, 63, 64, 65, 127-129, 200) beside
    decode tokens and an empty sequence, half of them from the trash block."""
    lengths = [2, 3, 63, 64, 65, 1, 127, 128, 0, 129, 200]
    b = workloads.random_batch(workloads.BIG, lengths, seed=71, fresh=[i % 2 for i in range(len(lengths))])
    _check("chunk-edges", b, _g(b, 72), heads=[0, 1, 16, 31])


def test_chunked_prefill_workload_sampled_heads():
    """The gated-delta-net prefill workload (8 sequences of 256-4096 tokens,
    about 20k tokens) with a decay per key channel; the oracle runs two value
    heads of every sequence token by token."""
    b = workloads.config(1)
    _check("kda-prefill", b, _g(b, 73), heads=[0, 31])


def test_strong_decay_blocks_take_the_exact_path():
    """A decay of -8 per row on some channels over whole 16-row blocks (their
    own decay e^-128 would overflow the fp32 factor of the block products):
    those diagonal blocks are computed from the channel sums in fp32."""
    layer = workloads.Layer(2, 4, 128, 128, 4, "bf16")
    b = workloads.random_batch(layer, [100, 70, 1], seed=74, fresh=[1, 0, 0])
    g = _g(b, 75)
    g[10:40, :, :32] = -8.0    # rows 10-39 of the first sequence, channels 0-31
    g[120:150, 1, 64:] = -8.0  # rows 20-49 of the second sequence, head 1, channels 64-127
    _check("strong-decay", b, g)


def test_chunked_split_over_two_calls():
    """A sequence split at rows 70 and 130 over three calls, each continuing
    from the block the previous one wrote, equals one call (and the oracle)."""
    layer = workloads.Layer(2, 4, 128, 128, 4, "bf16")
    b = workloads.random_batch(layer, [200], seed=76)
    g = _g(b, 77)
    one, cp1, sp1 = _run(b, g)
    cut = [0, 70, 130, 200]
    outs = []
    cp, sp = b.conv_pool, b.ssm_pool
    for i in range(3):
        r0, r1 = cut[i], cut[i + 1]
        part = workloads.Batch("part", layer, b.x[r0:r1].contiguous(), b.conv_weight, b.g[r0:r1].contiguous(),
                               b.beta[r0:r1].contiguous(), torch.tensor([0, r1 - r0], dtype=torch.int32),
                               (b.read_idx if i == 0 else b.write_idx).clone(), b.write_idx.clone(), cp, sp)
        o, cp, sp = _run(part, g[r0:r1].contiguous())
        outs.append(o)
    wb = int(b.write_idx[0])
    assert torch.equal(cp.view(torch.uint8), cp1.view(torch.uint8)), "conv states differ"
    assert rel_l2(torch.cat(outs).double().numpy(), one.double().numpy()) <= 1e-2
    assert rel_l2(sp[wb].double().numpy(), sp1[wb].double().numpy()) <= 1e-2
    _check("kda-one-pass", b, g)


def _run_placed(batch, g, mode):
    """_run with the conv placement forced (GDN_CONV_IN_SCAN) and the kernels
    that ran recorded."""
    old = os.environ.get("GDN_CONV_IN_SCAN")
    os.environ["GDN_CONV_IN_SCAN"] = mode
    try:
        gdn.gdn_kernel_timing(True)
        res = _run(batch, g)
        kernels = gdn.gdn_kernel_times()
    finally:
        gdn.gdn_kernel_timing(False)
        if old is None:
            del os.environ["GDN_CONV_IN_SCAN"]
        else:
            os.environ["GDN_CONV_IN_SCAN"] = old
    return res, kernels


def test_conv_inside_the_chunk_kernel_matches_the_conv_kernel_bitwise():
    """The conv of the chunked rows run by the KDA chunk kernel's own
    workgroups (its scans waiting chunk by chunk) against the conv kernel
    before it: outputs, conv states and recurrent states bit for bit the same,
    on lengths around the chunk size beside a decode token and an empty
    sequence (7 chunked sequences: every workgroup resident), and the oracle
    bar met."""
    lengths = [2, 65, 1, 129, 0, 200, 63, 3, 64]
    b = workloads.random_batch(workloads.BIG, lengths, seed=78, fresh=[i % 2 for i in range(len(lengths))])
    g = _g(b, 79)
    print("case kda-fused: lengths %s" % lengths, flush=True)
    (out_f, cp_f, sp_f), k_f = _run_placed(b, g, "always")
    (out_s, cp_s, sp_s), k_s = _run_placed(b, g, "never")
    assert "conv_silu_norm" not in k_f and "kda_chunk" in k_f, k_f
    assert "conv_silu_norm" in k_s and "kda_chunk" in k_s, k_s
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(cp_f.view(torch.int16), cp_s.view(torch.int16))
    assert torch.equal(sp_f, sp_s)
    _check("kda-fused", b, g, heads=[0, 1, 16, 31])


def test_reused_workspace_reads_no_stale_rows():
    """Two KDA batches of the same lengths and different inputs back to back on
    one workspace, the conv inside the chunk kernel: the second call equals the
    same call on a fresh workspace bit for bit (no scan reads the first call's
    rows)."""
    lengths = [300, 70, 129, 64]
    first = workloads.random_batch(workloads.BIG, lengths, seed=80)
    second = workloads.random_batch(workloads.BIG, lengths, seed=81)
    g1, g2 = _g(first, 82), _g(second, 83)
    print("case kda-reuse: lengths %s" % lengths, flush=True)
    L = workloads.BIG
    nbytes = gdn.gdn_workspace_size(L, second.total_tokens, len(lengths))

    def call(batch, g, ws):
        d = to_device(batch)
        out = torch.empty(batch.total_tokens, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device="cuda")
        gdn.kda_varlen_forward(L, d["x"], d["conv_weight"], g.cuda().contiguous(), d["beta"], d["cu_seqlens"],
                               batch.cu_seqlens, d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out,
                               workspace=ws)
        return out, d["conv_pool"], d["ssm_pool"]

    old = os.environ.get("GDN_CONV_IN_SCAN")
    os.environ["GDN_CONV_IN_SCAN"] = "always"
    try:
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        gdn.gdn_kernel_timing(True)
        try:
            call(first, g1, ws)
            reused = call(second, g2, ws)
            torch.cuda.synchronize()
            kernels = gdn.gdn_kernel_times()
        finally:
            gdn.gdn_kernel_timing(False)
        ref = call(second, g2, torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["GDN_CONV_IN_SCAN"]
        else:
            os.environ["GDN_CONV_IN_SCAN"] = old
    assert "conv_silu_norm" not in kernels and kernels["kda_chunk"][1] == 2, kernels
    for a, b in zip(reused, ref):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_conv_inside_for_a_single_sequence():
    """One chunked KDA sequence (its workgroups convert every row themselves)
    beside a decode token: bitwise equal to the conv kernel placement."""
    lengths = [700, 1]
    b = workloads.random_batch(workloads.BIG, lengths, seed=84)
    g = _g(b, 85)
    print("case kda-fused-single: lengths %s" % lengths, flush=True)
    (out_f, cp_f, sp_f), k_f = _run_placed(b, g, "always")
    (out_s, cp_s, sp_s), k_s = _run_placed(b, g, "never")
    assert "conv_silu_norm" not in k_f and "kda_chunk" in k_f, k_f
    assert "conv_silu_norm" in k_s, k_s
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(cp_f.view(torch.int16), cp_s.view(torch.int16))
    assert torch.equal(sp_f, sp_s)


def test_more_sequences_than_the_launch_order_holds():
    """1,030 chunked sequences beside short ones, more than the 1,024 the
    longest-first launch order holds: the conv kernel then runs first and the
    KDA chunk kernel covers every sequence in index order."""
    layer = workloads.Layer(2, 4, 128, 128, 4, "bf16")
    lengths = ([2, 3, 66, 5, 2, 9, 4, 2, 7, 3] * 103)[:1030] + [1, 0, 1, 1]
    b = workloads.random_batch(layer, lengths, seed=18)
    _check("many", b, _g(b, 19))
