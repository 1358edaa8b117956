"""GPU parity: the HIP library against the fp64 oracle, through the C ABI.

Bar: conv states (and every block no sequence writes) bit-exact; outputs and
final recurrent states within max relative L2 error 1e-2 per (sequence, value
head) slab with bf16 activations and fp32 state, 1e-4 with all-fp32.
"""
import pytest
import torch

import workloads
from gpu_util import TOL, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print("%s: out %.3e state %.3e" % (name, errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)


def test_config0_tiny_fp32():
    b = workloads.config(0)
    _report("cfg0", compare(b, run_gpu(b), run_oracle(b)))


def test_config0_one_based_sequence_reading():
    """The other reading of which sequence starts from the trash block."""
    b = workloads.config(0)
    b.read_idx = torch.tensor([3, 0, 6], dtype=torch.int32)
    b.write_idx = torch.tensor([3, 1, 6], dtype=torch.int32)
    _report("cfg0-1based", compare(b, run_gpu(b), run_oracle(b)))


def test_config1_prefill():
    b = workloads.config(1)
    _report("cfg1", compare(b, run_gpu(b), run_oracle(b)))


def test_config2_decode():
    b = workloads.config(2)
    _report("cfg2", compare(b, run_gpu(b), run_oracle(b)))


def test_config3_mixed():
    b = workloads.config(3)
    _report("cfg3", compare(b, run_gpu(b), run_oracle(b)))


def test_config4_long_prefill():
    """Full 4 x 32768 run on the GPU against the oracle on every (sequence,
    value head) slab of outputs and final states (the oracle runs the 128
    chains token by token, about 10 s on 16 host cores)."""
    b = workloads.config(4)
    gpu = run_gpu(b)
    _report("cfg4", compare(b, gpu, run_oracle(b)))


EDGE = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 200]


def test_edge_lengths_chunked_path():
    """Lengths around the chunk size, 0 and 1 in one packed batch, half of them
    without a past."""
    b = workloads.random_batch(workloads.BIG, EDGE, seed=21, fresh=[i % 2 for i in range(len(EDGE))])
    _report("edge", compare(b, run_gpu(b), run_oracle(b)))


@pytest.mark.parametrize("dims", [(16, 16, 2, 2), (32, 64, 2, 4), (64, 64, 4, 8), (128, 64, 2, 2)])
def test_other_head_shapes_bf16(dims):
    dk, dv, hk, hv = dims
    layer = workloads.Layer(hk, hv, dk, dv, 4, "bf16")
    b = workloads.random_batch(layer, [5, 1, 70, 0, 2], seed=22)
    _report("dims%s" % (dims,), compare(b, run_gpu(b), run_oracle(b)))


@pytest.mark.parametrize("W", [1, 2, 3])
def test_conv_widths(W):
    layer = workloads.Layer(2, 4, 128, 128, W, "bf16")
    b = workloads.random_batch(layer, [1, 2, 3, 66], seed=23 + W)
    _report("W%d" % W, compare(b, run_gpu(b), run_oracle(b)))


def test_fp32_longer_sequences():
    layer = workloads.Layer(2, 4, 64, 32, 4, "f32")
    b = workloads.random_batch(layer, [130, 1, 7], seed=26)
    _report("f32", compare(b, run_gpu(b), run_oracle(b)))


# ------------------------------------------------------------- invariants

def test_packed_equals_single_sequences_bitwise():
    """No reduction crosses a sequence: the packed call equals one call per
    sequence bit for bit (outputs and blocks)."""
    b = workloads.random_batch(workloads.BIG, [70, 1, 130, 3], seed=31)
    out, cp, sp = run_gpu(b)
    cu = b.cu_seqlens.tolist()
    for s in range(4):
        one = workloads.Batch("one", b.layer, b.x[cu[s]:cu[s + 1]].contiguous(), b.conv_weight,
                              b.g[cu[s]:cu[s + 1]].contiguous(), b.beta[cu[s]:cu[s + 1]].contiguous(),
                              torch.tensor([0, cu[s + 1] - cu[s]], dtype=torch.int32),
                              b.read_idx[s:s + 1].clone(), b.write_idx[s:s + 1].clone(),
                              b.conv_pool, b.ssm_pool)
        o1, cp1, sp1 = run_gpu(one)
        wb = int(b.write_idx[s])
        assert torch.equal(out[cu[s]:cu[s + 1]].view(torch.int16), o1.view(torch.int16))
        assert torch.equal(cp[wb].view(torch.int16), cp1[wb].view(torch.int16))
        assert torch.equal(sp[wb], sp1[wb])


@pytest.mark.parametrize("split", [1, 2, 63, 64, 100])
def test_split_and_carry(split):
    """Two calls, the second continuing from the block the first wrote, equal
    one pass: conv state bit-exact, outputs and state within the bar."""
    b = workloads.random_batch(workloads.BIG, [150], seed=32)
    ref = run_oracle(b)
    first = workloads.Batch("a", b.layer, b.x[:split].contiguous(), b.conv_weight, b.g[:split].contiguous(),
                            b.beta[:split].contiguous(), torch.tensor([0, split], dtype=torch.int32),
                            b.read_idx.clone(), b.write_idx.clone(), b.conv_pool, b.ssm_pool)
    o1, cp1, sp1 = run_gpu(first)
    second = workloads.Batch("b", b.layer, b.x[split:].contiguous(), b.conv_weight, b.g[split:].contiguous(),
                             b.beta[split:].contiguous(), torch.tensor([0, 150 - split], dtype=torch.int32),
                             b.write_idx.clone(), b.write_idx.clone(), cp1, sp1)
    o2, cp2, sp2 = run_gpu(second)
    out = torch.cat([o1, o2], dim=0)
    compare(b, (out, cp2, sp2), ref)


def test_trash_block_equals_explicit_zero_block():
    b = workloads.random_batch(workloads.BIG, [1, 90], seed=33, fresh=[1, 1])
    out, cp, sp = run_gpu(b)
    spare = [x for x in range(1, b.ssm_pool.shape[0]) if x not in b.write_idx.tolist()][0]
    b.conv_pool[spare] = 0
    b.ssm_pool[spare] = 0
    b.read_idx = torch.tensor([spare, spare], dtype=torch.int32)
    out2, cp2, sp2 = run_gpu(b)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    for wb in b.write_idx.tolist():
        assert torch.equal(sp[wb], sp2[wb]) and torch.equal(cp[wb].view(torch.int16), cp2[wb].view(torch.int16))


def test_padding_sequence_touches_nothing():
    b = workloads.random_batch(workloads.BIG, [5, 70, 1], seed=34)
    b.write_idx[1] = -2
    out, cp, sp = run_gpu(b, out_fill=7.0)
    assert (out[5:75].float() == 7.0).all()
    ref = run_oracle(b)
    compare(b, (out, cp, sp), ref)


def test_stream_contract_host_and_device_inputs_reusable():
    """Host offsets may be overwritten as soon as the call returns, and device
    inputs by later work on the same stream, without changing the result (the
    warmup race on the page "Continuous batching for linear attention
    layers")."""
    import linear_attention_state_amd as gdn
    from gpu_util import to_device

    b = workloads.random_batch(workloads.BIG, [100, 1, 40], seed=35)
    ref_out, ref_cp, ref_sp = run_gpu(b)
    d = to_device(b)
    L = b.layer
    out = torch.empty(b.total_tokens, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device="cuda")
    cu_host = b.cu_seqlens.clone()
    gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], cu_host,
                           d["read_idx"], d["write_idx"], d["conv_pool"], d["ssm_pool"], out)
    cu_host.fill_(-1)
    d["cu_seqlens"].fill_(0)
    d["x"].fill_(3.0)
    d["g"].fill_(0.0)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(d["ssm_pool"].cpu(), ref_sp)


def test_out_of_pool_index_is_skipped_and_reported():
    """A read block outside the pool is skipped (nothing read or written for
    that sequence, its out rows untouched) and raises GDN_DEV_BAD_INDEX; the
    other sequences are unaffected."""
    import linear_attention_state_amd as gdn

    b = workloads.random_batch(workloads.BIG, [70, 1, 5], seed=36)
    P = b.ssm_pool.shape[0]
    bad = b.read_idx.clone()
    bad[0] = P + 5
    b_bad = workloads.Batch("bad", b.layer, b.x, b.conv_weight, b.g, b.beta, b.cu_seqlens, bad,
                            b.write_idx.clone(), b.conv_pool, b.ssm_pool)
    out, cp, sp = run_gpu(b_bad, out_fill=7.0)
    bits = gdn.gdn_device_status(clear=True)
    assert bits == gdn.GDN_DEV_BAD_INDEX, bits
    assert (out[:70].float() == 7.0).all()
    # the same batch with sequence 0 as padding is what the oracle runs
    pad = b.write_idx.clone()
    pad[0] = -1
    b_pad = workloads.Batch("pad", b.layer, b.x, b.conv_weight, b.g, b.beta, b.cu_seqlens, b.read_idx.clone(),
                            pad, b.conv_pool, b.ssm_pool)
    compare(b_pad, (out, cp, sp), run_oracle(b_pad))


def test_more_sequences_than_the_launch_order_holds():
    """1,030 chunked sequences of 2-66 tokens beside one-token and empty ones,
    more than the 1,024 the longest-first launch order holds: the conv kernel
    then runs first and the chunk kernel covers every sequence in index order."""
    layer = workloads.Layer(2, 4, 128, 128, 4, "bf16")
    lengths = ([2, 3, 66, 5, 2, 9, 4, 2, 7, 3] * 103)[:1030] + [1, 0, 1, 1]
    b = workloads.random_batch(layer, lengths, seed=17)
    print("case many: %d sequences, T=%d" % (len(lengths), b.total_tokens), flush=True)
    errs = compare(b, run_gpu(b), run_oracle(b))
    print("many: out %.3e state %.3e" % (errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)
