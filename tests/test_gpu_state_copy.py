"""GPU: the fork copy (gdn_state_copy) through the C ABI.

A copy is checked bit for bit against indexing on the host; a forked request
must then continue exactly like its parent (outputs and states bitwise equal,
and within the bar of the fp64 oracle's continuation).
"""
import numpy as np
import pytest
import torch

import linear_attention_state_amd as gdn
import workloads
from gpu_util import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _copy(layer, conv_pool, ssm_pool, src, dst):
    cp, sp = conv_pool.cuda().contiguous(), ssm_pool.cuda().contiguous()
    gdn.gdn_state_copy(layer, cp, sp, torch.tensor(src, dtype=torch.int32, device="cuda"),
                       torch.tensor(dst, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return cp.cpu(), sp.cpu()


@pytest.mark.parametrize("layer", [workloads.BIG, workloads.Layer(2, 4, 64, 32, 1, "f32")])
def test_copy_is_bitwise_and_skips_bad_pairs(layer):
    b = workloads.random_batch(layer, [3, 4, 5, 6, 7, 8], seed=81, num_blocks=10)
    cp, sp = b.conv_pool, b.ssm_pool
    src, dst = [2, 5, 7, 4, 12, 6], [3, 8, 1, 4, 9, -1]  # (4, 4): same block; (12, 9), (6, -1): out of range
    gcp, gsp = _copy(layer, cp, sp, src, dst)
    ecp, esp = cp.clone(), sp.clone()
    for s_, d_ in zip(src[:3], dst[:3]):
        ecp[d_] = cp[s_]
        esp[d_] = sp[s_]
    bits = (lambda t: t.view(torch.int16)) if cp.dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(bits(gcp), bits(ecp))
    assert torch.equal(gsp, esp)


def test_forked_request_continues_like_its_parent():
    """Prefill a request into block 3, fork it into block 6, then continue both
    with the same 70 tokens in one packed batch."""
    layer = workloads.BIG
    first = workloads.random_batch(layer, [150], seed=82, num_blocks=8, fresh=[1])
    first.write_idx = torch.tensor([3], dtype=torch.int32)
    _, cp1, sp1 = run_gpu(first)
    cp2, sp2 = _copy(layer, cp1, sp1, [3], [6])
    nxt = workloads.random_batch(layer, [70], seed=83, num_blocks=8)
    x = torch.cat([nxt.x, nxt.x], dim=0)
    g = torch.cat([nxt.g, nxt.g], dim=0)
    beta = torch.cat([nxt.beta, nxt.beta], dim=0)
    both = workloads.Batch("fork", layer, x, first.conv_weight, g, beta,
                           torch.tensor([0, 70, 140], dtype=torch.int32),
                           torch.tensor([3, 6], dtype=torch.int32), torch.tensor([3, 6], dtype=torch.int32),
                           cp2, sp2)
    out, cp3, sp3 = run_gpu(both)
    assert torch.equal(out[:70].view(torch.int16), out[70:].view(torch.int16))
    assert torch.equal(sp3[3], sp3[6])
    assert torch.equal(cp3[3].view(torch.int16), cp3[6].view(torch.int16))
    errs = compare(both, (out, cp3, sp3), run_oracle(both))
    print("fork: out %.3e state %.3e" % (errs["out_rel_l2"], errs["state_rel_l2"]), flush=True)
