"""The allocation-free entry point gdn_varlen_forward_noalloc: the forward
with the library's static scratch buffer in place of a caller's workspace.

On the GPU it must equal gdn_varlen_forward bit for bit (same kernels, same
arithmetic) and meet the oracle's bar, on two calls in a row with the second
batch smaller than the first (the buffer keeps what the first call left in
it), with the launch planned on the host and on the device.  On the CPU, a
batch that needs more scratch than the buffer holds is refused before any
device work.
"""
import ctypes

import pytest
import torch

import linear_attention_state_amd as gdn
import workloads


def test_noalloc_refuses_batches_beyond_the_static_buffer():
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    T = 5000  # 5000 rows of 8192 bf16 channels: about 82 MB of scratch
    cu = (ctypes.c_int32 * 2)(0, T)
    rc = lib.gdn_varlen_forward_noalloc(ctypes.byref(gdn.make_desc(workloads.BIG)), fake, fake, fake, fake, fake, cu,
                                        1, T, fake, fake, fake, 3 * 8192 * 2, fake, 2 << 20, 8, fake, None)
    msg = gdn.gdn_last_error()
    assert rc == gdn.GDN_EWORKSPACE and "static buffer" in msg, (rc, msg)


def _run(batch, noalloc: bool, host_plan: bool):
    from gpu_util import to_device

    d = to_device(batch)
    L = batch.layer
    out = torch.full((batch.total_tokens, L.num_v_heads, L.head_v_dim), 7.0, dtype=L.torch_act, device="cuda")
    cu_host = batch.cu_seqlens if host_plan else None
    args = (L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"], cu_host, d["read_idx"],
            d["write_idx"], d["conv_pool"], d["ssm_pool"], out)
    if noalloc:
        gdn.gdn_varlen_forward_noalloc(*args)
    else:
        gdn.gdn_varlen_forward(*args)
    torch.cuda.synchronize()
    return out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu()


@pytest.mark.gpu
@pytest.mark.parametrize("host_plan", [True, False])
def test_noalloc_equals_workspace_entry_point_on_two_calls(host_plan):
    from gpu_util import compare, run_oracle

    first = workloads.random_batch(workloads.BIG, [300, 1, 70, 5, 129], seed=91, fresh=[1, 0, 1, 0, 0])
    second = workloads.random_batch(workloads.BIG, [65, 1, 2], seed=92, fresh=[0, 1, 0])
    tiny = workloads.config(0)
    for b in (first, second, tiny):
        ref = _run(b, False, host_plan)
        got = _run(b, True, host_plan)
        assert torch.equal(got[0].view(torch.uint8), ref[0].view(torch.uint8)), "outputs differ"
        assert torch.equal(got[1].view(torch.uint8), ref[1].view(torch.uint8)), "conv pools differ"
        assert torch.equal(got[2], ref[2]), "recurrent pools differ"
        errs = compare(b, got, run_oracle(b))
        print("noalloc %s host_plan=%s: %s" % (b.name, host_plan, errs), flush=True)
