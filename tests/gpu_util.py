"""Helpers for the GPU parity tests: run a batch through the HIP library and
through the oracle, and compare the two the way the tests require."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import linear_attention_state_amd as gdn

TOL = {"bf16": 1e-2, "f32": 1e-4}


def to_device(batch, dev="cuda"):
    return {name: getattr(batch, name).to(dev).contiguous()
            for name in ("x", "conv_weight", "g", "beta", "cu_seqlens", "read_idx", "write_idx",
                         "conv_pool", "ssm_pool")}


def run_gpu(batch, out_fill: float | None = None, sync=True):
    """One call of gdn_varlen_forward on a fresh device copy of the batch.
    Returns CPU copies of (out, conv_pool, ssm_pool)."""
    d = to_device(batch)
    L = batch.layer
    T = batch.total_tokens
    out = torch.empty(T, L.num_v_heads, L.head_v_dim, dtype=L.torch_act, device="cuda")
    if out_fill is not None:
        out.fill_(out_fill)
    gdn.gdn_varlen_forward(L, d["x"], d["conv_weight"], d["g"], d["beta"], d["cu_seqlens"],
                           batch.cu_seqlens, d["read_idx"], d["write_idx"], d["conv_pool"],
                           d["ssm_pool"], out)
    if sync:
        torch.cuda.synchronize()
    return out.cpu(), d["conv_pool"].cpu(), d["ssm_pool"].cpu()


def run_oracle(batch, head_mask=None):
    return oracle.forward(batch.layer, batch.x, batch.conv_weight, batch.g, batch.beta,
                          batch.cu_seqlens, batch.read_idx, batch.write_idx, batch.conv_pool,
                          batch.ssm_pool, head_mask=head_mask)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / max(nb, 1e-300)


def compare(batch, gpu, ref, head_mask=None, tol=None):
    """Max relative L2 error over (sequence, value head) slabs of the outputs
    and of the final recurrent states; conv pool bit-exact; blocks that no
    sequence writes bit-identical; the trash block still zero.  Returns a dict
    of the worst errors (asserts the bar)."""
    out_g, cp_g, sp_g = gpu
    out_r, fin_r, cp_r, sp_r = ref
    L = batch.layer
    tol = TOL[L.act_dtype] if tol is None else tol
    heads = range(L.num_v_heads) if head_mask is None else [m for m in range(L.num_v_heads) if head_mask[m]]
    cu = batch.cu_seqlens.tolist()
    og = out_g.double().numpy()
    worst_o = worst_s = 0.0
    for s in range(len(cu) - 1):
        wb = int(batch.write_idx[s])
        if wb < 0:
            continue
        for m in heads:
            if cu[s + 1] > cu[s]:
                e = rel_l2(og[cu[s]:cu[s + 1], m], out_r[cu[s]:cu[s + 1], m])
                worst_o = max(worst_o, e)
            e = rel_l2(sp_g[wb, m].double().numpy(), fin_r[s, m])
            worst_s = max(worst_s, e)
    assert worst_o <= tol, "output rel L2 %.3e > %.1e" % (worst_o, tol)
    assert worst_s <= tol, "state rel L2 %.3e > %.1e" % (worst_s, tol)
    # conv states: bit-exact, whole pool (written blocks and untouched ones)
    assert torch.equal(cp_g.view(torch.uint8) if cp_g.numel() else cp_g,
                       cp_r.view(torch.uint8) if cp_r.numel() else cp_r), "conv pool differs"
    written = set(int(v) for v in batch.write_idx.tolist() if v >= 0)
    untouched = [b for b in range(batch.ssm_pool.shape[0]) if b not in written]
    idx = torch.tensor(untouched, dtype=torch.long)
    assert torch.equal(sp_g[idx], batch.ssm_pool[idx]), "a block no sequence writes changed"
    assert not sp_g[0].any(), "trash block written"
    return {"out_rel_l2": worst_o, "state_rel_l2": worst_s}
