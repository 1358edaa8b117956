"""GPU parity of the standalone varlen conv layer (gdn_varlen_conv) against the
fp64 oracle (oracle.varlen_conv), through the C ABI.

Bar: conv states bit-exact (they are copies of stored rows); y per sequence
within relative L2 error 1e-2 in bf16 (one bf16 rounding of the output) and
1e-5 in float32; rows of a padding sequence and blocks no sequence writes
untouched.
"""
import math

import numpy as np
import pytest
import torch

import linear_attention_state_amd as gdn
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}


def _batch(C, W, lengths, seed, dtype, fresh=None, P=None):
    rng = np.random.default_rng(seed)
    n = len(lengths)
    P = P or n + 3
    T = sum(lengths)
    x = torch.tensor(rng.standard_normal((T, C)), dtype=torch.float32).to(dtype)
    w = torch.tensor(rng.standard_normal((C, W)) / math.sqrt(W), dtype=torch.float32).to(dtype)
    pool = torch.tensor(rng.standard_normal((P, max(W - 1, 0), C)), dtype=torch.float32).to(dtype)
    pool[0] = 0
    blocks = rng.choice(np.arange(1, P), size=n, replace=False).tolist()
    fresh = fresh or [False] * n
    ri = torch.tensor([0 if f else b for f, b in zip(fresh, blocks)], dtype=torch.int32)
    wi = torch.tensor(blocks, dtype=torch.int32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return x, w, pool, cu, ri, wi


def _run(x, w, pool, cu, ri, wi, silu, fill=5.0):
    d = lambda t: t.cuda().contiguous()
    y = torch.full(x.shape, fill, dtype=x.dtype, device="cuda")
    pool_d = d(pool)
    gdn.gdn_varlen_conv(d(x), d(w), d(cu), cu, d(ri), d(wi), pool_d, y, silu=silu)
    torch.cuda.synchronize()
    return y.cpu(), pool_d.cpu()


def _check(name, x, w, pool, cu, ri, wi, silu):
    print("case %s: C=%d W=%d lengths %s" % (name, x.shape[1], w.shape[1], np.diff(cu.numpy()).tolist()), flush=True)
    y, pool_g = _run(x, w, pool, cu, ri, wi, silu)
    ref, pool_r = oracle.varlen_conv(x, w, cu, ri, wi, pool, silu=silu)
    assert torch.equal(pool_g.view(torch.int16) if x.dtype == torch.bfloat16 else pool_g,
                       pool_r.view(torch.int16) if x.dtype == torch.bfloat16 else pool_r)
    worst = 0.0
    for s in range(len(ri)):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        if int(wi[s]) < 0:
            assert (y[rows].float() == 5.0).all()
            continue
        if rows.stop == rows.start:
            continue
        a, b = y[rows].double().numpy(), ref[rows]
        err = float(np.linalg.norm(a - b)) / max(float(np.linalg.norm(b)), 1e-300)
        worst = max(worst, err)
    print("%s: y %.3e" % (name, worst), flush=True)
    assert worst <= TOL[x.dtype], worst


def test_bf16_silu_ragged_in_place_and_fresh():
    x, w, pool, cu, ri, wi = _batch(8192, 4, [1, 2, 3, 17, 80, 300], seed=71, dtype=torch.bfloat16,
                                    fresh=[0, 1, 0, 0, 1, 0])
    _check("bf16-silu", x, w, pool, cu, ri, wi, True)


def test_bf16_no_activation():
    x, w, pool, cu, ri, wi = _batch(8192, 4, [40, 5, 129], seed=72, dtype=torch.bfloat16)
    _check("bf16-linear", x, w, pool, cu, ri, wi, False)


@pytest.mark.parametrize("W", [1, 2, 3])
def test_conv_widths(W):
    x, w, pool, cu, ri, wi = _batch(2048, W, [1, 9, 70], seed=73 + W, dtype=torch.bfloat16)
    _check("W%d" % W, x, w, pool, cu, ri, wi, True)


def test_float32_odd_channel_count():
    """C = 1032: not a multiple of the 512 channels a block covers."""
    x, w, pool, cu, ri, wi = _batch(1032, 4, [33, 2, 260], seed=77, dtype=torch.float32)
    _check("f32-1032", x, w, pool, cu, ri, wi, True)


def test_padding_sequence_untouched():
    x, w, pool, cu, ri, wi = _batch(1024, 4, [12, 30, 7], seed=78, dtype=torch.bfloat16)
    wi[1] = -1
    _check("padding", x, w, pool, cu, ri, wi, True)


def test_empty_and_zero_length_sequences():
    x, w, pool, cu, ri, wi = _batch(512, 4, [0, 6, 0, 1], seed=79, dtype=torch.bfloat16)
    _check("empty", x, w, pool, cu, ri, wi, False)
