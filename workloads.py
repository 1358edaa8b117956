"""Seeded synthetic inputs for the packed-batch gated-delta-net layer forward.

This module only draws numbers: it holds none of the layer's arithmetic, and
both the oracle side and the GPU side of every test and of the benchmark take
their inputs from here.  Everything is returned as CPU torch tensors in the
stored dtypes the layer uses (activations bf16 or fp32, g/beta/SSM state fp32,
indices int32).

Workloads follow the continuous-batching setting of the page "Continuous
batching for linear attention layers" (PR description and the commit that adds
the linear attention cache allocator): many requests of different lengths are
packed into one row delimited by cu_seqlens; each request owns one block of a
state pool, block 0 is the zeroed trash block that a request with no past
reads, and the request's block is overwritten in place.

Value distributions (the same for every workload):
  x ~ N(0, 1); conv weight ~ N(0, 1/W); g = -softplus(N(0, 1)) (so a = exp(g)
  lies in (0, 1)); beta = sigmoid(N(0, 1)); prior conv state ~ N(0, 1); prior
  SSM state ~ N(0, 0.1^2); every block that is neither the trash block nor a
  prior holds N(0, 1) filler so that a stray write shows up.
Draw order from ``numpy.random.default_rng(seed)``: lengths / order / block
indices, x, conv weight, g, beta, prior tails, prior states, filler.
Normal draws are taken in float32 (``standard_normal(dtype=float32)``), then
cast to the stored dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Layer:
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_width: int
    act_dtype: str  # "bf16" or "f32"
    l2norm_eps: float = 1e-6
    q_scale: float = 0.0  # <= 0 means 1/sqrt(head_k_dim)

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def torch_act(self) -> torch.dtype:
        return torch.bfloat16 if self.act_dtype == "bf16" else torch.float32


TINY = Layer(2, 2, 16, 16, 4, "f32")
BIG = Layer(16, 32, 128, 128, 4, "bf16")


@dataclasses.dataclass
class Batch:
    name: str
    layer: Layer
    x: torch.Tensor            # [T][C] act
    conv_weight: torch.Tensor  # [C][W] act
    g: torch.Tensor            # [T][H_v] fp32 (log decay, a = exp(g))
    beta: torch.Tensor         # [T][H_v] fp32
    cu_seqlens: torch.Tensor   # [N+1] int32
    read_idx: torch.Tensor     # [N] int32
    write_idx: torch.Tensor    # [N] int32
    conv_pool: torch.Tensor    # [P][W-1][C] act
    ssm_pool: torch.Tensor     # [P][H_v][d_k][d_v] fp32

    @property
    def lengths(self) -> list:
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    @property
    def total_tokens(self) -> int:
        return int(self.x.shape[0])


def _normal(rng, shape, std=1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _act(a: np.ndarray, layer: Layer) -> torch.Tensor:
    return torch.from_numpy(a).to(layer.torch_act).contiguous()


def make_batch(layer: Layer, lengths, read_idx, write_idx, num_blocks: int,
               prior_blocks, rng, name: str = "custom") -> Batch:
    """Draws x, weights, g, beta and the two pools for a batch whose lengths and
    block indices are already fixed (drawn by the caller from ``rng``)."""
    lengths = [int(v) for v in lengths]
    T = sum(lengths)
    C, W, Hv = layer.conv_channels, layer.conv_width, layer.num_v_heads
    dk, dv = layer.head_k_dim, layer.head_v_dim
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x = _normal(rng, (T, C))
    w = _normal(rng, (C, W), std=1.0 / math.sqrt(W))
    g_raw = rng.standard_normal(size=(T, Hv))
    b_raw = rng.standard_normal(size=(T, Hv))
    g = -np.logaddexp(0.0, g_raw)             # -softplus
    beta = 1.0 / (1.0 + np.exp(-b_raw))        # sigmoid
    prior_blocks = [int(b) for b in prior_blocks]
    conv_pool = np.zeros((num_blocks, max(W - 1, 0), C), dtype=np.float32)
    ssm_pool = np.zeros((num_blocks, Hv, dk, dv), dtype=np.float32)
    for b in prior_blocks:
        conv_pool[b] = _normal(rng, (W - 1, C))
    for b in prior_blocks:
        ssm_pool[b] = _normal(rng, (Hv, dk, dv), std=0.1)
    prior = set(prior_blocks)
    for b in range(1, num_blocks):
        if b not in prior:
            conv_pool[b] = _normal(rng, (W - 1, C))
            ssm_pool[b] = _normal(rng, (Hv, dk, dv))
    return Batch(
        name=name, layer=layer, x=_act(x, layer), conv_weight=_act(w, layer),
        g=torch.from_numpy(g.astype(np.float32)), beta=torch.from_numpy(beta.astype(np.float32)),
        cu_seqlens=torch.from_numpy(cu),
        read_idx=torch.tensor(read_idx, dtype=torch.int32),
        write_idx=torch.tensor(write_idx, dtype=torch.int32),
        conv_pool=_act(conv_pool, layer), ssm_pool=torch.from_numpy(ssm_pool))


def config(i: int, seed: int | None = None) -> Batch:
    """The five reference workloads.

    0: tiny all-fp32 layer (H_k=H_v=2, d=16, W=4, C=96), lengths {5, 17, 1};
       8 blocks; sequences 0 and 1 continue from blocks 3 and 6, sequence 2 has
       no past (reads block 0) and owns block 1.
    1: prefill, H_k=16, H_v=32, d=128, W=4, C=8192, bf16; 8 sequences with
       lengths uniform in [256, 4096]; 16 blocks; all start from the trash block.
    2: decode, same heads: 256 sequences of one token; 1024 blocks; blocks are
       the first 256 of a seeded permutation of 1..1023; all continue.
    3: mixed step, same heads: 64 one-token sequences and 4 chunks of 512 in a
       seeded order; 512 blocks; decodes and two chunks continue, two chunks
       start from the trash block.
    4: long prefill, same heads: 4 x 32768 tokens; 512 blocks; blocks
       {11, 200, 37, 499}, all continue.
    """
    rng = np.random.default_rng(1000 + i if seed is None else seed)
    if i == 0:
        return make_batch(TINY, [5, 17, 1], [3, 6, 0], [3, 6, 1], 8, [3, 6], rng, "tiny-fp32")
    if i == 1:
        lengths = rng.integers(256, 4096, size=8, endpoint=True)
        blocks = rng.choice(np.arange(1, 16), size=8, replace=False)
        return make_batch(BIG, lengths, [0] * 8, blocks.tolist(), 16, [], rng, "prefill-8x[256,4096]")
    if i == 2:
        perm = rng.permutation(np.arange(1, 1024))[:256]
        return make_batch(BIG, [1] * 256, perm.tolist(), perm.tolist(), 1024, perm.tolist(), rng,
                          "decode-256x1")
    if i == 3:
        kinds = ["d"] * 64 + ["c_prior"] * 2 + ["c_fresh"] * 2
        order = rng.permutation(len(kinds))
        blocks = rng.choice(np.arange(1, 512), size=len(kinds), replace=False)
        lengths, reads, writes, priors = [], [], [], []
        for pos in range(len(kinds)):
            kind = kinds[order[pos]]
            b = int(blocks[pos])
            lengths.append(1 if kind == "d" else 512)
            writes.append(b)
            if kind == "c_fresh":
                reads.append(0)
            else:
                reads.append(b)
                priors.append(b)
        return make_batch(BIG, lengths, reads, writes, 512, priors, rng, "mixed-64x1+4x512")
    if i == 4:
        blocks = [11, 200, 37, 499]
        return make_batch(BIG, [32768] * 4, blocks, blocks, 512, blocks, rng, "long-prefill-4x32768")
    raise ValueError("no workload %r" % i)


def random_batch(layer: Layer, lengths, seed: int, num_blocks: int | None = None,
                 fresh=None) -> Batch:
    """A batch of the given lengths; sequence i continues from its own block
    unless ``fresh[i]`` is true, in which case it reads the trash block."""
    rng = np.random.default_rng(seed)
    n = len(lengths)
    P = num_blocks if num_blocks is not None else n + 2
    blocks = rng.choice(np.arange(1, P), size=n, replace=False).tolist()
    fresh = fresh if fresh is not None else [False] * n
    reads = [0 if f else b for f, b in zip(fresh, blocks)]
    priors = [b for f, b in zip(fresh, blocks) if not f]
    return make_batch(layer, lengths, reads, blocks, P, priors, rng, "random")


# ---------------------------------------------------------------- Mamba2 scan
#
# Inputs of the Mamba2 scan (ssd_varlen_scan) in the same packed-batch,
# paged-state setting.  The pages give no Mamba2 shapes or distributions; the
# layer below has the mixer shape of an 8B-class Mamba2 hybrid (128 heads of
# 64, 8 groups of B and C, state 128, conv width 4), and the draws follow the
# Mamba2 initialisation: dt_bias = softplus^-1(d0) with d0 log-uniform in
# [0.001, 0.1], A = -U[1, 16], D = 1 + N(0, 0.1^2).  The conv output rows
# x | B | C ~ N(0, 1) in bf16 (one row of conv_channels, so the scan reads
# x, B and C as strided views), dt ~ N(0, 0.5^2), prior states ~ N(0, 0.5^2),
# filler blocks N(0, 1), block 0 zero.
# Draw order: lengths / blocks (by the caller), xbc, dt, dt_bias, A, D, prior
# states, filler.

@dataclasses.dataclass(frozen=True)
class SsdLayer:
    num_heads: int
    head_dim: int
    num_groups: int
    state_dim: int
    conv_width: int = 4
    dt_softplus: bool = True

    @property
    def conv_channels(self) -> int:
        return self.num_heads * self.head_dim + 2 * self.num_groups * self.state_dim


MAMBA2 = SsdLayer(128, 64, 8, 128, 4)
MAMBA2_SMALL = SsdLayer(8, 64, 2, 128, 4)


@dataclasses.dataclass
class SsdBatch:
    layer: SsdLayer
    lengths: list
    xbc: torch.Tensor        # [T][conv_channels] bf16: x | B | C
    dt: torch.Tensor         # [T][H] fp32
    dt_bias: torch.Tensor    # [H] fp32
    A: torch.Tensor          # [H] fp32
    D: torch.Tensor          # [H] fp32
    cu_seqlens: torch.Tensor
    read_idx: torch.Tensor
    write_idx: torch.Tensor
    ssm_pool: torch.Tensor   # [P][H][head_dim][state_dim] fp32

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def views(self, xbc):
        """x [T][H*P], B [T][G*N], C [T][G*N]: column slices of the xbc rows."""
        L = self.layer
        hp, gn = L.num_heads * L.head_dim, L.num_groups * L.state_dim
        return xbc[:, :hp], xbc[:, hp:hp + gn], xbc[:, hp + gn:hp + 2 * gn]


def ssd_batch(layer: SsdLayer, lengths, seed: int, fresh=None, num_blocks: int | None = None) -> SsdBatch:
    """A batch of the given lengths; sequence i continues from its own block
    unless ``fresh[i]``, in which case it reads the trash block."""
    rng = np.random.default_rng(seed)
    n = len(lengths)
    P = num_blocks if num_blocks is not None else n + 2
    blocks = rng.choice(np.arange(1, P), size=n, replace=False).tolist()
    fresh = fresh if fresh is not None else [False] * n
    reads = [0 if f else b for f, b in zip(fresh, blocks)]
    lengths = [int(v) for v in lengths]
    T = sum(lengths)
    H, Pd, N = layer.num_heads, layer.head_dim, layer.state_dim
    xbc = torch.from_numpy(_normal(rng, (T, layer.conv_channels))).to(torch.bfloat16)
    dt = _normal(rng, (T, H), std=0.5)
    d0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = d0 + np.log(-np.expm1(-d0))  # softplus^-1(d0)
    A = -rng.uniform(1.0, 16.0, size=H)
    D = 1.0 + _normal(rng, (H,), std=0.1)
    pool = np.zeros((P, H, Pd, N), dtype=np.float32)
    priors = [b for f, b in zip(fresh, blocks) if not f]
    for b in priors:
        pool[b] = _normal(rng, (H, Pd, N), std=0.5)
    for b in range(1, P):
        if b not in set(priors):
            pool[b] = _normal(rng, (H, Pd, N))
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    f32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))
    return SsdBatch(layer=layer, lengths=lengths, xbc=xbc, dt=f32(dt), dt_bias=f32(dt_bias), A=f32(A), D=f32(D),
                    cu_seqlens=torch.from_numpy(cu), read_idx=torch.tensor(reads, dtype=torch.int32),
                    write_idx=torch.tensor(blocks, dtype=torch.int32), ssm_pool=torch.from_numpy(pool))


def ssd_config(i: int, seed: int | None = None) -> SsdBatch:
    """Mamba2 workloads on MAMBA2: 0 prefill, 8 sequences of lengths uniform
    in [256, 4096], all from the trash block; 1 decode, 256 one-token
    sequences continuing from 256 of 512 blocks."""
    rng = np.random.default_rng(2000 + i if seed is None else seed)
    if i == 0:
        lengths = rng.integers(256, 4096, size=8, endpoint=True).tolist()
        return ssd_batch(MAMBA2, lengths, int(rng.integers(1 << 30)), fresh=[True] * 8, num_blocks=16)
    if i == 1:
        return ssd_batch(MAMBA2, [1] * 256, int(rng.integers(1 << 30)), num_blocks=512)
    raise ValueError("no Mamba2 workload %d" % i)
