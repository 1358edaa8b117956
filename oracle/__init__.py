"""fp64 CPU oracle for the packed-batch gated-delta-net layer forward.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU library never does,
and it imports nothing from the GPU library.  It is a thin ctypes wrapper around
``gdn_oracle.c`` (plain C, fp64, token by token); see that file's header for
what it follows and the readings it takes.

Parity pins: ``tests/test_oracle_pins.py`` ties each function here to closed
forms, invariants, a library routine and brute force.  The GQA head map and the
[q | k | v] channel order are conventions: parity unpinned for those two.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libgdn_oracle.so")
_lib = None


class _Layer(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("act_bf16", ctypes.c_int32),
        ("l2norm_eps", ctypes.c_double),
        ("q_scale", ctypes.c_double),
    ]


def build() -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
    )
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.gdn_oracle_forward.argtypes = [
            ctypes.POINTER(_Layer), P, P, P, P, P, ctypes.c_int32, P, P, P, P,
            ctypes.c_int32, P, P, P, ctypes.c_int32,
        ]
        lib.gdn_oracle_conv_silu.restype = None
        lib.gdn_oracle_conv_silu.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, P, P, P, P]
        lib.gdn_oracle_varlen_conv.restype = ctypes.c_int
        lib.gdn_oracle_varlen_conv.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               P, P, P, ctypes.c_int32, P, P, P, ctypes.c_int32, P]
        lib.gdn_oracle_l2norm.restype = None
        lib.gdn_oracle_l2norm.argtypes = [ctypes.c_int64, P, ctypes.c_double, ctypes.c_double]
        lib.gdn_oracle_delta_rule.restype = None
        lib.gdn_oracle_delta_rule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P, P, P, P, P, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        assert a.device.type == "cpu" and a.is_contiguous()
        return ctypes.c_void_p(a.data_ptr())
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def conv_silu(tail, x, w) -> np.ndarray:
    """Depthwise causal conv of one sequence continued from ``tail`` [W-1][C], then SiLU."""
    w = _f64(w)
    C, W = w.shape
    x = _f64(x).reshape(-1, C)
    L = x.shape[0]
    tail = _f64(tail).reshape(W - 1, C) if W > 1 else np.zeros((1, C))
    xb = x if L else np.zeros((1, C))
    y = np.zeros((max(L, 1), C))
    _load().gdn_oracle_conv_silu(C, W, L, _ptr(tail), _ptr(xb), _ptr(w), _ptr(y))
    return y[:L]


def varlen_conv(x, conv_weight, cu_seqlens, read_idx, write_idx, conv_pool, silu: bool = True):
    """Standalone varlen conv layer over a packed row (see gdn_oracle.c).

    CPU torch tensors: x [T][C] and conv_weight [C][W] and conv_pool [P][W-1][C]
    in one act dtype (bf16 or float32), indices int32.  Returns ``(y, conv_pool_new)``:
    y [T][C] float64, NaN on the rows of padding sequences."""
    bf16 = x.dtype == torch.bfloat16
    assert conv_weight.dtype == x.dtype and conv_pool.dtype == x.dtype
    x = x.contiguous()
    w = conv_weight.contiguous()
    C, W = w.shape
    T = x.shape[0]
    cu = cu_seqlens.to(torch.int32).contiguous()
    ri = read_idx.to(torch.int32).contiguous()
    wi = write_idx.to(torch.int32).contiguous()
    pool = conv_pool.clone().contiguous()
    y = np.full((max(T, 1), C), np.nan)
    rc = _load().gdn_oracle_varlen_conv(C, W, int(bf16), int(bool(silu)), _ptr(x), _ptr(w), _ptr(cu),
                                        cu.numel() - 1, _ptr(ri), _ptr(wi), _ptr(pool), pool.shape[0], _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return y[:T], pool


def l2norm(v, eps: float = 1e-6, scale: float = 1.0) -> np.ndarray:
    v = _f64(v).copy()
    _load().gdn_oracle_l2norm(v.size, _ptr(v), eps, scale)
    return v


def delta_rule(q, k, v, g, beta, S0):
    """Gated delta rule of one (sequence, value head); returns (o [L][dv], S_L [dk][dv])."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    S = _f64(S0).copy()
    L, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((max(L, 1), dv))
    if L == 0:
        return o[:0], S
    _load().gdn_oracle_delta_rule(dk, dv, L, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o))
    return o, S


def forward(layer, x, conv_weight, g, beta, cu_seqlens, read_idx, write_idx,
            conv_pool, ssm_pool, head_mask=None, threads: int | None = None):
    """Packed-batch layer forward on the CPU.

    ``layer`` has attributes num_k_heads, num_v_heads, head_k_dim, head_v_dim,
    conv_width, act_dtype ('bf16' or 'f32'), l2norm_eps and q_scale.  Tensors are
    CPU torch tensors in their stored dtypes: x/conv_weight/conv_pool in the act
    dtype, g/beta/ssm_pool float32, cu_seqlens/read_idx/write_idx int32.

    Returns ``(out, final_ssm, conv_pool_new, ssm_pool_new)``: ``out`` [T][H_v][d_v]
    float64 (NaN where a value head was masked out or a row belongs to a padding
    sequence), ``final_ssm`` [N][H_v][d_k][d_v] float64 (NaN likewise), and copies
    of both pools after the call.
    """
    lib = _load()
    bf16 = layer.act_dtype == "bf16"
    act = torch.bfloat16 if bf16 else torch.float32
    x = x.contiguous()
    conv_weight = conv_weight.contiguous()
    assert x.dtype == act and conv_weight.dtype == act and conv_pool.dtype == act
    g = g.to(torch.float32).contiguous()
    beta = beta.to(torch.float32).contiguous()
    cu = cu_seqlens.to(torch.int32).contiguous()
    ri = read_idx.to(torch.int32).contiguous()
    wi = write_idx.to(torch.int32).contiguous()
    conv_new = conv_pool.clone().contiguous()
    ssm_new = ssm_pool.clone().contiguous()
    T = x.shape[0]
    N = cu.numel() - 1
    Hv, dk, dv = layer.num_v_heads, layer.head_k_dim, layer.head_v_dim
    out = np.full((T, Hv, dv), np.nan)
    fin = np.full((N, Hv, dk, dv), np.nan)
    mask = None
    if head_mask is not None:
        mask = np.ascontiguousarray(np.asarray(head_mask, dtype=np.uint8))
        assert mask.shape == (Hv,)
    desc = _Layer(layer.num_k_heads, Hv, dk, dv, layer.conv_width, int(bf16),
                  float(layer.l2norm_eps), float(layer.q_scale))
    nthreads = threads if threads else len(os.sched_getaffinity(0))
    rc = lib.gdn_oracle_forward(
        ctypes.byref(desc), _ptr(x), _ptr(conv_weight), _ptr(g), _ptr(beta), _ptr(cu), N,
        _ptr(ri), _ptr(wi), _ptr(conv_new), _ptr(ssm_new), ssm_pool.shape[0], _ptr(mask),
        _ptr(out), _ptr(fin), nthreads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return out, fin, conv_new, ssm_new
