"""Python binding of the gfx950 gated-delta-net varlen forward library.

Thin ctypes marshalling over ``include/gdn.h``: every function has the C name
and only turns torch tensors into pointers, sizes and strides; all computation
happens in the HIP kernels of ``_lib/libgdn.so``.  PyTorch is used for device
memory and the current HIP stream only.  There is no fallback: if the library
is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP, GDN_EDEVICE = 0, -1, -2, -3, -4, -5
GDN_F32, GDN_BF16 = 0, 1
GDN_DEV_WAIT_EXPIRED, GDN_DEV_BAD_INDEX = 1, 2
EXPORTS = ("gdn_state_spec", "gdn_workspace_size", "gdn_varlen_forward", "gdn_varlen_forward_noalloc",
           "gdn_varlen_conv", "gdn_state_copy",
           "ssd_varlen_scan", "kda_varlen_forward", "gdn_last_error", "gdn_device_status",
           "gdn_kernel_timing", "gdn_kernel_times", "gdn_mfma_peak_probe",
           "gdn_hbm_copy_probe")

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("gdn status %d: %s" % (status, message))
        self.status = status
        self.message = message


class gdn_layer_desc(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("l2norm_eps", ctypes.c_float),
        ("q_scale", ctypes.c_float),
    ]


class gdn_state_decl(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 16),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("dtype", ctypes.c_int32),
        ("bytes", ctypes.c_int64),
        ("align", ctypes.c_int32),
    ]


class ssd_layer_desc(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("state_dim", ctypes.c_int32),
        ("dt_softplus", ctypes.c_int32),
    ]


class gdn_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("total_ms", ctypes.c_double), ("launches", ctypes.c_int64)]


def load_library():
    """Loads ``_lib/libgdn.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgdn.so is not built (expected %s); run `python -m linear_attention_state_amd.build`"
                % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.gdn_state_spec.restype = ctypes.c_int
        lib.gdn_state_spec.argtypes = [ctypes.POINTER(gdn_layer_desc), ctypes.POINTER(gdn_state_decl)]
        lib.gdn_workspace_size.restype = ctypes.c_int
        lib.gdn_workspace_size.argtypes = [ctypes.POINTER(gdn_layer_desc), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_size_t)]
        lib.gdn_last_error.restype = ctypes.c_char_p
        lib.gdn_last_error.argtypes = []
        lib.gdn_varlen_forward.restype = ctypes.c_int
        lib.gdn_varlen_forward.argtypes = [
            ctypes.POINTER(gdn_layer_desc), P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P,
            P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32, P, P, ctypes.c_size_t, P]
        lib.gdn_varlen_forward_noalloc.restype = ctypes.c_int
        lib.gdn_varlen_forward_noalloc.argtypes = [
            ctypes.POINTER(gdn_layer_desc), P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P,
            P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32, P, P]
        lib.gdn_varlen_conv.restype = ctypes.c_int
        lib.gdn_varlen_conv.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, ctypes.c_int32,
            ctypes.c_int32, P, P, P, ctypes.c_int64, ctypes.c_int32, P, P]
        lib.gdn_state_copy.restype = ctypes.c_int
        lib.gdn_state_copy.argtypes = [ctypes.POINTER(gdn_layer_desc), P, ctypes.c_int64, P, ctypes.c_int64,
                                       ctypes.c_int32, P, P, ctypes.c_int32, P]
        lib.kda_varlen_forward.restype = ctypes.c_int
        lib.kda_varlen_forward.argtypes = [
            ctypes.POINTER(gdn_layer_desc), P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P,
            ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32, P, P, ctypes.c_size_t, P]
        lib.ssd_varlen_scan.restype = ctypes.c_int
        lib.ssd_varlen_scan.argtypes = [
            ctypes.POINTER(ssd_layer_desc), P, ctypes.c_int64, P, P, ctypes.c_int64, P, P, P, P, P, P,
            ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int64, ctypes.c_int32, P, P]
        lib.gdn_device_status.restype = ctypes.c_int
        lib.gdn_device_status.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_uint32), P]
        lib.gdn_kernel_timing.restype = ctypes.c_int
        lib.gdn_kernel_timing.argtypes = [ctypes.c_int]
        lib.gdn_kernel_times.restype = ctypes.c_int
        lib.gdn_kernel_times.argtypes = [ctypes.POINTER(gdn_kernel_time), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int32)]
        lib.gdn_mfma_peak_probe.restype = ctypes.c_int
        lib.gdn_mfma_peak_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_double), P]
        lib.gdn_hbm_copy_probe.restype = ctypes.c_int
        lib.gdn_hbm_copy_probe.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_double), P]
        _lib = lib
    return _lib


def make_desc(layer) -> gdn_layer_desc:
    """Descriptor from any object with the layer's attributes (``workloads.Layer``)."""
    return gdn_layer_desc(int(layer.num_k_heads), int(layer.num_v_heads), int(layer.head_k_dim),
                          int(layer.head_v_dim), int(layer.conv_width),
                          GDN_BF16 if layer.act_dtype == "bf16" else GDN_F32,
                          float(layer.l2norm_eps), float(layer.q_scale))


def gdn_last_error() -> str:
    return load_library().gdn_last_error().decode()


def _check(rc: int):
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())


def gdn_state_spec(layer) -> list:
    arr = (gdn_state_decl * 2)()
    _check(load_library().gdn_state_spec(ctypes.byref(make_desc(layer)), arr))
    return [dict(name=d.name.decode(), shape=tuple(d.shape[i] for i in range(d.ndim)), dtype=d.dtype,
                 bytes=d.bytes, align=d.align) for d in arr]


def gdn_workspace_size(layer, total_tokens: int, num_seqs: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().gdn_workspace_size(ctypes.byref(make_desc(layer)), int(total_tokens), int(num_seqs),
                                             ctypes.byref(out)))
    return out.value


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _view_ptr(t, name):
    """Device pointer of a strided view (rows at the tensor's own stride)."""
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return ctypes.c_void_p(t.data_ptr())


def gdn_varlen_forward(layer, x, conv_weight, g, beta, cu_seqlens, cu_seqlens_host, read_idx, write_idx,
                       conv_pool, ssm_pool, out, workspace=None, stream=None):
    """Enqueues the packed-batch forward on ``stream`` (default: torch's current
    stream).  Device tensors as in ``gdn.h``; ``cu_seqlens_host`` is a CPU int32
    tensor (or list) with the same offsets, or None to plan the launch on the
    device (graph capture).  Pools are updated in place; block strides are taken
    from the pool tensors' first dimension."""
    import torch

    lib = load_library()
    if cu_seqlens_host is None:  # plan on the device (graph capture)
        cu_h = None
        num_seqs = cu_seqlens.numel() - 1
    else:
        if not isinstance(cu_seqlens_host, torch.Tensor):
            cu_seqlens_host = torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
        cu_h = cu_seqlens_host.to(torch.int32).contiguous()
        if cu_h.is_cuda:
            raise ValueError("cu_seqlens_host must be host memory")
        num_seqs = cu_h.numel() - 1
    total = int(x.shape[0])
    for name, t, dt in (("cu_seqlens", cu_seqlens, torch.int32), ("read_idx", read_idx, torch.int32),
                        ("write_idx", write_idx, torch.int32), ("g", g, torch.float32),
                        ("beta", beta, torch.float32), ("ssm_pool", ssm_pool, torch.float32)):
        if t.dtype != dt:
            raise ValueError("%s must be %s" % (name, dt))
    if workspace is None:
        nbytes = gdn_workspace_size(layer, total, num_seqs)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    conv_stride = conv_pool.stride(0) * conv_pool.element_size() if conv_pool is not None and conv_pool.dim() else 0
    ssm_stride = ssm_pool.stride(0) * ssm_pool.element_size()
    rc = lib.gdn_varlen_forward(
        ctypes.byref(make_desc(layer)), _dev_ptr(x, "x"), _dev_ptr(conv_weight, "conv_weight"),
        _dev_ptr(g, "g"), _dev_ptr(beta, "beta"), _dev_ptr(cu_seqlens, "cu_seqlens"),
        ctypes.c_void_p(cu_h.data_ptr()) if cu_h is not None else None, num_seqs, total,
        _dev_ptr(read_idx, "read_idx"),
        _dev_ptr(write_idx, "write_idx"),
        _dev_ptr(conv_pool, "conv_pool") if conv_pool is not None and conv_pool.numel() else None,
        conv_stride, _dev_ptr(ssm_pool, "ssm_pool"), ssm_stride, int(ssm_pool.shape[0]),
        _dev_ptr(out, "out"), _dev_ptr(workspace, "workspace"), workspace.numel(),
        ctypes.c_void_p(stream))
    _check(rc)
    return out


def gdn_varlen_forward_noalloc(layer, x, conv_weight, g, beta, cu_seqlens, cu_seqlens_host, read_idx, write_idx,
                               conv_pool, ssm_pool, out, stream=None):
    """gdn_varlen_forward without a workspace: the library's static scratch
    buffer serves instead (at most GDN_STATIC_SCRATCH_BYTES; calls that overlap
    in time on one device race).  Arguments as for gdn_varlen_forward."""
    import torch

    lib = load_library()
    if cu_seqlens_host is None:
        cu_h = None
        num_seqs = cu_seqlens.numel() - 1
    else:
        if not isinstance(cu_seqlens_host, torch.Tensor):
            cu_seqlens_host = torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
        cu_h = cu_seqlens_host.to(torch.int32).contiguous()
        if cu_h.is_cuda:
            raise ValueError("cu_seqlens_host must be host memory")
        num_seqs = cu_h.numel() - 1
    for name, t, dt in (("cu_seqlens", cu_seqlens, torch.int32), ("read_idx", read_idx, torch.int32),
                        ("write_idx", write_idx, torch.int32), ("g", g, torch.float32),
                        ("beta", beta, torch.float32), ("ssm_pool", ssm_pool, torch.float32)):
        if t.dtype != dt:
            raise ValueError("%s must be %s" % (name, dt))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    conv_stride = conv_pool.stride(0) * conv_pool.element_size() if conv_pool is not None and conv_pool.dim() else 0
    ssm_stride = ssm_pool.stride(0) * ssm_pool.element_size()
    rc = lib.gdn_varlen_forward_noalloc(
        ctypes.byref(make_desc(layer)), _dev_ptr(x, "x"), _dev_ptr(conv_weight, "conv_weight"),
        _dev_ptr(g, "g"), _dev_ptr(beta, "beta"), _dev_ptr(cu_seqlens, "cu_seqlens"),
        ctypes.c_void_p(cu_h.data_ptr()) if cu_h is not None else None, num_seqs, int(x.shape[0]),
        _dev_ptr(read_idx, "read_idx"), _dev_ptr(write_idx, "write_idx"),
        _dev_ptr(conv_pool, "conv_pool") if conv_pool is not None and conv_pool.numel() else None,
        conv_stride, _dev_ptr(ssm_pool, "ssm_pool"), ssm_stride, int(ssm_pool.shape[0]),
        _dev_ptr(out, "out"), ctypes.c_void_p(stream))
    _check(rc)
    return out


def gdn_varlen_conv(x, conv_weight, cu_seqlens, cu_seqlens_host, read_idx, write_idx, conv_pool, y,
                    silu: bool = True, stream=None):
    """Enqueues the standalone varlen conv layer (``gdn.h``): x [T][C] and
    conv_weight [C][W] in bf16 or float32, conv_pool [P][W-1][C] updated in place,
    y [T][C] written."""
    import torch

    lib = load_library()
    if not isinstance(cu_seqlens_host, torch.Tensor):
        cu_seqlens_host = torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
    cu_h = cu_seqlens_host.to(torch.int32).contiguous()
    if cu_h.is_cuda:
        raise ValueError("cu_seqlens_host must be host memory")
    if x.dtype not in (torch.bfloat16, torch.float32) or conv_weight.dtype != x.dtype or y.dtype != x.dtype:
        raise ValueError("x, conv_weight and y must share one dtype, bf16 or float32")
    for name, t in (("cu_seqlens", cu_seqlens), ("read_idx", read_idx), ("write_idx", write_idx)):
        if t.dtype != torch.int32:
            raise ValueError("%s must be int32" % name)
    C, W = int(conv_weight.shape[0]), int(conv_weight.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    has_pool = conv_pool is not None and conv_pool.numel() > 0
    conv_stride = conv_pool.stride(0) * conv_pool.element_size() if has_pool else 0
    num_blocks = int(conv_pool.shape[0]) if conv_pool is not None else 0
    rc = lib.gdn_varlen_conv(
        C, W, GDN_BF16 if x.dtype == torch.bfloat16 else GDN_F32, 1 if silu else 0,
        _dev_ptr(x, "x"), _dev_ptr(conv_weight, "conv_weight"), _dev_ptr(cu_seqlens, "cu_seqlens"),
        ctypes.c_void_p(cu_h.data_ptr()), cu_h.numel() - 1, int(x.shape[0]), _dev_ptr(read_idx, "read_idx"),
        _dev_ptr(write_idx, "write_idx"), _dev_ptr(conv_pool, "conv_pool") if has_pool else None, conv_stride,
        num_blocks, _dev_ptr(y, "y"), ctypes.c_void_p(stream))
    _check(rc)
    return y


def gdn_state_copy(layer, conv_pool, ssm_pool, src, dst, stream=None):
    """Enqueues the fork copy of both states of blocks ``src`` to blocks ``dst``
    (device int32 tensors of equal length); the pools are updated in place."""
    import torch

    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.numel() != dst.numel():
        raise ValueError("src and dst must be int32 tensors of one length")
    if ssm_pool.dtype != torch.float32:
        raise ValueError("ssm_pool must be float32")
    if stream is None:
        stream = torch.cuda.current_stream(ssm_pool.device).cuda_stream
    has_conv = conv_pool is not None and conv_pool.numel() > 0
    conv_stride = conv_pool.stride(0) * conv_pool.element_size() if has_conv else 0
    _check(load_library().gdn_state_copy(
        ctypes.byref(make_desc(layer)), _dev_ptr(conv_pool, "conv_pool") if has_conv else None, conv_stride,
        _dev_ptr(ssm_pool, "ssm_pool"), ssm_pool.stride(0) * ssm_pool.element_size(), int(ssm_pool.shape[0]),
        _dev_ptr(src, "src"), _dev_ptr(dst, "dst"), int(src.numel()), ctypes.c_void_p(stream)))


def kda_varlen_forward(layer, x, conv_weight, g, beta, cu_seqlens, cu_seqlens_host, read_idx, write_idx,
                       conv_pool, ssm_pool, out, workspace=None, stream=None):
    """Enqueues the KDA layer forward: as gdn_varlen_forward, with g [T][H_v][d_k]
    float32 (a log decay per key channel); cu_seqlens_host is required.
    ``workspace``: a uint8 device tensor of at least gdn_workspace_size bytes
    (allocated here when None); ``False`` runs every sequence token by token."""
    import torch

    if g.dtype != torch.float32 or g.dim() != 3 or g.shape[2] != layer.head_k_dim:
        raise ValueError("g must be float32 [T][H_v][d_k]")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    host = cu_seqlens_host.to(torch.int32).contiguous()
    if workspace is None:
        nbytes = gdn_workspace_size(layer, int(x.shape[0]), int(read_idx.numel()))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    ws_ptr = None if workspace is False else _dev_ptr(workspace, "workspace")
    ws_bytes = 0 if workspace is False else workspace.numel()
    W = int(layer.conv_width)
    has_conv = conv_pool is not None and conv_pool.numel() > 0
    conv_stride = conv_pool.stride(0) * conv_pool.element_size() if has_conv else 0
    _check(load_library().kda_varlen_forward(
        ctypes.byref(make_desc(layer)), _dev_ptr(x, "x"), _dev_ptr(conv_weight, "conv_weight"), _dev_ptr(g, "g"),
        _dev_ptr(beta, "beta"), _dev_ptr(cu_seqlens, "cu_seqlens"), ctypes.cast(host.data_ptr(), ctypes.c_void_p),
        int(read_idx.numel()), int(x.shape[0]), _dev_ptr(read_idx, "read_idx"), _dev_ptr(write_idx, "write_idx"),
        _dev_ptr(conv_pool, "conv_pool") if (has_conv and W > 1) else None, conv_stride,
        _dev_ptr(ssm_pool, "ssm_pool"), ssm_pool.stride(0) * ssm_pool.element_size(), int(ssm_pool.shape[0]),
        _dev_ptr(out, "out"), ws_ptr, ws_bytes, ctypes.c_void_p(stream)))


def ssd_varlen_scan(layer, x, B, C, dt, A, cu_seqlens, cu_seqlens_host, read_idx, write_idx, ssm_pool, y,
                    dt_bias=None, D=None, stream=None):
    """Enqueues the Mamba2 scan of a packed batch (``layer``: num_heads,
    head_dim, num_groups, state_dim, dt_softplus).  x: [T][>= H*P] bf16 rows
    (a 2-D view, row stride x.stride(0)); B and C: [T][>= G*N] bf16 views with
    one row stride; dt [T][H] fp32; A, D, dt_bias [H] fp32; ssm_pool
    [P_blocks][H][head_dim][state_dim] fp32 (updated in place); y
    [T][H][head_dim] bf16.  cu_seqlens_host may be None."""
    import torch

    for name, t in (("x", x), ("B", B), ("C", C)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("%s must be a 2-D bf16 view with unit column stride" % name)
    if B.stride(0) != C.stride(0):
        raise ValueError("B and C must share one row stride")
    for name, t in (("dt", dt), ("A", A), ("ssm_pool", ssm_pool)) + tuple(
            (n, t) for n, t in (("dt_bias", dt_bias), ("D", D)) if t is not None):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float32 tensor" % name)
    if y.dtype != torch.bfloat16 or not y.is_contiguous():
        raise ValueError("y must be a contiguous bf16 tensor")
    if stream is None:
        stream = torch.cuda.current_stream(y.device).cuda_stream
    T, n = int(dt.shape[0]), int(read_idx.numel())
    host = None
    if cu_seqlens_host is not None:
        h = cu_seqlens_host.to(torch.int32).contiguous()
        host = ctypes.cast(h.data_ptr(), ctypes.c_void_p)
    desc = ssd_layer_desc(int(layer.num_heads), int(layer.head_dim), int(layer.num_groups), int(layer.state_dim),
                          1 if layer.dt_softplus else 0)
    opt = lambda t, nm: _dev_ptr(t, nm) if t is not None else None
    _check(load_library().ssd_varlen_scan(
        ctypes.byref(desc), _view_ptr(x, "x"), int(x.stride(0)), _view_ptr(B, "B"), _view_ptr(C, "C"), int(B.stride(0)),
        _dev_ptr(dt, "dt"), opt(dt_bias, "dt_bias"), _dev_ptr(A, "A"), opt(D, "D"), _dev_ptr(cu_seqlens, "cu_seqlens"),
        host, n, T, _dev_ptr(read_idx, "read_idx"), _dev_ptr(write_idx, "write_idx"), _dev_ptr(ssm_pool, "ssm_pool"),
        ssm_pool.stride(0) * ssm_pool.element_size(), int(ssm_pool.shape[0]), _dev_ptr(y, "y"),
        ctypes.c_void_p(stream)))


def gdn_device_status(clear: bool = True, stream=None) -> int:
    """The device-side status bits raised since the last clear (0 when none;
    GDN_DEV_WAIT_EXPIRED, GDN_DEV_BAD_INDEX).  Waits for ``stream`` (default:
    torch's current stream) first.  Does not raise for set bits: the caller
    decides what they mean for its test."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    bits = ctypes.c_uint32(0)
    rc = load_library().gdn_device_status(int(bool(clear)), ctypes.byref(bits), ctypes.c_void_p(stream))
    if rc not in (GDN_OK, GDN_EDEVICE):
        _check(rc)
    return int(bits.value)


def gdn_mfma_peak_probe(dtype: str = "bf16", iters: int = 4096, stream=None) -> float:
    """The dense MFMA rate the device reaches on back-to-back products, TFLOP/s
    (dtype "bf16" or "f32"); waits for the probe."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    lib = load_library()
    out = ctypes.c_double(0.0)
    _check(lib.gdn_mfma_peak_probe(GDN_BF16 if dtype == "bf16" else GDN_F32, int(iters), ctypes.byref(out),
                                   ctypes.c_void_p(stream)))
    return out.value


def gdn_hbm_copy_probe(src, dst, reps: int = 10, stream=None) -> float:
    """The HBM rate of the library's streaming copy from the device tensor
    ``src`` into ``dst`` (contiguous, same number of bytes), GB/s of bytes read
    plus bytes written; waits for the copies."""
    import torch

    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    out = ctypes.c_double(0.0)
    _check(load_library().gdn_hbm_copy_probe(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                             nbytes, int(reps), ctypes.byref(out), ctypes.c_void_p(stream)))
    return out.value


def gdn_kernel_timing(enable: bool) -> None:
    """Turns per-kernel HIP event timing of later forward calls on or off."""
    _check(load_library().gdn_kernel_timing(1 if enable else 0))


def gdn_kernel_times() -> dict:
    """{kernel: (total_ms, launches)} of the timed launches so far (waits for them)."""
    arr = (gdn_kernel_time * 16)()
    n = ctypes.c_int32(0)
    _check(load_library().gdn_kernel_times(arr, 16, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].total_ms, arr[i].launches) for i in range(min(n.value, 16))}
