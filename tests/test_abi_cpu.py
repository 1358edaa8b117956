"""The C ABI on the CPU: the library loads, exports every function gdn.h
declares, describes the states, and rejects bad arguments with a readable
message before touching the GPU (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import linear_attention_state_amd as gdn
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b((?:gdn|ssd|kda)_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gdn.load_library()
    names = _declared()
    assert set(names) == set(gdn.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_state_spec_bf16_layer():
    conv, rec = gdn.gdn_state_spec(workloads.BIG)
    assert conv["name"] == "conv" and conv["shape"] == (3, 8192) and conv["bytes"] == 3 * 8192 * 2
    assert rec["name"] == "recurrent" and rec["shape"] == (32, 128, 128) and rec["bytes"] == 2 * 1024 * 1024
    assert conv["align"] == rec["align"] == 128


def test_state_spec_width1_has_empty_conv_state():
    conv, _ = gdn.gdn_state_spec(workloads.Layer(1, 1, 16, 16, 1, "f32"))
    assert conv["shape"] == (0, 48) and conv["bytes"] == 0


def test_workspace_size():
    n = gdn.gdn_workspace_size(workloads.BIG, 1000, 3)
    assert n >= 1000 * 8192 * 2 and n % 256 == 0


@pytest.mark.parametrize("field,value,status", [
    ("num_k_heads", 0, gdn.GDN_EINVAL),
    ("num_v_heads", 3, gdn.GDN_EINVAL),
    ("head_k_dim", 48, gdn.GDN_EUNSUPPORTED),
    ("head_v_dim", 256, gdn.GDN_EUNSUPPORTED),
    ("conv_width", 5, gdn.GDN_EUNSUPPORTED),
    ("conv_width", 0, gdn.GDN_EINVAL),
    ("act_dtype", "fp8", gdn.GDN_EINVAL),
])
def test_bad_layer_rejected(field, value, status):
    import dataclasses
    layer = dataclasses.replace(workloads.BIG, **{field: value})
    with pytest.raises(gdn.GdnError) as ei:
        if field == "act_dtype":
            d = gdn.make_desc(workloads.BIG)
            d.act_dtype = 7
            arr = (gdn.gdn_state_decl * 2)()
            rc = gdn.load_library().gdn_state_spec(ctypes.byref(d), arr)
            gdn._check(rc)
        else:
            gdn.gdn_state_spec(layer)
    assert ei.value.status == status and ei.value.message


def _call(layer, cu_host, T, n=None, **over):
    """gdn_varlen_forward with fake (never dereferenced) device pointers."""
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    n = len(cu_host) - 1 if n is None else n
    cu = (ctypes.c_int32 * len(cu_host))(*cu_host)
    args = dict(x=fake, w=fake, g=fake, b=fake, cu=fake, cuh=cu, n=n, T=T, ri=fake, wi=fake,
                conv=fake, cstride=3 * 8192 * 2, ssm=fake, sstride=2 << 20, P=8, out=fake,
                ws=fake, wsb=1 << 40, st=None)
    args.update(over)
    rc = lib.gdn_varlen_forward(ctypes.byref(gdn.make_desc(layer)), args["x"], args["w"], args["g"], args["b"],
                                args["cu"], args["cuh"], args["n"], args["T"], args["ri"], args["wi"],
                                args["conv"], args["cstride"], args["ssm"], args["sstride"], args["P"],
                                args["out"], args["ws"], args["wsb"], args["st"])
    return rc, gdn.gdn_last_error()


@pytest.mark.parametrize("cu,T,over,status,needle", [
    ([0], 0, {}, gdn.GDN_EINVAL, "no sequences"),
    ([1, 4], 4, {}, gdn.GDN_EINVAL, "cu_seqlens[0]"),
    ([0, 5, 3], 3, {}, gdn.GDN_EINVAL, "decreases"),
    ([0, 5, 9], 8, {}, gdn.GDN_EINVAL, "total_tokens"),
    ([0] * 1026, 0, {"cuh": None}, gdn.GDN_EUNSUPPORTED, "planning on the device"),
    ([0, 4], 4, {"ssm": None}, gdn.GDN_EINVAL, "ssm_pool"),
    ([0, 4], 4, {"conv": None}, gdn.GDN_EINVAL, "conv_pool"),
    ([0, 4], 4, {"P": 1}, gdn.GDN_EINVAL, "num_blocks"),
    ([0, 4], 4, {"sstride": (2 << 20) - 128}, gdn.GDN_EINVAL, "ssm_block_stride"),
    ([0, 4], 4, {"sstride": (2 << 20) + 8}, gdn.GDN_EINVAL, "ssm_block_stride"),
    ([0, 4], 4, {"cstride": 3 * 8192 * 2 - 16}, gdn.GDN_EINVAL, "conv_block_stride"),
    ([0, 4], 4, {"cstride": 3 * 8192 * 2 + 4}, gdn.GDN_EINVAL, "conv_block_stride"),
    ([0, 4], 4, {"wsb": 100}, gdn.GDN_EWORKSPACE, "workspace"),
    ([0, 4], 4, {"ws": None}, gdn.GDN_EWORKSPACE, "workspace"),
    ([0, 4], 4, {"x": ctypes.c_void_p((1 << 20) + 8)}, gdn.GDN_EINVAL, "aligned"),
])
def test_forward_rejects_bad_arguments(cu, T, over, status, needle):
    rc, msg = _call(workloads.BIG, cu, T, **over)
    assert rc == status and needle in msg, (rc, msg)


def _conv_call(cu_host, T, C=1024, W=4, act=gdn.GDN_BF16, **over):
    """gdn_varlen_conv with fake (never dereferenced) device pointers."""
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    cu = (ctypes.c_int32 * len(cu_host))(*cu_host)
    args = dict(C=C, W=W, act=act, x=fake, w=fake, cu=fake, cuh=cu, n=len(cu_host) - 1, T=T, ri=fake, wi=fake,
                conv=fake, cstride=(W - 1) * C * 2, P=8, y=fake)
    args.update(over)
    rc = lib.gdn_varlen_conv(args["C"], args["W"], args["act"], 1, args["x"], args["w"], args["cu"], args["cuh"],
                             args["n"], args["T"], args["ri"], args["wi"], args["conv"], args["cstride"], args["P"],
                             args["y"], None)
    return rc, gdn.gdn_last_error()


@pytest.mark.parametrize("cu,T,over,status,needle", [
    ([0], 0, {}, gdn.GDN_EINVAL, "no sequences"),
    ([0, 5, 3], 3, {}, gdn.GDN_EINVAL, "decreases"),
    ([0, 5, 9], 8, {}, gdn.GDN_EINVAL, "total_tokens"),
    ([0, 4], 4, {"C": 1020, "cstride": 3 * 1020 * 2}, gdn.GDN_EUNSUPPORTED, "multiple of 8"),
    ([0, 4], 4, {"W": 5}, gdn.GDN_EUNSUPPORTED, "conv_width"),
    ([0, 4], 4, {"W": 0}, gdn.GDN_EINVAL, "conv_width"),
    ([0, 4], 4, {"act": 7}, gdn.GDN_EINVAL, "act_dtype"),
    ([0, 4], 4, {"conv": None}, gdn.GDN_EINVAL, "conv_pool"),
    ([0, 4], 4, {"P": 1}, gdn.GDN_EINVAL, "num_blocks"),
    ([0, 4], 4, {"cstride": 3 * 1024 * 2 - 16}, gdn.GDN_EINVAL, "conv_block_stride"),
    ([0, 4], 4, {"y": ctypes.c_void_p((1 << 20) + 8)}, gdn.GDN_EINVAL, "aligned"),
    ([0, 4], 4, {"cuh": None}, gdn.GDN_EINVAL, "cu_seqlens_host"),
])
def test_varlen_conv_rejects_bad_arguments(cu, T, over, status, needle):
    rc, msg = _conv_call(cu, T, **over)
    assert rc == status and needle in msg, (rc, msg)


def _copy_call(**over):
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    args = dict(conv=fake, cstride=3 * 8192 * 2, ssm=fake, sstride=2 << 20, P=8, src=fake, dst=fake, n=3)
    args.update(over)
    rc = lib.gdn_state_copy(ctypes.byref(gdn.make_desc(workloads.BIG)), args["conv"], args["cstride"], args["ssm"],
                            args["sstride"], args["P"], args["src"], args["dst"], args["n"], None)
    return rc, gdn.gdn_last_error()


@pytest.mark.parametrize("over,status,needle", [
    ({"n": -1}, gdn.GDN_EINVAL, "negative"),
    ({"src": None}, gdn.GDN_EINVAL, "src or dst"),
    ({"ssm": None}, gdn.GDN_EINVAL, "ssm_pool"),
    ({"conv": None}, gdn.GDN_EINVAL, "conv_pool"),
    ({"sstride": (2 << 20) - 16}, gdn.GDN_EINVAL, "ssm_block_stride"),
    ({"cstride": 3 * 8192 * 2 + 8}, gdn.GDN_EINVAL, "conv_block_stride"),
    ({"ssm": ctypes.c_void_p((1 << 20) + 4)}, gdn.GDN_EINVAL, "aligned"),
])
def test_state_copy_rejects_bad_arguments(over, status, needle):
    rc, msg = _copy_call(**over)
    assert rc == status and needle in msg, (rc, msg)


def test_state_copy_of_nothing_is_ok():
    rc, _ = _copy_call(n=0, src=None, dst=None)
    assert rc == gdn.GDN_OK


def _ssd_call(cu_host, T, H=128, P=64, G=8, N=128, **over):
    """ssd_varlen_scan with fake (never dereferenced) device pointers."""
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    cu = (ctypes.c_int32 * len(cu_host))(*cu_host)
    args = dict(x=fake, xs=H * P + 2 * G * N, b=fake, c=fake, bcs=H * P + 2 * G * N, dt=fake, bias=None, A=fake,
                D=None, cu=fake, cuh=cu, n=len(cu_host) - 1, T=T, ri=fake, wi=fake, ssm=fake,
                sstride=H * P * N * 4, nb=8, y=fake)
    args.update(over)
    desc = gdn.ssd_layer_desc(H, P, G, N, 1)
    rc = lib.ssd_varlen_scan(ctypes.byref(desc), args["x"], args["xs"], args["b"], args["c"], args["bcs"], args["dt"],
                             args["bias"], args["A"], args["D"], args["cu"], args["cuh"], args["n"], args["T"],
                             args["ri"], args["wi"], args["ssm"], args["sstride"], args["nb"], args["y"], None)
    return rc, gdn.gdn_last_error()


@pytest.mark.parametrize("cu,T,kw,status,needle", [
    ([0, 4], 4, {"H": 12, "G": 8}, gdn.GDN_EINVAL, "multiple of G"),
    ([0, 4], 4, {"P": 128}, gdn.GDN_EUNSUPPORTED, "head_dim"),
    ([0, 4], 4, {"N": 64}, gdn.GDN_EUNSUPPORTED, "state_dim"),
    ([0, 5, 3], 3, {}, gdn.GDN_EINVAL, "decreases"),
    ([0, 5, 9], 8, {}, gdn.GDN_EINVAL, "total_tokens"),
    ([0, 4], 4, {"A": None}, gdn.GDN_EINVAL, "NULL"),
    ([0, 4], 4, {"y": None}, gdn.GDN_EINVAL, "NULL"),
    ([0, 4], 4, {"nb": 0}, gdn.GDN_EINVAL, "num_blocks"),
    ([0, 4], 4, {"sstride": 128 * 64 * 128 * 4 - 16}, gdn.GDN_EINVAL, "ssm_block_stride"),
    ([0, 4], 4, {"xs": 10244}, gdn.GDN_EINVAL, "row strides"),
    ([0, 4], 4, {"bcs": 1016}, gdn.GDN_EINVAL, "row strides"),
    ([0, 4], 4, {"xs": 1 << 24}, gdn.GDN_EUNSUPPORTED, "2^23"),
    ([0, 4], 4, {"b": ctypes.c_void_p((1 << 20) + 8)}, gdn.GDN_EINVAL, "aligned"),
])
def test_ssd_scan_rejects_bad_arguments(cu, T, kw, status, needle):
    shape = {k: kw.pop(k) for k in ("H", "P", "G", "N") if k in kw}
    rc, msg = _ssd_call(cu, T, **shape, **kw)
    assert rc == status and needle in msg, (rc, msg)


def test_ssd_scan_of_no_sequences_is_ok():
    rc, _ = _ssd_call([0], 0, cuh=None, cu=None, n=0)
    assert rc == gdn.GDN_OK


def _kda_call(cu_host, T, **over):
    """kda_varlen_forward with fake (never dereferenced) device pointers."""
    lib = gdn.load_library()
    fake = ctypes.c_void_p(1 << 20)
    cu = (ctypes.c_int32 * len(cu_host))(*cu_host) if cu_host is not None else None
    args = dict(x=fake, w=fake, g=fake, b=fake, cu=fake, cuh=cu, n=(len(cu_host) - 1) if cu_host else 1, T=T,
                ri=fake, wi=fake, conv=fake, cstride=3 * 8192 * 2, ssm=fake, sstride=2 << 20, P=8, out=fake,
                ws=None, wsb=0)
    args.update(over)
    rc = lib.kda_varlen_forward(ctypes.byref(gdn.make_desc(workloads.BIG)), args["x"], args["w"], args["g"], args["b"],
                                args["cu"], args["cuh"], args["n"], args["T"], args["ri"], args["wi"], args["conv"],
                                args["cstride"], args["ssm"], args["sstride"], args["P"], args["out"], args["ws"],
                                args["wsb"], None)
    return rc, gdn.gdn_last_error()


@pytest.mark.parametrize("cu,T,over,status,needle", [
    ([0], 0, {}, gdn.GDN_EINVAL, "no sequences"),
    (None, 4, {}, gdn.GDN_EINVAL, "cu_seqlens_host"),
    ([0, 5, 3], 3, {}, gdn.GDN_EINVAL, "decreases"),
    ([0, 5, 9], 8, {}, gdn.GDN_EINVAL, "total_tokens"),
    ([0, 4], 4, {"g": None}, gdn.GDN_EINVAL, "non-NULL"),
    ([0, 4], 4, {"ssm": None}, gdn.GDN_EINVAL, "ssm_pool"),
    ([0, 4], 4, {"P": 1}, gdn.GDN_EINVAL, "num_blocks"),
    ([0, 4], 4, {"sstride": (2 << 20) - 16}, gdn.GDN_EINVAL, "ssm_block_stride"),
    ([0, 4], 4, {"out": ctypes.c_void_p((1 << 20) + 8)}, gdn.GDN_EINVAL, "aligned"),
    ([0, 4], 4, {"ws": ctypes.c_void_p(1 << 20), "wsb": 1000}, gdn.GDN_EWORKSPACE, "workspace"),
    ([0, 4], 4, {"ws": ctypes.c_void_p((1 << 20) + 64), "wsb": 1 << 30}, gdn.GDN_EINVAL, "256-byte"),
])
def test_kda_forward_rejects_bad_arguments(cu, T, over, status, needle):
    rc, msg = _kda_call(cu, T, **over)
    assert rc == status and needle in msg, (rc, msg)


def test_mfma_probe_rejects_bad_arguments_before_any_launch():
    lib = gdn.load_library()
    out = ctypes.c_double(0.0)
    assert lib.gdn_mfma_peak_probe(gdn.GDN_BF16, 16, None, None) == gdn.GDN_EINVAL
    assert b"tflops" in lib.gdn_last_error()
    assert lib.gdn_mfma_peak_probe(7, 16, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert b"dtype" in lib.gdn_last_error()
    assert lib.gdn_mfma_peak_probe(gdn.GDN_F32, 0, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert lib.gdn_mfma_peak_probe(gdn.GDN_F32, (1 << 20) + 1, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert b"iters" in lib.gdn_last_error()


def test_copy_probe_rejects_bad_arguments_before_any_launch():
    """Every check runs on the host before the device is touched (the pointers
    below are never dereferenced)."""
    lib = gdn.load_library()
    out = ctypes.c_double(0.0)
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 30)
    assert lib.gdn_hbm_copy_probe(a, b, 1024, 1, None, None) == gdn.GDN_EINVAL
    assert b"gbs" in lib.gdn_last_error()
    assert lib.gdn_hbm_copy_probe(None, b, 1024, 1, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert b"NULL" in lib.gdn_last_error()
    for n in (0, -16, 1000, (1 << 36) + 16):
        assert lib.gdn_hbm_copy_probe(a, b, n, 1, ctypes.byref(out), None) == gdn.GDN_EINVAL
        assert b"multiple of 16" in lib.gdn_last_error()
    assert lib.gdn_hbm_copy_probe(ctypes.c_void_p((1 << 20) + 8), b, 1024, 1, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert b"aligned" in lib.gdn_last_error()
    assert lib.gdn_hbm_copy_probe(a, ctypes.c_void_p((1 << 20) + 512), 1024, 1, ctypes.byref(out), None) == gdn.GDN_EINVAL
    assert b"overlap" in lib.gdn_last_error()
    for r in (0, 1001):
        assert lib.gdn_hbm_copy_probe(a, b, 1024, r, ctypes.byref(out), None) == gdn.GDN_EINVAL
        assert b"reps" in lib.gdn_last_error()
