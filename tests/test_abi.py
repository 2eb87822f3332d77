"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/kfac.h declares, answers workspace queries, and rejects bad arguments
before touching the device."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kfac.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:kfac_status|int32_t|size_t|const char\s*\*)\s*(kfac_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import fac_second_order_amd._lib as L
    return L


def test_header_declares_the_five_calls():
    names = declared_functions()
    for base in ("kfac_factors", "kfac_invert", "kfac_precondition", "kfac_bn_diag", "kfac_pack_sym"):
        assert base in names and base + "_workspace" in names


def test_every_declared_symbol_is_exported(lib):
    so = ctypes.CDLL(lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(so, n)]
    assert not missing, missing


def test_status_strings_and_version(lib):
    so = lib._lib
    assert lib.kfac_version() >= 100
    for code in (0, -1, -2, -3, -4):
        assert so.kfac_status_string(code)
    assert so.kfac_status_string(12345) == b"unknown status"


def test_kernel_names(lib):
    n = lib.kfac_timing_kernels()
    names = [lib.kfac_kernel_name(i) for i in range(n)]
    assert "inv_update_kernel" in names and "syrk_tile_kernel" in names
    assert lib.kfac_kernel_name(n) == ""


def test_timing_only_validates_ids(lib):
    so = lib._lib
    n = lib.kfac_timing_kernels()
    assert so.kfac_timing_only(n) == -1
    assert so.kfac_timing_only(-2) == -1
    assert so.kfac_timing_only(0) == 0
    assert so.kfac_timing_only(-1) == 0


def test_workspace_queries_resnet50(lib):
    L = synth.conv_layers(32)
    n_all = [l.d_a for l in L] + [l.d_g for l in L]
    assert lib.kfac_factors_workspace(L) > 0
    assert lib.kfac_invert_workspace(n_all) > 0
    assert lib.kfac_pack_sym_workspace(n_all) > 0
    assert lib.kfac_precondition_workspace([l.d_g for l in L], [l.d_a for l in L]) > 0
    assert lib.kfac_bn_diag_workspace(synth.bn_layers(32)) > 0
    assert lib.kfac_invert_workspace([]) == 0


def test_invert_workspace_covers_panels(lib):
    # per matrix: two blocks (U_kk^-1 and P^-1 of the pivot) and a (group x block) x n
    # panel buffer (the Y panels of a group's steps) with rows padded to 16 bytes
    block, group = lib.kfac_invert_schedule()
    assert block == 128 and 1 <= group <= 8
    b = lib.kfac_invert_workspace([4609])
    assert b >= 4 * (2 * block * block + group * block * 4612)


def _status(fn, *args):
    return fn(*args)


def test_invalid_arguments_return_errors(lib):
    so = lib._lib
    c = ctypes
    n = (c.c_int32 * 2)(4, 0)
    sz = c.c_size_t()
    assert so.kfac_pack_sym_workspace(2, n, c.byref(sz)) == -1
    assert b"n[1]" in so.kfac_last_error()
    n = (c.c_int32 * 1)(4)
    ptrs = (c.c_void_p * 1)(None)
    assert so.kfac_pack_sym(1, n, ptrs, ptrs, 3, None, 0, None) == -1       # bad direction
    assert so.kfac_pack_sym(1, n, ptrs, ptrs, -1, None, 0, None) == -1      # bad direction
    assert so.kfac_pack_sym(1, n, ptrs, ptrs, 0, None, 0, None) == -1       # NULL matrix
    big = (c.c_int32 * 1)(40000)
    assert so.kfac_invert_workspace(1, big, c.byref(sz)) == -1
    assert so.kfac_pack_sym(-1, n, ptrs, ptrs, 0, None, 0, None) == -1
    # count 0 is a no-op
    assert so.kfac_pack_sym(0, None, None, None, 0, None, 0, None) == 0


def test_invalid_layer_geometry(lib):
    bad = synth.Layer("bad", 2, 8, 8, 4, 7, 8, 4, 3, 3, 1, 1, 1, 1, 1)   # h_out should be 8
    with pytest.raises(lib.KfacError) as e:
        lib.kfac_factors_workspace([bad])
    assert "h_out" in str(e.value)
    good = synth.Layer("ok", 2, 8, 8, 4, 8, 8, 4, 3, 3, 1, 1, 1, 1, 1)
    so = lib._lib
    arr = lib._layers([good])
    p = (ctypes.c_void_p * 1)(None)
    # ema_decay out of range is refused before any pointer is looked at
    assert so.kfac_factors(arr, 1, 0, p, p, p, p, ctypes.c_float(1.5), None, 0, None) == -1
    assert so.kfac_factors(arr, 1, 7, p, p, p, p, ctypes.c_float(0.0), None, 0, None) == -2


def test_factors_full_validation(lib):
    """kfac_factors_full refuses a full-matrix pointer that is not 4-byte aligned and an
    out-of-range ema_decay before touching the device; the binding checks the full
    matrices' dtype, shape and count."""
    import torch
    layer = synth.Layer("c1x1", 2, 8, 8, 16, 8, 8, 8, 1, 1, 1, 1, 0, 0, 1)
    so = lib._lib
    arr = lib._layers([layer])
    c = ctypes
    act = (c.c_void_p * 1)(0x10000)        # never dereferenced: the call fails first
    gout = (c.c_void_p * 1)(0x20000)
    A = (c.c_void_p * 1)(0x30000)
    G = (c.c_void_p * 1)(0x40000)
    good = (c.c_void_p * 1)(0x50000)
    odd = (c.c_void_p * 1)(0x50002)
    assert so.kfac_factors_full(arr, 1, 0, act, gout, A, G, odd, good, c.c_float(0.0), None, 0, None) == -1
    assert b"misaligned" in so.kfac_last_error()
    assert so.kfac_factors_full(arr, 1, 0, act, gout, A, G, good, odd, c.c_float(0.0), None, 0, None) == -1
    assert so.kfac_factors_full(arr, 1, 0, act, gout, A, G, good, good, c.c_float(-0.5), None, 0, None) == -1
    x = torch.zeros(2, 8, 8, 16, dtype=torch.float16)
    g = torch.zeros(2, 8, 8, 8, dtype=torch.float16)
    Ap, Gp = torch.zeros(17 * 18 // 2), torch.zeros(8 * 9 // 2)
    with pytest.raises(TypeError):
        lib.kfac_factors_full([layer], [x], [g], [Ap], [Gp], [torch.zeros(16, 16)], [None])   # d_A is 17
    with pytest.raises(TypeError):
        lib.kfac_factors_full([layer], [x], [g], [Ap], [Gp], [torch.zeros(17, 17, dtype=torch.float64)], [None])
    with pytest.raises(ValueError):
        lib.kfac_factors_full([layer], [x], [g], [Ap], [Gp], [], [None])


def test_bn_and_precondition_validation(lib):
    so = lib._lib
    c = ctypes
    bn = lib._bns([synth.BNLayer("b", 2, 0, 4)])
    sz = c.c_size_t()
    assert so.kfac_bn_diag_workspace(bn, 1, c.byref(sz)) == -1
    dg = (c.c_int32 * 1)(0)
    da = (c.c_int32 * 1)(5)
    assert so.kfac_precondition_workspace(1, dg, da, c.byref(sz)) == -1


def test_update_variants_validation(lib):
    """The eq. (8) variants refuse a non-finite lr, a missing weight array and an
    output that is also the weight buffer, before any device work."""
    so = lib._lib
    c = ctypes
    dg = (c.c_int32 * 1)(4)
    da = (c.c_int32 * 1)(5)
    fake = (c.c_void_p * 1)(0x10000)
    other = (c.c_void_p * 1)(0x20000)
    nan = c.c_float(float("nan"))
    one = c.c_float(1.0)
    assert so.kfac_precondition_update(1, dg, da, fake, fake, fake, 1, fake, other, nan, None, 0, None) == -1
    assert b"lr" in so.kfac_last_error()
    assert so.kfac_precondition_update(1, dg, da, fake, fake, fake, 1, fake, None, one, None, 0, None) == -1
    assert so.kfac_precondition_update(1, dg, da, fake, fake, fake, 1, other, other, one, None, 0, None) == -1
    assert b"same buffer" in so.kfac_last_error()
    assert so.kfac_precondition_update(0, None, None, None, None, None, 1, None, None, one, None, 0, None) == 0
    bn = lib._bns([synth.BNLayer("b", 2, 3, 4)])
    assert so.kfac_bn_update(bn, 1, 1, fake, fake, fake, other, None, one, c.c_float(0.0),
                             c.c_float(1e-3), None, 0, None) == -1
    assert so.kfac_bn_update(bn, 1, 1, fake, fake, fake, other, other, one, c.c_float(0.0),
                             c.c_float(1e-3), None, 0, None) == -1
    assert b"overlaps" in so.kfac_last_error()
    # accumulation other than fp32 / fp64
    assert so.kfac_precondition_ex(1, dg, da, fake, fake, fake, 1, fake, None, one, 3, None, 0, None) == -2
    assert so.kfac_precondition_ex(1, dg, da, fake, fake, fake, 1, None, None, one, 2, None, 0, None) == -1
    inf = c.c_float(float("inf"))
    assert so.kfac_bn_update(bn, 1, 1, fake, fake, fake, other, (c.c_void_p * 1)(0x30000), inf,
                             c.c_float(0.0), c.c_float(1e-3), None, 0, None) == -1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing libkfac.so is an ImportError."""
    import importlib.util
    src = os.path.join(ROOT, "fac_second_order_amd", "_lib.py")
    pkg = tmp_path / "fake_pkg"
    pkg.mkdir()
    (pkg / "_lib.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("fake_lib", str(pkg / "_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="not built"):
        spec.loader.exec_module(mod)


def test_patch_rows_workspace(lib):
    """An fp16 convolution whose channel count rules out 16-byte gathers (conv1, 3
    channels) has its patch rows written to the workspace (row pitch rounded up to 8
    halves); a matrix of 2 GiB or more stays on the per-element gathers instead."""
    def conv1(n):
        return [synth.Layer("conv1", n, 224, 224, 3, 112, 112, 64, 7, 7, 2, 2, 3, 3, 1)]
    rows32 = 32 * 112 * 112
    small = lib.kfac_factors_workspace(conv1(32), lib.KFAC_F16)
    fp32 = lib.kfac_factors_workspace(conv1(32), lib.KFAC_F32)
    assert small >= rows32 * 152 * 2                 # 147 patch columns padded to 152
    assert fp32 < rows32 * 152 * 2                   # fp32 inputs take their own path
    big = lib.kfac_factors_workspace(conv1(600), lib.KFAC_F16)
    assert 600 * 112 * 112 * 152 * 2 >= 1 << 31
    assert big < 600 * 112 * 112 * 152 * 2           # no row buffer at this size


def test_invert_refine_validation(lib):
    """kfac_invert_refine rejects bad sizes, NULL, aliased or misaligned pointers and
    non-finite shifts before touching the device; its workspace holds E and C per matrix."""
    so = lib._lib
    c = ctypes
    sz = c.c_size_t()
    n = (c.c_int32 * 2)(300, 7)
    assert so.kfac_invert_refine_workspace(2, n, c.byref(sz)) == 0
    assert sz.value >= 4 * 2 * (300 * 300 + 7 * 7)
    bad = (c.c_int32 * 1)(0)
    assert so.kfac_invert_refine_workspace(1, bad, c.byref(sz)) == -1
    one = (c.c_int32 * 1)(4)
    shift = (c.c_float * 1)(1e-3)
    nan = (c.c_float * 1)(float("nan"))
    nullp = (c.c_void_p * 1)(None)
    a = (c.c_void_p * 1)(0x1000)
    b = (c.c_void_p * 1)(0x2000)
    odd = (c.c_void_p * 1)(0x2002)
    assert so.kfac_invert_refine(1, one, nullp, shift, b, None, 0, None) == -1   # NULL matrix
    assert so.kfac_invert_refine(1, one, a, shift, a, None, 0, None) == -1       # mat aliases inv
    assert so.kfac_invert_refine(1, one, a, shift, odd, None, 0, None) == -1     # misaligned
    assert so.kfac_invert_refine(1, one, a, nan, b, None, 0, None) == -1         # NaN shift
    assert so.kfac_invert_refine(0, None, None, None, None, None, 0, None) == 0  # no-op


def test_refine_rejects_partial_overlaps(lib):
    """Any byte shared by an inv buffer and a mat or another inv buffer is refused on
    the host; mat buffers may overlap each other."""
    so = lib._lib
    c = ctypes
    two = (c.c_int32 * 2)(4, 4)            # 64 bytes per matrix
    shift = (c.c_float * 2)(1e-3, 1e-3)

    def ptrs(*v):
        return (c.c_void_p * len(v))(*v)

    assert so.kfac_invert_refine(2, two, ptrs(0x1000, 0x2000), shift, ptrs(0x3000, 0x1020), None, 0, None) == -1
    assert b"overlaps" in so.kfac_last_error()
    assert so.kfac_invert_refine(2, two, ptrs(0x1000, 0x2000), shift, ptrs(0x2000, 0x3000), None, 0, None) == -1
    assert so.kfac_invert_refine(2, two, ptrs(0x1000, 0x2000), shift, ptrs(0x3000, 0x3030), None, 0, None) == -1
    # adjacent (not overlapping) buffers and overlapping mats pass the check; the call
    # then stops at the device check or the missing workspace, not at the arguments
    assert so.kfac_invert_refine(2, two, ptrs(0x1000, 0x1020), shift, ptrs(0x3000, 0x3040), None, 0, None) != -1


def test_sizes_past_32bit_offsets_are_unsupported(lib):
    """Input tensors of 2^31 bytes or more (factors) and operands of 2^31 bytes or more
    (preconditioning, refinement: d > 23170) are refused with KFAC_ERR_UNSUPPORTED."""
    so = lib._lib
    c = ctypes
    sz = c.c_size_t()
    big_act = synth.Layer("big", 64, 512, 512, 64, 512, 512, 8, 1, 1, 1, 1, 0, 0, 1)   # 2 GiB fp16
    with pytest.raises(lib.KfacError) as e:
        lib.kfac_factors_workspace([big_act], lib.KFAC_F16)
    assert e.value.status == -2
    ok = synth.Layer("ok", 32, 512, 512, 64, 512, 512, 8, 1, 1, 1, 1, 0, 0, 1)       # 1 GiB fp16
    assert lib.kfac_factors_workspace([ok], lib.KFAC_F16) > 0
    with pytest.raises(lib.KfacError):
        lib.kfac_factors_workspace([ok], lib.KFAC_F32)                                # 2 GiB fp32
    d = (c.c_int32 * 1)(23171)
    s = (c.c_int32 * 1)(64)
    assert so.kfac_precondition_workspace(1, s, d, c.byref(sz)) == -2
    assert so.kfac_precondition_workspace(1, d, s, c.byref(sz)) == -2
    assert so.kfac_invert_refine_workspace(1, d, c.byref(sz)) == -2
    d[0] = 23170
    assert so.kfac_precondition_workspace(1, s, d, c.byref(sz)) == 0
