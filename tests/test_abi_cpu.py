"""The C ABI on a host without a GPU: symbols, workspace arithmetic, host-side validation.

No call here reaches a kernel: every case returns from host validation before
any device work, and the device check itself is exercised on a host with no
GPU (it must report MOE_ERR_UNSUPPORTED_DEVICE, not crash).
"""

import ctypes
import os

import pytest
import torch

import ragged_grouped_gemm_histogram_amd as moe

OK, NULLP, SHAPE, ALIGN, WS, DEV, LAUNCH, TOO_LARGE = range(8)

# The host-sanitizer test re-runs this file against a build whose host code carries
# AddressSanitizer and UndefinedBehaviorSanitizer checks.
if os.environ.get("MOE_TEST_LIB"):
    moe.LIB_PATH = os.environ["MOE_TEST_LIB"]
    moe._LIB = None


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_exports_every_header_symbol(lib):
    names = moe.header_functions()
    assert set(names) >= {"moe_permute", "grouped_swiglu_expert", "moe_unpermute", "moe_permute_workspace_bytes",
                          "moe_gemm_up_swiglu", "moe_gemm_down", "moe_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert lib.moe_status_string(s).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(99)


def test_workspace_bytes(lib):
    f = moe.permute_workspace_bytes
    assert f(0, 1, 4) == 0
    assert f(10, 1, 4) == 1 * 4 * 4  # one chunk of 256 slots, 4 experts, int32
    assert f(8192, 8, 64) == (65536 // 256) * 64 * 4
    assert f(257, 1, 3) == 2 * 3 * 4
    assert f(-1, 1, 4) == 0 and f(1, 0, 4) == 0 and f(1, 1, 0) == 0 and f(1, 1, 1025) == 0
    assert f(2**31, 1, 4) == 0  # T*k must stay below 2^31


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def permute(lib, T=4, k=2, d=8, E=4, x=FAKE, ids=FAKE, xp=FAKE, counts=FAKE, offs=FAKE, perm=FAKE, inv=FAKE,
            ws=FAKE, wsb=1 << 20):
    return lib.moe_permute(x, ids, T, k, d, E, xp, counts, offs, perm, inv, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(E=0), SHAPE), (dict(E=1025), SHAPE), (dict(d=12), SHAPE),
    (dict(d=0), SHAPE), (dict(T=2**31, k=1), SHAPE), (dict(T=2**30, k=2), SHAPE),
    (dict(x=None), NULLP), (dict(ids=None), NULLP), (dict(counts=None), NULLP),
    (dict(offs=None), NULLP), (dict(perm=None), NULLP), (dict(inv=None), NULLP), (dict(ws=None), NULLP),
    (dict(x=FAKE + 8), ALIGN), (dict(xp=FAKE + 2), ALIGN), (dict(ids=FAKE + 2), ALIGN), (dict(inv=FAKE + 1), ALIGN),
    (dict(wsb=3), WS),
])
def test_permute_validation(lib, kw, status):
    assert permute(lib, **kw) == status


def permute_noalloc(lib, T=4, k=2, d=8, E=4, x=FAKE, ids=FAKE, xp=FAKE, counts=FAKE, offs=FAKE, perm=FAKE,
                    inv=FAKE):
    return lib.moe_permute_noalloc(x, ids, T, k, d, E, xp, counts, offs, perm, inv, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(E=0), SHAPE), (dict(E=1025), SHAPE), (dict(d=12), SHAPE),
    (dict(T=2**31, k=1), SHAPE),
    # the fixed table holds 2^20 entries: E * ceil(T*k / 256) beyond it is refused before anything else
    (dict(T=70000, k=4, E=1024), TOO_LARGE), (dict(T=1 << 22, k=1, E=65), TOO_LARGE),
    (dict(ids=None), NULLP), (dict(counts=None), NULLP), (dict(perm=None), NULLP), (dict(inv=None), NULLP),
    (dict(x=None), NULLP), (dict(ids=FAKE + 2), ALIGN), (dict(xp=FAKE + 2), ALIGN),
])
def test_permute_noalloc_validation(lib, kw, status):
    assert permute_noalloc(lib, **kw) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid sizes with placeholder pointers: host without a GPU only")
def test_permute_noalloc_limit_boundary(lib):
    # exactly 2^20 entries (E = 64, 16384 chunks of 256 slots) passes validation; one slot more does not
    T = 16384 * 256
    assert permute_noalloc(lib, T=T, k=1, E=64) in (OK, DEV)
    assert permute_noalloc(lib, T=T + 1, k=1, E=64) == TOO_LARGE
    # no row copy asked for: x may be NULL
    assert permute_noalloc(lib, x=None, xp=None) in (OK, DEV)


def test_permute_empty_tensors_may_be_null(lib):
    # T = 0: every slot tensor is empty, so NULL is fine; only offsets/counts (E entries) are required.
    st = permute(lib, T=0, x=None, ids=None, xp=None, perm=None, inv=None, ws=None, wsb=0)
    assert st in (OK, DEV)  # no GPU here: validation passes, then the device check reports
    assert permute(lib, T=0, x=None, ids=None, xp=None, perm=None, inv=None, ws=None, wsb=0, counts=None) == NULLP


def gemm(lib, fn, cap=16, d=16, h=16, E=2, a=FAKE, offs=FAKE, w=FAKE, out=FAKE):
    return getattr(lib, fn)(a, offs, w, cap, d, h, E, out, None)


@pytest.mark.parametrize("fn", ["moe_gemm_up_swiglu", "moe_gemm_down"])
@pytest.mark.parametrize("kw,status", [
    (dict(cap=-1), SHAPE), (dict(d=4), SHAPE), (dict(h=20), SHAPE), (dict(E=0), SHAPE), (dict(E=2000), SHAPE),
    (dict(a=None), NULLP), (dict(offs=None), NULLP), (dict(w=None), NULLP), (dict(out=None), NULLP),
    (dict(a=FAKE + 4), ALIGN), (dict(w=FAKE + 8), ALIGN), (dict(out=FAKE + 2), ALIGN), (dict(offs=FAKE + 2), ALIGN),
])
def test_gemm_validation(lib, fn, kw, status):
    assert gemm(lib, fn, **kw) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid sizes with placeholder pointers: host without a GPU only")
def test_gemm_width_limit(lib):
    # a 256-row output tile is addressed with 32-bit offsets: d and h stop at 2^20 for every grouped GEMM call
    top = 1 << 20
    for fn in ("moe_gemm_up_swiglu", "moe_gemm_down"):
        assert gemm(lib, fn, d=top, h=top) == DEV
        assert gemm(lib, fn, d=top + 8) == SHAPE and gemm(lib, fn, h=top + 8) == SHAPE
    assert lib.moe_gemm_up_swiglu_u(FAKE, FAKE, FAKE, 16, 16, top + 8, 2, FAKE, FAKE, None) == SHAPE
    assert lib.moe_gemm_up_swiglu_gather(FAKE, FAKE, 8, 2, FAKE, FAKE, top + 8, 16, 2, FAKE, None) == SHAPE
    assert dgrad(lib, d_in=top + 8) == SHAPE and wgrad(lib, d_out=top + 8) == SHAPE
    # the permute and unpermute rows stay valid up to 2^24 columns
    assert permute(lib, d=top + 8) == DEV
    assert lib.moe_unpermute(FAKE, FAKE, FAKE, 4, 2, top + 8, FAKE, None) == DEV


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(d=12), SHAPE), (dict(E=0), SHAPE), (dict(T=2**30, k=2), SHAPE),
    (dict(x=None), NULLP), (dict(perm=None), NULLP), (dict(offs=None), NULLP), (dict(w=None), NULLP),
    (dict(out=None), NULLP), (dict(x=FAKE + 8), ALIGN), (dict(perm=FAKE + 2), ALIGN), (dict(out=FAKE + 4), ALIGN),
])
def test_gather_gemm_validation(lib, kw, status):
    a = dict(x=FAKE, perm=FAKE, T=8, k=2, offs=FAKE, w=FAKE, d=16, h=16, E=2, out=FAKE)
    a.update(kw)
    assert lib.moe_gemm_up_swiglu_gather(a["x"], a["perm"], a["T"], a["k"], a["offs"], a["w"], a["d"], a["h"],
                                         a["E"], a["out"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(cap=-1), SHAPE), (dict(d=4), SHAPE), (dict(h=20), SHAPE), (dict(E=0), SHAPE),
    (dict(a=None), NULLP), (dict(offs=None), NULLP), (dict(w=None), NULLP), (dict(out=None), NULLP),
    (dict(u=None), NULLP), (dict(u=FAKE + 8), ALIGN), (dict(out=FAKE + 2), ALIGN), (dict(offs=FAKE + 2), ALIGN),
])
def test_save_u_gemm_validation(lib, kw, status):
    a = dict(a=FAKE, offs=FAKE, w=FAKE, cap=16, d=16, h=16, E=2, out=FAKE, u=FAKE)
    a.update(kw)
    assert lib.moe_gemm_up_swiglu_u(a["a"], a["offs"], a["w"], a["cap"], a["d"], a["h"], a["E"], a["out"], a["u"],
                                    None) == status
    if not torch.cuda.is_available():
        assert lib.moe_gemm_up_swiglu_u(FAKE, FAKE, FAKE, 16, 16, 16, 2, FAKE, FAKE, None) == DEV
    # an empty capacity needs no row buffers
    assert lib.moe_gemm_up_swiglu_u(None, FAKE, FAKE, 0, 16, 16, 2, None, None, None) in (OK, DEV)


def test_permute_without_gather_needs_no_rows(lib):
    # x_perm = NULL: no row copy, so x may be NULL too; everything else is still required
    assert permute(lib, x=None, xp=None) in (OK, DEV)
    assert permute(lib, x=None, xp=None, perm=None) == NULLP


def test_grouped_validation_checks_both_halves(lib):
    f = lib.grouped_swiglu_expert
    assert f(FAKE, FAKE, FAKE, None, 16, 16, 16, 2, FAKE, FAKE, None) == NULLP  # w_down
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 16, 16, 2, FAKE, None, None) == NULLP  # y_perm
    assert f(FAKE, FAKE, FAKE, FAKE + 2, 16, 16, 16, 2, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 12, 16, 2, FAKE, FAKE, None) == SHAPE


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(d=6), SHAPE),
    (dict(yp=None), NULLP), (dict(inv=None), NULLP), (dict(w=None), NULLP), (dict(y=None), NULLP),
    (dict(yp=FAKE + 2), ALIGN), (dict(y=FAKE + 8), ALIGN), (dict(w=FAKE + 2), ALIGN),
])
def test_unpermute_validation(lib, kw, status):
    a = dict(yp=FAKE, inv=FAKE, w=FAKE, T=4, k=2, d=8, y=FAKE)
    a.update(kw)
    assert lib.moe_unpermute(a["yp"], a["inv"], a["w"], a["T"], a["k"], a["d"], a["y"], None) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour on a host without a GPU")
def test_device_check_without_gpu(lib):
    assert permute(lib) == DEV
    assert permute_noalloc(lib) == DEV
    assert gemm(lib, "moe_gemm_down") == DEV
    assert lib.moe_unpermute(FAKE, FAKE, FAKE, 4, 2, 8, FAKE, None) == DEV


def test_binding_rejects_bad_tensors():
    x = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises((TypeError, ValueError)):
        moe.moe_permute(x, torch.zeros((4, 2), dtype=torch.int32), 4)


def dgrad(lib, dy=FAKE, offs=FAKE, w=FAKE, layout=0, cap=16, d_in=16, d_out=24, E=2, dx=FAKE):
    return lib.moe_grouped_dgrad(dy, offs, w, layout, cap, d_in, d_out, E, dx, None)


def wgrad(lib, x=FAKE, dy=FAKE, offs=FAKE, layout=0, cap=16, d_in=16, d_out=24, E=2, dw=FAKE, ws=FAKE,
          wsb=1 << 30):
    return lib.moe_grouped_wgrad(x, dy, offs, layout, cap, d_in, d_out, E, dw, ws, wsb, None)


def test_wgrad_workspace_bytes(lib):
    f = moe.wgrad_workspace_bytes
    assert f(4096, 64, 64, 4) == 0  # no expert can exceed 4096 rows
    assert f(4097, 64, 64, 4) == 3 * 64 * 64 * 4  # ceil(2 * 4097 / 4096) slots
    assert f(65536, 2048, 1536, 64) == 32 * 2048 * 1536 * 4
    assert f(-1, 64, 64, 4) == 0 and f(100, 12, 64, 4) == 0 and f(100, 64, 64, 0) == 0


def test_wgrad_workspace_validation(lib):
    assert wgrad(lib, cap=65536, ws=None) == NULLP
    assert wgrad(lib, cap=65536, wsb=100) == WS
    assert wgrad(lib, cap=65536, ws=FAKE + 8) == ALIGN
    assert wgrad(lib, cap=100, ws=None, wsb=0) in (OK, DEV)  # nothing to split: no workspace needed


@pytest.mark.parametrize("fn", [dgrad, wgrad])
@pytest.mark.parametrize("kw,status", [
    (dict(layout=2), SHAPE), (dict(layout=-1), SHAPE), (dict(cap=-1), SHAPE), (dict(d_in=12), SHAPE),
    (dict(d_out=0), SHAPE), (dict(E=0), SHAPE), (dict(E=1025), SHAPE),
    (dict(offs=None), NULLP), (dict(dy=None), NULLP), (dict(offs=FAKE + 2), ALIGN), (dict(dy=FAKE + 8), ALIGN),
])
def test_backward_gemm_validation(lib, fn, kw, status):
    assert fn(lib, **kw) == status


def test_backward_gemm_operand_checks(lib):
    assert dgrad(lib, w=None) == NULLP and dgrad(lib, dx=None) == NULLP and dgrad(lib, w=FAKE + 4) == ALIGN
    assert wgrad(lib, x=None) == NULLP and wgrad(lib, dw=None) == NULLP and wgrad(lib, x=FAKE + 2) == ALIGN
    # an empty capacity needs no row buffers (Wgrad still writes E * d_in * d_out zeros)
    assert dgrad(lib, dy=None, dx=None, cap=0) in (OK, DEV)
    assert wgrad(lib, x=None, dy=None, cap=0) in (OK, DEV)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(d=6), SHAPE),
    (dict(g=None), NULLP), (dict(inv=None), NULLP), (dict(dx=None), NULLP),
    (dict(g=FAKE + 2), ALIGN), (dict(dx=FAKE + 8), ALIGN), (dict(inv=FAKE + 2), ALIGN),
])
def test_permute_backward_validation(lib, kw, status):
    a = dict(g=FAKE, inv=FAKE, T=4, k=2, d=8, dx=FAKE)
    a.update(kw)
    assert lib.moe_permute_backward(a["g"], a["inv"], a["T"], a["k"], a["d"], a["dx"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(d=4), SHAPE),
    (dict(dy=None), NULLP), (dict(yp=None), NULLP), (dict(inv=None), NULLP), (dict(w=None), NULLP),
    (dict(dyp=None), NULLP), (dict(dw=None), NULLP),
    (dict(dy=FAKE + 8), ALIGN), (dict(yp=FAKE + 2), ALIGN), (dict(dyp=FAKE + 4), ALIGN), (dict(dw=FAKE + 2), ALIGN),
])
def test_unpermute_backward_validation(lib, kw, status):
    a = dict(dy=FAKE, yp=FAKE, inv=FAKE, w=FAKE, T=4, k=2, d=8, dyp=FAKE, dw=FAKE)
    a.update(kw)
    assert lib.moe_unpermute_backward(a["dy"], a["yp"], a["inv"], a["w"], a["T"], a["k"], a["d"], a["dyp"], a["dw"],
                                      None) == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour on a host without a GPU")
def test_backward_device_check_without_gpu(lib):
    assert dgrad(lib) == DEV and wgrad(lib) == DEV
    assert lib.moe_permute_backward(FAKE, FAKE, 4, 2, 8, FAKE, None) == DEV
    assert lib.moe_unpermute_backward(FAKE, FAKE, FAKE, FAKE, 4, 2, 8, FAKE, FAKE, None) == DEV


def test_binding_backward_rejects_bad_layout():
    w = torch.zeros((2, 16, 24), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_grouped_dgrad(torch.zeros((4, 24), dtype=torch.bfloat16), torch.zeros(3, dtype=torch.int32), w, "io")


def test_projection_and_swiglu_backward_validation(lib):
    f = lib.moe_grouped_projection
    assert f(FAKE, FAKE, FAKE, 3, 16, 16, 24, 2, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 0, 16, 12, 24, 2, FAKE, None) == SHAPE
    assert f(None, FAKE, FAKE, 0, 16, 16, 24, 2, FAKE, None) == NULLP
    assert f(FAKE, FAKE, FAKE, 1, 16, 16, 24, 2, FAKE + 8, None) == ALIGN
    g = lib.moe_swiglu_backward
    assert g(FAKE, FAKE, FAKE, 2, 16, 12, FAKE, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, 0, 16, 16, FAKE, None) == SHAPE
    assert g(FAKE, None, FAKE, 2, 16, 16, FAKE, None) == NULLP
    assert g(FAKE, FAKE, FAKE, 2, 16, 16, FAKE + 2, None) == ALIGN
    if not torch.cuda.is_available():
        assert f(FAKE, FAKE, FAKE, 0, 16, 16, 24, 2, FAKE, None) == DEV
        assert g(FAKE, FAKE, FAKE, 2, 16, 16, FAKE, None) == DEV
