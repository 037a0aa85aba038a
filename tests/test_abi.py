"""The C ABI on the host: libdora.so loads, exports every declared symbol, and
rejects bad arguments before touching the GPU.  No compute calls here."""
import ctypes
import os
import re

import pytest

from parameter_efficient_fine_dora_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dora.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libdora.so not built")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"DORA_API\s+[\w\s\*]+?\b(dora_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared_symbols())
    assert {"dora_norm", "dora_forward", "dora_backward", "dora_merge", "dora_vera_scale",
            "dora_vera_grads", "dora_workspace_bytes",
            "dora_strerror", "dora_timing_enable", "dora_timing_collect", "dora_probe_mfma",
            "dora_probe_mfma_flops", "dora_probe_stream"} <= names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_shape_struct_matches_header():
    assert ctypes.sizeof(_lib.DoraShape) == 48
    assert _lib.DoraShape.s.offset == 36 and _lib.DoraShape.flags.offset == 40


def test_strerror_texts():
    for code in _lib.ERR:
        assert _lib.strerror(code)
    assert "unknown" in _lib.strerror(-99)


FAKE = 0x10000  # 16-byte aligned host address; validation never dereferences it


def _norm(sh, W0=FAKE, A=FAKE, B=FAKE, out=FAKE, ws=FAKE, nb=1 << 40):
    return _lib.lib().dora_norm(ctypes.byref(sh) if sh is not None else None, W0, A, B, out, ws,
                                nb, None)


@pytest.mark.parametrize("dims,code", [
    ((0, 64, 8, 4), "DORA_ERR_SHAPE"), ((64, 0, 8, 4), "DORA_ERR_SHAPE"),
    ((64, 64, -8, 4), "DORA_ERR_SHAPE"), ((64, 64, 8, -1), "DORA_ERR_SHAPE"),
    ((60, 64, 8, 4), "DORA_ERR_SHAPE"), ((64, 66, 8, 4), "DORA_ERR_SHAPE"),
    ((64, 64, 12, 4), "DORA_ERR_SHAPE"), ((1 << 31, 8, 8, 4), "DORA_ERR_SHAPE"),
    ((1 << 22, 64, 8, 4), "DORA_ERR_SHAPE"), ((64, 1 << 22, 8, 4), "DORA_ERR_SHAPE"),
    ((64, 64, 1 << 22, 8), "DORA_ERR_SHAPE"), ((64, 64, 8, 1 << 31), "DORA_ERR_SHAPE"),
])
def test_bad_shapes_rejected(dims, code):
    sh = _lib.shape(*dims, _lib.BF16, 2.0)
    assert _norm(sh) == _lib.ERR_CODE[code]
    assert _lib.workspace_bytes(sh, _lib.OP_NORM) == 0


def test_validation_codes():
    ok = _lib.shape(64, 64, 8, 4, _lib.BF16, 2.0)
    assert _norm(None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert _norm(_lib.shape(64, 64, 8, 4, 7, 2.0)) == _lib.ERR_CODE["DORA_ERR_DTYPE"]
    assert _norm(_lib.shape(64, 64, 8, 4, _lib.BF16, float("nan"))) == _lib.ERR_CODE["DORA_ERR_FLAGS"]
    assert _norm(_lib.shape(64, 64, 8, 4, _lib.BF16, 2.0, 1 << 7)) == _lib.ERR_CODE["DORA_ERR_FLAGS"]
    bad = _lib.shape(64, 64, 8, 4, _lib.BF16, 2.0)
    bad.reserved = 1
    assert _norm(bad) == _lib.ERR_CODE["DORA_ERR_FLAGS"]
    assert _norm(ok, W0=None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert _norm(ok, A=None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert _norm(ok, out=None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert _norm(ok, ws=None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert _norm(ok, W0=FAKE + 2) == _lib.ERR_CODE["DORA_ERR_ALIGN"]
    assert _norm(ok, ws=FAKE + 8) == _lib.ERR_CODE["DORA_ERR_ALIGN"]
    need = _lib.workspace_bytes(ok, _lib.OP_NORM)
    assert _norm(ok, nb=need - 1) == _lib.ERR_CODE["DORA_ERR_WORKSPACE"]
    # rank 0: A and B may be NULL, W0 may not (only failing paths are exercised here:
    # a call that passes validation would enqueue kernels)
    r0 = _lib.shape(64, 64, 0, 4, _lib.BF16, 2.0)
    assert _norm(r0, W0=None, A=None, B=None) == _lib.ERR_CODE["DORA_ERR_NULL"]


def test_merge_validation():
    """dora_merge: every tensor but norm is required; its workspace comes from DORA_OP_MERGE."""
    L = _lib.lib()
    sh = _lib.shape(64, 64, 8, 0, _lib.BF16, 2.0)
    need = _lib.workspace_bytes(sh, _lib.OP_MERGE)
    assert need > 0

    def merge(W0=FAKE, A=FAKE, B=FAKE, m=FAKE, norm=FAKE, out=FAKE, ws=FAKE, nb=need):
        return L.dora_merge(ctypes.byref(sh), W0, A, B, m, norm, out, ws, nb, None)

    for kw in ("W0", "A", "B", "m", "out", "ws"):
        assert merge(**{kw: None}) == _lib.ERR_CODE["DORA_ERR_NULL"], kw
    assert merge(out=FAKE + 4) == _lib.ERR_CODE["DORA_ERR_ALIGN"]
    assert merge(norm=FAKE + 4) == _lib.ERR_CODE["DORA_ERR_ALIGN"]
    assert merge(nb=need - 1) == _lib.ERR_CODE["DORA_ERR_WORKSPACE"]
    bad = _lib.shape(64, 60, 8, 0, _lib.BF16, 2.0)
    assert L.dora_merge(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, need,
                        None) == _lib.ERR_CODE["DORA_ERR_SHAPE"]
    # merge workspace: the norm's, plus the norms themselves; never d_out x d_in
    big = _lib.shape(8192, 8192, 384, 0, _lib.BF16, 2.0)
    assert (_lib.workspace_bytes(big, _lib.OP_MERGE) - _lib.workspace_bytes(big, _lib.OP_NORM)
            <= 8192 * 4 + 1024)


def test_vera_validation():
    """dora_vera_scale / dora_vera_grads: required tensors, optional outputs, workspace."""
    L = _lib.lib()
    sh = _lib.shape(64, 64, 8, 0, _lib.BF16, 1.0)
    assert L.dora_vera_scale(ctypes.byref(sh), FAKE, FAKE, FAKE, None, None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert L.dora_vera_scale(ctypes.byref(sh), FAKE, None, FAKE, FAKE, None) == _lib.ERR_CODE["DORA_ERR_NULL"]
    assert L.dora_vera_scale(ctypes.byref(sh), FAKE, FAKE, FAKE + 2, FAKE, None) == _lib.ERR_CODE["DORA_ERR_ALIGN"]
    need = _lib.workspace_bytes(sh, _lib.OP_VERA_GRADS)
    assert 0 < need <= 64 * 8 * 4 + 1024

    def grads(gBe=FAKE, Bsh=FAKE, b=FAKE, d=FAKE, gb=FAKE, gd=FAKE, ws=FAKE, nb=need):
        return L.dora_vera_grads(ctypes.byref(sh), gBe, Bsh, b, d, gb, gd, ws, nb, None)

    for kw in ("gBe", "Bsh", "b", "d", "ws"):
        assert grads(**{kw: None}) == _lib.ERR_CODE["DORA_ERR_NULL"], kw
    assert grads(nb=need - 1) == _lib.ERR_CODE["DORA_ERR_WORKSPACE"]
    assert grads(gd=FAKE + 4) == _lib.ERR_CODE["DORA_ERR_ALIGN"]


def test_exact_flag_needs_its_own_workspace():
    """The undetached gradient needs more workspace; the detached size is rejected for it."""
    det = _lib.shape(64, 64, 8, 4, _lib.BF16, 2.0)
    ex = _lib.shape(64, 64, 8, 4, _lib.BF16, 2.0, _lib.FLAG_EXACT_NORM_GRAD)
    nb_det = _lib.workspace_bytes(det, _lib.OP_BACKWARD)
    nb_ex = _lib.workspace_bytes(ex, _lib.OP_BACKWARD)
    assert nb_ex > nb_det
    rc = _lib.lib().dora_backward(ctypes.byref(ex), *([FAKE] * 13), FAKE, nb_det, None)
    assert rc == _lib.ERR_CODE["DORA_ERR_WORKSPACE"]


def test_workspace_never_scales_with_d_out_times_d_in():
    """Zero transient d_out x d_in buffers: the workspace is O(d_out r + r^2 + T r) (+ [T, d_out])."""
    for d_out, d_in, r, T in [(8192, 8192, 384, 4096), (27648, 5120, 256, 8192), (2048, 6144, 64, 2048)]:
        sh = _lib.shape(d_out, d_in, r, T, _lib.BF16, 2.0)
        dense = d_out * d_in * 2
        norm_ws = _lib.workspace_bytes(sh, _lib.OP_NORM)
        fwd_ws = _lib.workspace_bytes(sh, _lib.OP_FORWARD)
        bwd_ws = _lib.workspace_bytes(sh, _lib.OP_BACKWARD)
        assert norm_ws < dense / 3
        # at most 16 split-K partial Gram matrices and 16 partial projections P [d_out, r]
        assert norm_ws <= 16 * r * r * 4 + r * r * 4 + 16 * d_out * r * 4 + 4096
        # forward adds xs [T, r] and one split-K region: at most 16 [T, r] float32 blocks
        # (the down-projection), or, when the fused GEMM's 128 x 128 tiles cannot fill
        # the chip, its float32 partials: split * tiles <= 384 + tiles / 2 with
        # tiles = T d_out / 128^2, i.e. at most (384 * 128^2 + T d_out / 2) floats
        fused_k = 4 * (384 * 128 * 128 + T * d_out // 2)
        assert fwd_ws - norm_ws <= T * r * 2 + max(16 * T * r * 4, fused_k) + 4096
        split_k = 16 * max(T * r, d_out * r, r * d_in) * 4
        assert bwd_ws <= T * d_out * 2 + 2 * T * r * 2 + ((T + 63) // 64) * d_out * 4 + split_k + 4096
        sep = _lib.shape(d_out, d_in, r, T, _lib.BF16, 2.0, _lib.FLAG_SEPARATE_COMPOSE)
        assert _lib.workspace_bytes(sep, _lib.OP_FORWARD) - fwd_ws >= T * d_out * 2


def test_timing_collect_empty_on_host():
    L = _lib.lib()
    assert L.dora_timing_enable(0) == 0
    buf = ctypes.create_string_buffer(64)
    assert L.dora_timing_collect(buf, 64) == 0
    assert buf.value == b"{}"


def test_library_has_no_device_allocation_calls():
    """The library allocates nothing: no hipMalloc/hipFree in its sources."""
    csrc = os.path.join(ROOT, "parameter_efficient_fine_dora_amd", "csrc")
    for fn in os.listdir(csrc):
        text = open(os.path.join(csrc, fn)).read()
        for bad in ("hipMalloc", "hipFree", "hipHostMalloc", "hipExtMalloc"):
            assert bad not in text, (fn, bad)


def test_mfma_probe_validation_and_flop_count():
    L = _lib.lib()
    shape_err = [k for k, v in _lib.ERR.items() if v == "DORA_ERR_SHAPE"][0]
    assert L.dora_probe_mfma(0, 1, None, None) == shape_err        # no launch
    assert L.dora_probe_mfma(1, 0, None, None) == shape_err
    # blocks * 4 waves * iters * 4 chains * (2 * 32 * 32 * 16) flops
    assert L.dora_probe_mfma_flops(10, 3) == 3 * 4 * 10 * 4 * 32768


def test_stream_probe_validation():
    L = _lib.lib()
    E = _lib.ERR_CODE
    assert L.dora_probe_stream(None, None, None, 16, None) == E["DORA_ERR_NULL"]
    assert L.dora_probe_stream(16, 32, 48, 8, None) == E["DORA_ERR_SHAPE"]      # not a multiple of 16
    assert L.dora_probe_stream(16, 32, 52, 16, None) == E["DORA_ERR_ALIGN"]     # c misaligned

