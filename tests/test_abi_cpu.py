"""The C ABI without a GPU: libdobb.so loads, exports every entry point include/dobb.h declares, and
rejects bad arguments on the host before anything is enqueued.

Every call below is invalid in at least one argument, so validation returns before any launch; the
non-null "device pointers" are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from block_diagonal_eigenbasis_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: each call fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dobb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dobb_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    names = declared_functions()
    assert len(names) == 15
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert _abi.dobb_abi_version() == 2
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert _abi.status_string(st)
    assert "unknown" in _abi.status_string(42)


def _shape(m, n, nb):
    return _abi.Shape(m, n, nb)


@pytest.mark.parametrize("m,n,nb,status", [
    (0, 8, 4, _abi.DOBB_ERR_SHAPE), (4, 0, 4, _abi.DOBB_ERR_SHAPE), (4, 8, 0, _abi.DOBB_ERR_SHAPE),
    (4, 10, 4, _abi.DOBB_ERR_SHAPE), (4, 4096, 2048, _abi.DOBB_ERR_SHAPE)])
def test_step_shape_errors(m, n, nb, status):
    s = _shape(m, n, nb)
    hp = _abi.make_hparams(0.1, 0.0, 0.9, 0.2)
    st = _abi.lib().dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 1 << 30, None)
    assert st == status


def test_step_argument_errors():
    L = _abi.lib()
    s = _shape(64, 64, 16)
    hp = _abi.make_hparams(0.1, 0.0, 0.9, 0.2)
    assert L.dobb_step(None, FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 1 << 30, None) == -1
    assert L.dobb_step(ctypes.byref(s), None, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 1 << 30, None) == -1
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, None, None, None, FAKE, 1 << 30, None) == -1
    assert L.dobb_step(ctypes.byref(s), FAKE, 7, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 1 << 30, None) == -3
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 5, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 1 << 30, None) == -3
    bad = _abi.make_hparams(0.1, 0.0, 0.9, 0.2, norm=9)
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(bad), None, None, FAKE, 1 << 30, None) == -1
    # workspace: missing, too small, misaligned
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, None, 0, None) == -4
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE, 16, None) == -4
    assert L.dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None,
                       ctypes.c_void_p(0x10010), 1 << 30, None) == -4


def test_accumulate_argument_errors():
    L = _abi.lib()
    s = _shape(1, 64, 16)
    ok = dict(X=FAKE, dt=0, N=128, ldx=64, beta=0.5, A=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.dobb_accumulate_moment(ctypes.byref(s), a["X"], a["dt"], a["N"], a["ldx"], a["beta"], a["A"],
                                        None, 0, None)
    assert call(X=None) == -1
    assert call(A=None) == -1
    assert call(dt=3) == -3
    assert call(N=0) == -1
    assert call(ldx=32) == -2
    assert call(beta=1.0) == -1
    assert call(beta=-0.1) == -1
    assert call(beta=float("nan")) == -1
    # token split needs a workspace for this small shape: missing workspace is reported
    assert _abi.dobb_workspace_size(_abi.DOBB_OP_ACCUMULATE, [(1, 64, 16)], 4096) > 0
    assert call(N=4096) == -4


def test_refresh_argument_errors():
    L = _abi.lib()
    s = _shape(1, 64, 16)

    def call(A=FAKE, Q=FAKE, mode=0, iters=0, tol=0.0, ws=None, wsb=0, qdt=0):
        return L.dobb_refresh_basis(ctypes.byref(s), A, Q, qdt, None, mode, iters, 0, tol, None, ws, wsb, None)
    assert call(A=None) == -1
    assert call(Q=None) == -1
    assert call(mode=4) == -1
    assert call(mode=1, iters=0) == -1      # orthogonal iteration needs k >= 1
    assert call(mode=2, iters=0) == -1      # with either QR routine
    assert call(iters=-2) == -1
    assert call(tol=-1.0) == -1
    assert call(qdt=2) == -3                # basis dtype fp32 or bf16
    assert call() == -4                     # the refresh always needs a workspace


def test_workspace_sizes():
    ws = _abi.dobb_workspace_size
    assert ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, _abi.DOBB_NORM_SIGN) >= 768 * 768
    assert ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, _abi.DOBB_NORM_COL_L2) >= 4 * 768 * 768 + 4 * 768
    assert ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, 7) == 0
    r = ws(_abi.DOBB_OP_REFRESH, [(1, 768, 192)])
    assert r >= 4 * (192 * 192 * (4 + 8 + 4))
    assert ws(_abi.DOBB_OP_REFRESH, [(1, 770, 192)]) == 0         # n % nb != 0
    assert ws(_abi.DOBB_OP_ACCUMULATE, [(1, 768, 192)], 0) == 0   # N < 1
    # a group larger than one launch chunk (48 matrices) reuses the chunk's workspace
    big = ws(_abi.DOBB_OP_STEP, [(64, 64, 16)] * 60, 0, 0)
    assert big == ws(_abi.DOBB_OP_STEP, [(64, 64, 16)] * 48, 0, 0)
    assert big > ws(_abi.DOBB_OP_STEP, [(64, 64, 16)] * 16, 0, 0)
    # a bf16 basis adds an fp32 copy of every basis of a launch chunk
    bf = _abi.DOBB_WS_BF16_BASIS
    assert ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, bf) >= ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, 0) + 4 * 768 * 192
    assert ws(_abi.DOBB_OP_REFRESH, [(1, 768, 192)] * 3, 0, bf) >= ws(_abi.DOBB_OP_REFRESH, [(1, 768, 192)] * 3) + 3 * 4 * 768 * 192
    assert ws(_abi.DOBB_OP_STEP, [(768, 768, 192)], 0, bf | 7) == 0


def test_grouped_rejects_mixed_norms():
    L = _abi.lib()
    shapes = (_abi.Shape * 2)(_shape(64, 64, 16), _shape(64, 64, 16))
    hps = (_abi.HParams * 2)(_abi.make_hparams(0.1, 0, 0.9, 0.2), _abi.make_hparams(0.1, 0, 0.9, 0.2, norm=2))
    P = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    st = L.dobb_step_grouped(2, shapes, P, 0, P, 0, P, P, 0, hps, None, None, FAKE, 1 << 30, None)
    assert st == -1


def test_step_rejects_bad_basis_dtype():
    s = _shape(64, 64, 16)
    hp = _abi.make_hparams(0.1, 0.0, 0.9, 0.2)
    st = _abi.lib().dobb_step(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 3, ctypes.byref(hp), None, None, FAKE,
                              1 << 30, None)
    assert st == _abi.DOBB_ERR_DTYPE


def test_grouped_binding_rejects_mixed_dtypes():
    """The C ABI takes one dtype per argument of a grouped call; a list mixing fp32 and bf16 tensors
    is refused before any pointer is passed (an element-size mismatch would run past a buffer)."""
    import torch
    xs = [torch.zeros(4, 8), torch.zeros(4, 8, dtype=torch.bfloat16)]
    with pytest.raises(TypeError, match="same dtype"):
        _abi._common_dtype(xs, "X")
    assert _abi._common_dtype([torch.zeros(2), torch.zeros(3)], "X") == _abi.DOBB_F32


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        _abi.dobb_step(torch.zeros(4, 4), torch.zeros(4, 4), torch.zeros(4, 4), torch.zeros(1, 4, 4), 4,
                       _abi.make_hparams(0.1, 0, 0.9, 0.2))


def test_step_noalloc_refuses_before_any_launch():
    """The allocation-free step checks its arguments and that the shape's workspace fits the static
    scratch before it touches a device: a column-l2 step of an 11008 x 4096 weight needs 4 bytes per
    entry, more than DOBB_NOALLOC_SCRATCH_BYTES."""
    L = _abi.lib()
    big = _shape(11008, 4096, 128)
    l2 = _abi.make_hparams(0.1, 0.0, 0.9, 0.2, norm=_abi.DOBB_NORM_COL_L2)
    assert _abi.dobb_workspace_size(_abi.DOBB_OP_STEP, [(11008, 4096, 128)], 0, 2) > _abi.DOBB_NOALLOC_SCRATCH_BYTES
    assert L.dobb_step_noalloc(ctypes.byref(big), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(l2), None, None,
                               None) == _abi.DOBB_ERR_WORKSPACE
    hp = _abi.make_hparams(0.1, 0.0, 0.9, 0.2)
    s = _shape(64, 64, 16)
    assert L.dobb_step_noalloc(ctypes.byref(s), None, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None,
                               None) == -1
    assert L.dobb_step_noalloc(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 5, ctypes.byref(hp), None, None,
                               None) == -3
    assert L.dobb_step_noalloc(ctypes.byref(_shape(64, 65, 16)), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp),
                               None, None, None) == -2
    # every single weight of the GPT-2 XL and 7B-style sets fits with sign normalisation
    for shp in [(4800, 1600, 100), (6400, 1600, 100), (1600, 6400, 400), (11008, 4096, 128), (4096, 11008, 128)]:
        assert 0 < _abi.dobb_workspace_size(_abi.DOBB_OP_STEP, [shp], 0, 0) <= _abi.DOBB_NOALLOC_SCRATCH_BYTES


def test_step_g_shape_errors_and_workspace():
    """Dobb-G's blocks are rows: m % nb == 0 is required and n is free."""
    L = _abi.lib()
    hp = _abi.make_hparams(0.1, 0.0, 0.9, 0.2)
    for (m, n, nb), want in [((10, 8, 4), -2), ((0, 8, 4), -2), ((8, 0, 4), -2), ((8, 6, 0), -2)]:
        s = _shape(m, n, nb)
        st = L.dobb_step_g(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, FAKE,
                           1 << 30, None)
        assert st == want, (m, n, nb)
    s = _shape(8, 6, 4)   # n % nb != 0 is fine for row blocks: fails only on the missing workspace
    assert L.dobb_step_g(ctypes.byref(s), FAKE, 0, FAKE, 0, FAKE, FAKE, 0, ctypes.byref(hp), None, None, None, 0,
                         None) == -4
    ws = _abi.dobb_workspace_size
    assert ws(_abi.DOBB_OP_STEP_G, [(768, 770, 192)], 0, 0) >= 768 * 770
    assert ws(_abi.DOBB_OP_STEP_G, [(768, 770, 192)], 0, 2) >= 4 * 768 * 770 + 4 * 768
    assert ws(_abi.DOBB_OP_STEP_G, [(770, 768, 192)], 0, 0) == 0
