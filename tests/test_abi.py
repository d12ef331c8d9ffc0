"""CPU-only checks of the C ABI: libprn loads, exports every symbol of
include/prn.h, and rejects bad arguments on the host before launching
anything (no GPU needed, no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import nonlinear_rnn_amd as prn
from nonlinear_rnn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libprn.so not built")


def header_symbols():
    src = open(os.path.join(ROOT, "include", "prn.h")).read()
    return sorted(set(re.findall(r"\b(prn_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree_and_library_exports_all():
    syms = header_symbols()
    assert syms == sorted(B.EXPORTS)
    L = B.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert B.prn_version() >= 100


def test_struct_layout_matches_header(tmp_path):
    """Field offsets of the ctypes mirror equal what a C compiler makes of prn.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = [f[0] for f in B.prn_params._fields_]
    src = tmp_path / "off.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "prn.h"\nint main(void){\n'
                   + "".join(f'printf("%zu\\n", offsetof(prn_params, {n}));\n' for n in names)
                   + 'printf("%zu\\n", sizeof(prn_params));return 0;}\n')
    exe = tmp_path / "off"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [getattr(B.prn_params, n).offset for n in names] + [ctypes.sizeof(B.prn_params)]
    assert got == want


def _params(**kw):
    p = B.prn_params()
    p.cell, p.dtype, p.B, p.T, p.d_in, p.d_h, p.n_seqs = 0, 0, 2, 100, 8, 16, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = 1 << 20   # an aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,K,status", [
    (dict(cell=7), 3, B.PRN_ERR_INVALID_ARG),
    (dict(dtype=5), 3, B.PRN_ERR_INVALID_ARG),
    (dict(B=0), 3, B.PRN_ERR_INVALID_ARG),
    (dict(d_h=0), 3, B.PRN_ERR_INVALID_ARG),
    (dict(T=-1), 3, B.PRN_ERR_INVALID_ARG),
    (dict(), 0, B.PRN_ERR_INVALID_ARG),
    (dict(n_seqs=3), 3, B.PRN_ERR_INVALID_ARG),                       # B=2 with a pack
    (dict(a=None), 3, B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), 3, B.PRN_ERR_WORKSPACE),                          # no workspace given
    (dict(a=FAKE, workspace=FAKE, workspace_bytes=16), 3, B.PRN_ERR_WORKSPACE),
    (dict(a=FAKE + 2), 3, B.PRN_ERR_INVALID_ARG),                    # misaligned
    (dict(a=FAKE, picard_iters=-1), 3, B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE, picard_iters=2), 3, B.PRN_ERR_WORKSPACE),          # any P >= 0 passes validation
    (dict(a=FAKE, error_out=FAKE + 2), 3, B.PRN_ERR_INVALID_ARG),    # misaligned error word
])
def test_newton_forward_rejects_bad_arguments_before_launch(kw, K, status):
    p = _params(**kw)
    st = B.lib().prn_newton_forward(FAKE, ctypes.byref(p), None, K, None, FAKE, None)
    assert st == status, B.prn_last_error()
    assert B.prn_last_error()


def test_newton_forward_rejects_pack_inconsistency():
    p = _params(B=1, a=FAKE)
    assert B.lib().prn_newton_forward(FAKE, ctypes.byref(p), None, 3, FAKE, FAKE, None) == B.PRN_ERR_INVALID_ARG
    p = _params(B=1, n_seqs=4, a=FAKE)
    assert B.lib().prn_newton_forward(FAKE, ctypes.byref(p), None, 3, None, FAKE, None) == B.PRN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,args,status", [
    (dict(a=FAKE), dict(x=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(W=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(K=0), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE, d_in=0), dict(), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE, d_in=6), dict(), B.PRN_ERR_UNSUPPORTED),                 # fp32 needs d_in % 4 == 0
    (dict(a=FAKE, dtype=1, d_in=4), dict(), B.PRN_ERR_UNSUPPORTED),        # bf16 needs d_in % 8 == 0
    (dict(a=FAKE, picard_iters=1), dict(), B.PRN_ERR_UNSUPPORTED),
    (dict(a=FAKE), dict(x=FAKE + 8), B.PRN_ERR_INVALID_ARG),                 # 16-byte alignment
    (dict(a=FAKE), dict(xproj_out=FAKE + 4), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(), B.PRN_ERR_WORKSPACE),                             # no workspace given
    (dict(a=FAKE, workspace=FAKE, workspace_bytes=16), dict(), B.PRN_ERR_WORKSPACE),
    (dict(a=None), dict(), B.PRN_ERR_INVALID_ARG),
])
def test_fused_forward_rejects_bad_arguments_before_launch(kw, args, status):
    p = _params(**kw)
    a = dict(x=FAKE, W=FAKE, K=3, xproj_out=None)
    a.update(args)
    st = B.lib().prn_newton_forward_fused(a["x"], a["W"], None, ctypes.byref(p), None, a["K"], None, FAKE, None,
                                          a["xproj_out"])
    assert st == status, B.prn_last_error()
    assert B.prn_last_error()


def test_workspace_bytes_cover_the_fused_forward():
    """prn_workspace_bytes sizes the workspace of both forwards (the fused GRU
    with many chains runs shorter chunks, hence more chunk records).  Only the
    rejection path runs: a too-small workspace reports the size it needs."""
    for cell, Bn in (("gru", 128), ("lstm", 2), ("gru", 2)):
        p = _params(cell=B.CELLS[cell], B=Bn, T=4096, d_h=256, a=FAKE, workspace=FAKE, workspace_bytes=16)
        n = B.lib().prn_workspace_bytes(ctypes.byref(p), 3)
        st = B.lib().prn_newton_forward_fused(FAKE, FAKE, None, ctypes.byref(p), None, 3, None, FAKE, None, None)
        assert st == B.PRN_ERR_WORKSPACE
        need = int(re.search(r"; (\d+) bytes needed", B.prn_last_error()).group(1))
        st = B.lib().prn_newton_forward(FAKE, ctypes.byref(p), None, 3, None, FAKE, None)
        assert st == B.PRN_ERR_WORKSPACE
        need_unfused = int(re.search(r"; (\d+) bytes needed", B.prn_last_error()).group(1))
        assert n >= need and n >= need_unfused and n == max(need, need_unfused)


def test_grids_too_large_for_one_launch_are_rejected_on_the_host():
    """More workgroups than one launch takes (2^31 - 1) is PRN_ERR_UNSUPPORTED,
    checked before anything is launched."""
    p = _params(T=1 << 36, d_in=8, d_h=1024)   # 5.4e8 row tiles x 24 column tiles
    assert B.lib().prn_input_proj(FAKE, FAKE, None, ctypes.byref(p), FAKE) == B.PRN_ERR_UNSUPPORTED
    assert "too large" in B.prn_last_error()
    p = _params(B=1, T=1 << 38, d_h=64, a=FAKE, workspace=FAKE, workspace_bytes=1 << 62)   # 2^32 chunks
    assert B.lib().prn_newton_forward(FAKE, ctypes.byref(p), None, 2, None, FAKE, None) == B.PRN_ERR_UNSUPPORTED
    assert "too many chunks" in B.prn_last_error()


def test_input_proj_rejects_unsupported_shapes():
    p = _params(d_in=6)   # fp32 needs d_in % 4 == 0
    assert B.lib().prn_input_proj(FAKE, FAKE, None, ctypes.byref(p), FAKE) == B.PRN_ERR_UNSUPPORTED
    p = _params(d_in=8)
    assert B.lib().prn_input_proj(None, FAKE, None, ctypes.byref(p), FAKE) == B.PRN_ERR_INVALID_ARG


def test_workspace_bytes_grows_with_K_and_is_zero_on_bad_params():
    w1 = B.prn_workspace_bytes("lstm", torch.float32, 2, 1000, 64, 1)
    w2 = B.prn_workspace_bytes("lstm", torch.float32, 2, 1000, 64, 2)
    w3 = B.prn_workspace_bytes("lstm", torch.float32, 2, 1000, 64, 3)
    assert 0 < w1 < w2 < w3
    assert w3 % 256 == 0
    p = _params(d_h=0)
    assert B.lib().prn_workspace_bytes(ctypes.byref(p), 3) == 0


@pytest.mark.parametrize("cu,N,ok", [
    ([0, 5, 5, 9], 9, True),
    ([0, 9], 9, True),
    ([1, 5, 9], 9, False),
    ([0, 6, 5, 9], 9, False),
    ([0, 5, 8], 9, False),
    ([0], 0, False),
])
def test_validate_cu_seqlens(cu, N, ok):
    if ok:
        B.prn_validate_cu_seqlens(np.array(cu), N)
    else:
        with pytest.raises(B.PrnError):
            B.prn_validate_cu_seqlens(np.array(cu), N)


def test_k_table_and_residual_gate_on_host():
    assert prn.resolve_k(100, {64: 2, 1024: 3}) == 3
    assert prn.resolve_k(10 ** 6, {64: 2, 1024: 3}) == 3
    prn.gate_residual([0.9, 1e-6], torch.float32)
    with pytest.warns(RuntimeWarning, match="newton_residual_high"):
        prn.gate_residual([0.9, 0.5], torch.float32)
    for bad in (1.5, float("inf"), float("nan")):
        with pytest.raises(prn.NewtonDivergenceError):
            prn.gate_residual([0.9, bad], torch.float32)
    prn.gate_residual([0.9, 1.0], torch.float32, residual_warn=2.0)   # exactly 1.0 passes (">" gate)


@pytest.mark.parametrize("kw,args,status", [
    (dict(cell=7), {}, B.PRN_ERR_INVALID_ARG),
    (dict(a=None), {}, B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(da=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(states=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(dH=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(dx=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=FAKE), dict(cu=FAKE), B.PRN_ERR_INVALID_ARG),                  # rectangular with offsets
    (dict(a=FAKE), dict(dsl=FAKE + 2), B.PRN_ERR_INVALID_ARG),             # misaligned
    (dict(a=FAKE), {}, B.PRN_ERR_WORKSPACE),                              # no workspace
    (dict(a=FAKE, workspace=FAKE, workspace_bytes=64), {}, B.PRN_ERR_WORKSPACE),
    (dict(a=FAKE, workspace=FAKE + 64, workspace_bytes=1 << 40), {}, B.PRN_ERR_WORKSPACE),   # misaligned
])
def test_newton_backward_rejects_bad_arguments_before_launch(kw, args, status):
    p = _params(**kw)
    a = dict(xproj=FAKE, h0=None, cu=None, states=FAKE, dH=FAKE, dsl=None, dx=FAKE, da=FAKE, dh0=None)
    a.update(args)
    st = B.lib().prn_newton_backward(a["xproj"], ctypes.byref(p), a["h0"], a["cu"], a["states"], a["dH"],
                                     a["dsl"], a["dx"], a["da"], a["dh0"])
    assert st == status, B.prn_last_error()
    assert B.prn_last_error()


def test_backward_workspace_bytes():
    w = B.prn_backward_workspace_bytes("lstm", torch.float32, 2, 1000, 64)
    assert w > 0 and w % 256 == 0
    assert B.prn_backward_workspace_bytes("gru", torch.float32, 2, 1000, 64) < w
    p = _params(d_h=0)
    assert B.lib().prn_backward_workspace_bytes(ctypes.byref(p)) == 0


def test_committed_kstar_table_is_well_formed():
    """The measured K*(T) tables: both cells, positive K, monotone in T, and
    resolvable for any T (no GPU needed to read them)."""
    from nonlinear_rnn_amd import kstar as gk
    for cell in ("gru", "lstm"):
        tab = gk.load_table(cell)
        ks = [tab[T] for T in sorted(tab)]
        assert ks and all(k >= 1 for k in ks) and ks == sorted(ks)
        assert prn.resolve_k(1, tab) == ks[0] and prn.resolve_k(10 ** 7, tab) == ks[-1]


@pytest.mark.parametrize("kw,args,status", [
    (dict(T=100, a=FAKE), {}, B.PRN_ERR_INVALID_ARG),                     # a decode step has T = 1
    (dict(T=1, a=FAKE, n_seqs=2, B=1), {}, B.PRN_ERR_INVALID_ARG),        # no ragged packs
    (dict(T=1, a=None), {}, B.PRN_ERR_INVALID_ARG),
    (dict(T=1, a=FAKE), dict(x=None), B.PRN_ERR_INVALID_ARG),
    (dict(T=1, a=FAKE), dict(so=None), B.PRN_ERR_INVALID_ARG),
    (dict(T=1, a=FAKE), dict(x=FAKE + 2), B.PRN_ERR_INVALID_ARG),         # fp32 x not 4-byte aligned
    (dict(T=1, a=FAKE, dtype=1), dict(W=FAKE + 1), B.PRN_ERR_INVALID_ARG),  # bf16 W not 2-byte aligned
    (dict(T=1, a=FAKE), dict(si=FAKE + 4096, so=FAKE + 4096), B.PRN_ERR_INVALID_ARG),   # aliasing carry
    (dict(T=1, a=FAKE, d_in=0), {}, B.PRN_ERR_INVALID_ARG),
])
def test_decode_step_rejects_bad_arguments_before_launch(kw, args, status):
    p = _params(**kw)
    a = dict(x=FAKE, W=FAKE, bias=None, si=None, so=FAKE + 8192, h=None)
    a.update(args)
    st = B.lib().prn_decode_step(a["x"], a["W"], a["bias"], ctypes.byref(p), a["si"], a["so"], a["h"])
    assert st == status, B.prn_last_error()
    assert B.prn_last_error()


@pytest.mark.parametrize("kw,args,status", [
    (dict(cell=1, a=None), {}, B.PRN_ERR_UNSUPPORTED),                   # LSTM head-mix is not built
    (dict(dtype=1, a=None), {}, B.PRN_ERR_WORKSPACE),                    # bf16 head-mix: checked up to the workspace
    (dict(dtype=1, a=None, d_h=32), dict(xproj=FAKE + 4), B.PRN_ERR_INVALID_ARG),   # bf16 rows need 8-byte alignment
    (dict(B=1, n_seqs=2, a=None), {}, B.PRN_ERR_UNSUPPORTED),            # no ragged pack for head-mix
    (dict(a=None), dict(d_head=8), B.PRN_ERR_UNSUPPORTED),
    (dict(a=None, d_h=24), {}, B.PRN_ERR_INVALID_ARG),                   # d_h not a multiple of d_head
    (dict(a=None, d_h=32), dict(A=None), B.PRN_ERR_INVALID_ARG),
    (dict(a=None, d_h=32), dict(K=0), B.PRN_ERR_INVALID_ARG),
    (dict(a=None, d_h=32), dict(A=FAKE + 2), B.PRN_ERR_INVALID_ARG),
    (dict(a=None, d_h=32), {}, B.PRN_ERR_WORKSPACE),                     # no workspace
    (dict(a=None, d_h=32, states_out=FAKE), {}, B.PRN_ERR_UNSUPPORTED),
])
def test_head_newton_forward_rejects_bad_arguments_before_launch(kw, args, status):
    p = _params(**kw)
    a = dict(xproj=FAKE, A=FAKE, d_head=16, h0=None, K=3, H=FAKE, res=None)
    a.update(args)
    st = B.lib().prn_head_newton_forward(a["xproj"], ctypes.byref(p), a["A"], a["d_head"], a["h0"], a["K"], a["H"],
                                         a["res"])
    assert st == status, B.prn_last_error()
    assert B.prn_last_error()


def test_head_workspace_bytes():
    w3 = B.prn_head_workspace_bytes(2, 1000, 64, 3)
    w1 = B.prn_head_workspace_bytes(2, 1000, 64, 1)
    assert w3 > w1 > 0 and w3 % 256 == 0
    # bf16 iterates take half the bytes of fp32 ones; the rest is fp32 either way
    w3b = B.prn_head_workspace_bytes(2, 1000, 64, 3, dtype=torch.bfloat16)
    assert w1 < w3b < w3 and w3b % 256 == 0
    p = _params(d_h=64, cell=1)   # the LSTM has no head-mix: 0 bytes and a message
    assert B.lib().prn_head_workspace_bytes(ctypes.byref(p), 16, 3) == 0 and B.prn_last_error()


def test_bench_names_the_projection_tiles_the_library_uses():
    """bench.py reports which projection tile shape ran; its rule must be the
    library's (256 x 256 tiles from kLargeTiles of them on)."""
    import bench
    from workloads import Workload
    src = open(os.path.join(ROOT, "nonlinear_rnn_amd", "csrc", "proj.hip")).read()
    large = int(re.search(r"constexpr int64_t kLargeTiles = (\d+);", src).group(1))
    # rows x columns of 256 x 256 tiles: just below and at the threshold
    # G d_h = 768: 3 column tiles; rows of 256 tokens
    below = Workload("t", "gru", 1, 256 * (large // 3 - 1), 8, 256, "f32", 3)
    at = Workload("t", "gru", 1, 256 * (large // 3), 8, 256, "f32", 3)
    assert bench.proj_tiles(below) == "128x128"
    assert bench.proj_tiles(at) == "256x256"


def test_unsupported_status_raises_type_error():
    """A valid request pinned to a path the library does not implement raises
    TypeError (shapes/layout page: an unsupported pinned path raises, with no
    silent remap); other failures stay plain PrnError (RuntimeError)."""
    with pytest.raises(TypeError) as e:
        B._check(B.PRN_ERR_UNSUPPORTED)
    assert isinstance(e.value, B.PrnError) and e.value.status == B.PRN_ERR_UNSUPPORTED
    with pytest.raises(B.PrnError) as e:
        B._check(B.PRN_ERR_INVALID_ARG)
    assert not isinstance(e.value, TypeError)
    p = _params(a=FAKE, picard_iters=1, d_in=16)
    st = B.lib().prn_newton_forward_fused(FAKE, FAKE, None, ctypes.byref(p), None, 3, None, FAKE, None, None)
    with pytest.raises(TypeError, match="Picard"):
        B._check(st)


def test_noalloc_forward_rejects_calls_beyond_its_scratch_before_any_device_call():
    """The allocation-free forward checks its scratch need on the host: a
    call larger than the static array is PRN_ERR_WORKSPACE with a message that
    names both sizes, before any HIP call (this runs without a GPU)."""
    p = _params(cell=B.CELLS["lstm"], B=2, T=131072, d_h=256, a=FAKE)   # the long LSTM: ~67 MB of records
    st = B.lib().prn_newton_forward_noalloc(FAKE, ctypes.byref(p), None, 2, None, FAKE, None)
    assert st == B.PRN_ERR_WORKSPACE
    msg = B.prn_last_error()
    assert str(B.NOALLOC_SCRATCH_BYTES) in msg and "needs" in msg
    need = int(re.search(r"needs (\d+) bytes", msg).group(1))
    assert need == B.lib().prn_workspace_bytes(ctypes.byref(p), 2)
    # argument checks come first, as for prn_newton_forward
    p = _params(a=None)
    assert B.lib().prn_newton_forward_noalloc(FAKE, ctypes.byref(p), None, 3, None, FAKE, None) == \
        B.PRN_ERR_INVALID_ARG
