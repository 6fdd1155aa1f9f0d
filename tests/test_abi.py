"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before enqueueing anything.

Every call here fails validation (or is host-only), so no HIP work is issued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

L = pytest.importorskip("mamba_ssd_chunked_amd._lib")

# fake, 16-byte aligned "device" addresses: validation rejects the call before use
A16 = 0x10000
MIS = 0x10004


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L.LIB, n), n
    assert set(names) == set(L.EXPORTED)
    # and the library exports no other C (unmangled) function
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB._name], capture_output=True, text=True).stdout
    c_syms = {ln.split()[-1] for ln in out.splitlines()
              if len(ln.split()) == 3 and ln.split()[1] == "T" and not ln.split()[-1].startswith("_")}
    assert c_syms == set(names), c_syms ^ set(names)


def test_status_strings():
    for rc in range(10):
        assert L.status_string(rc)
    assert L.status_string(99) == "unknown status"


def shape(**kw):
    base = dict(batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, ngroups=1, chunk=64, dtype="fp16")
    base.update(kw)
    return L.make_shape(**base)


_UNSET = object()


def fwd(sh, path=L.SSD_PATH_FLOAT, scales=None, ws=_UNSET, wsb=_UNSET, **ptr):
    """ssd_forward on fake addresses. Every use expects a validation error (or the
    empty no-op), so nothing is ever enqueued; a call that would pass validation
    is refused here instead of being sent to the library."""
    p = dict(X=A16, dt=A16, A=A16, B=A16, C=A16, D=A16, Y=A16, init=None, final=None)
    p.update(ptr)
    need = L.LIB.ssd_workspace_bytes(ctypes.byref(sh), path)
    ws = A16 if ws is _UNSET else ws
    wsb = need if wsb is _UNSET else wsb
    args = (ctypes.byref(sh), path, p["X"], p["dt"], p["A"], p["B"], p["C"], p["D"], scales,
            p["Y"], p["init"], p["final"], ws, wsb, None, None)
    return L.LIB.ssd_forward(*args)


@pytest.mark.parametrize("kw,rc", [
    (dict(chunk=32), L.SSD_E_UNSUPPORTED),
    (dict(chunk=100), L.SSD_E_UNSUPPORTED),
    (dict(headdim=8), L.SSD_E_UNSUPPORTED),
    (dict(headdim=128), L.SSD_E_UNSUPPORTED),
    (dict(dstate=256), L.SSD_E_UNSUPPORTED),
    (dict(dtype=7), L.SSD_E_UNSUPPORTED),
    (dict(nheads=6, ngroups=4), L.SSD_E_SHAPE),
    (dict(nheads=0), L.SSD_E_SHAPE),
    (dict(batch=-1), L.SSD_E_SHAPE),
    (dict(seqlen=-5), L.SSD_E_SHAPE),
    (dict(batch=70000), L.SSD_E_SHAPE),
    (dict(seqlen=1 << 40, batch=1 << 15, nheads=1 << 12), L.SSD_E_SHAPE),
])
def test_invalid_shapes(kw, rc):
    assert fwd(shape(**kw)) == rc


@pytest.mark.parametrize("sched", [-1, 3, 1 << 20])
def test_unknown_schedule(sched):
    sh = shape()
    sh.schedule = sched
    assert fwd(sh) == L.SSD_E_SHAPE


def test_noalloc_rejects_a_problem_beyond_its_array():
    # returned before the entry point looks up its device array, so no GPU is
    # touched; an explicitly chunk-parallel INT8 layer of 4 x 4096 positions,
    # 128 heads and 8 groups needs about 148 MiB of workspace
    sh = L.make_shape(4, 4096, 128, 64, 128, 8, 256, "bf16", L.SSD_SCHED_CHUNK)
    assert L.ssd_workspace_bytes(sh, L.SSD_PATH_INT8) > L.NOALLOC_SCRATCH_BYTES
    rc = L.LIB.ssd_forward_noalloc(ctypes.byref(sh), L.SSD_PATH_INT8, A16, A16, A16, A16, A16, A16, None,
                                   A16, None, None, None, None)
    assert rc == L.SSD_E_TOO_LARGE
    assert L.LIB.ssd_forward_noalloc(None, 0, A16, A16, A16, A16, A16, A16, None, A16, None, None, None,
                                     None) == L.SSD_E_NULL


def test_schedule_sets_int8_workspace():
    # the chunk-parallel schedule keeps every chunk's int8 state in the
    # workspace, the head-persistent one keeps it on chip; the float path has
    # one schedule
    def ws(sched, path):
        return L.ssd_workspace_bytes(L.make_shape(2, 1000, 8, 64, 128, 1, 256, "fp16", sched), path)

    assert ws(L.SSD_SCHED_CHUNK, L.SSD_PATH_INT8) >= ws(L.SSD_SCHED_HEAD, L.SSD_PATH_INT8) + 2 * 4 * 8 * 64 * 128
    assert ws(L.SSD_SCHED_CHUNK, L.SSD_PATH_FLOAT) == ws(L.SSD_SCHED_HEAD, L.SSD_PATH_FLOAT)


def test_null_and_alignment():
    sh = shape()
    assert fwd(sh, X=None) == L.SSD_E_NULL
    assert fwd(sh, Y=None) == L.SSD_E_NULL
    assert fwd(sh, B=MIS) == L.SSD_E_ALIGN
    assert fwd(sh, final=MIS) == L.SSD_E_ALIGN
    assert fwd(sh, init=MIS) == L.SSD_E_ALIGN
    assert L.LIB.ssd_forward(None, 0, A16, A16, A16, A16, A16, A16, None, A16, None, None, A16, 0, None,
                             None) == L.SSD_E_NULL


def test_bad_path_and_missing_scales():
    sh = shape()
    assert fwd(sh, path=5) == L.SSD_E_UNSUPPORTED
    assert fwd(sh, path=L.SSD_PATH_INT8, scales=None) == L.SSD_E_NULL
    bad = L.SsdScales(A16, A16, A16, A16, A16, A16, 0x10002)
    assert fwd(sh, path=L.SSD_PATH_INT8, scales=ctypes.byref(bad)) == L.SSD_E_ALIGN


def test_workspace_checks():
    sh = shape()
    for path in (L.SSD_PATH_FLOAT, L.SSD_PATH_INT8):
        need = L.LIB.ssd_workspace_bytes(ctypes.byref(sh), path)
        assert need > 0
        sc = L.SsdScales(*([A16] * 7))
        assert fwd(sh, path=path, scales=ctypes.byref(sc), wsb=need - 1) == L.SSD_E_WORKSPACE
        assert fwd(sh, path=path, scales=ctypes.byref(sc), ws=None, wsb=need) == L.SSD_E_WORKSPACE
    # invalid shapes report 0 bytes
    assert L.LIB.ssd_workspace_bytes(ctypes.byref(shape(chunk=3)), 0) == 0


def test_empty_problem_is_a_noop():
    for kw in (dict(batch=0), dict(seqlen=0)):
        sh = shape(**kw)
        assert L.LIB.ssd_workspace_bytes(ctypes.byref(sh), 0) == 0
        assert fwd(sh, ws=None, wsb=0) == L.SSD_OK


def test_module_calls_validate():
    sh = shape()
    sc = L.SsdScales(*([A16] * 7))
    b = ctypes.byref
    assert L.LIB.ssd_quantize_bc(b(sh), A16, A16, None, A16, A16, None) == L.SSD_E_NULL
    assert L.LIB.ssd_quantize_bc(b(sh), A16, MIS, b(sc), A16, A16, None) == L.SSD_E_ALIGN
    assert L.LIB.ssd_chunk_cumsum(b(sh), A16, None, A16, None, None, None) == L.SSD_E_NULL
    assert L.LIB.ssd_chunk_cumsum(b(sh), A16, A16, A16, MIS, None, None) == L.SSD_E_ALIGN
    assert L.LIB.ssd_chunk_state(b(sh), 1, A16, A16, A16, None, A16, None, None) == L.SSD_E_NULL
    assert L.LIB.ssd_chunk_state(b(sh), 3, A16, A16, A16, None, A16, None, None) == L.SSD_E_UNSUPPORTED
    assert L.LIB.ssd_state_passing(b(sh), 1, A16, None, None, None, None, None) == L.SSD_E_NULL
    assert L.LIB.ssd_state_passing(b(sh), 0, A16, None, None, None, None, None) == L.SSD_E_NULL
    assert L.LIB.ssd_state_passing(b(sh), 1, A16, None, A16, MIS, None, None) == L.SSD_E_ALIGN
    assert L.LIB.ssd_chunk_bmm(b(shape(chunk=48)), 1, A16, A16, A16, None) == L.SSD_E_UNSUPPORTED
    assert L.LIB.ssd_chunk_scan(b(sh), 1, A16, A16, A16, A16, A16, A16, None, A16, None, A16, None) == L.SSD_E_NULL
    assert L.LIB.ssd_chunk_scan(b(sh), 0, A16, A16, A16, A16, A16, A16, MIS, A16, None, A16, None) == L.SSD_E_ALIGN
    assert L.LIB.ssd_calibrate_amax(b(sh), A16, A16, A16, A16, A16, A16, A16, 0, None) == L.SSD_E_WORKSPACE


def test_scales_from_amax_matches_the_oracle_rule():
    """The host scale pack equals the oracle's pack for the same maxima, bit for bit."""
    from oracle import ssd_oracle as O
    rng = np.random.default_rng(0)
    G, H, P = 2, 4, 16
    amB = np.abs(rng.standard_normal(G)).astype(np.float32) * 4
    amC = np.abs(rng.standard_normal(G)).astype(np.float32) * 4
    amX = np.abs(rng.standard_normal((H, P))).astype(np.float32) * 3
    amS = np.abs(rng.standard_normal((H, P))).astype(np.float32) * 50
    amX[1, 3] = 0.0
    amax = np.concatenate([amB, amC, amX.ravel(), amS.ravel()])
    got = L.ssd_scales_from_amax(G, H, P, amax)
    ref = O.scale_pack(amB.astype(np.float64), amC.astype(np.float64), amX.astype(np.float64),
                       amS.astype(np.float64), H)
    for k in ("s_B", "s_C", "inv_B", "inv_C", "s_X", "inv_X", "s_S", "M_req"):
        assert np.array_equal(got[k], ref[k].reshape(-1)), k
    assert L.LIB.ssd_scales_from_amax(2, 5, 16, amax.ctypes.data, got["s_B"].ctypes.data) == L.SSD_E_SHAPE
    # a maximum that is negative or not finite has no scale, on both sides, and
    # the call writes nothing
    for i, bad in ((0, np.inf), (3, np.nan), (2 * G + 5, -1.0), (amax.size - 1, -np.inf)):
        a2 = amax.copy()
        a2[i] = bad
        pack = np.full(4 * G + 4 * H * P, 7.0, np.float32)
        assert L.LIB.ssd_scales_from_amax(G, H, P, a2.ctypes.data, pack.ctypes.data) == L.SSD_E_VALUE
        assert np.all(pack == 7.0)
        parts = np.split(a2.astype(np.float64), [G, 2 * G, 2 * G + H * P])
        with pytest.raises(ValueError):
            O.scale_pack(parts[0], parts[1], parts[2].reshape(H, P), parts[3].reshape(H, P), H)


def test_decode_step_validates():
    b = ctypes.byref
    sc = L.SsdScales(*([A16] * 7))

    def dec(sh, path=L.SSD_PATH_INT8, scales=b(sc), **ptr):
        p = dict(X=A16, dt=A16, A=A16, B=A16, C=A16, D=A16, state=A16, Y=A16)
        p.update(ptr)
        return L.LIB.ssd_decode_step(b(sh), path, p["X"], p["dt"], p["A"], p["B"], p["C"], p["D"],
                                     scales, p["state"], p["Y"], None)

    one = shape(seqlen=1)
    # only one position per call
    assert dec(shape(seqlen=2)) == L.SSD_E_SHAPE
    assert dec(shape(seqlen=0, batch=3)) == L.SSD_E_SHAPE
    # the one-wave-per-(batch, head) grid bound
    assert dec(shape(seqlen=1, batch=65535, nheads=512, ngroups=1)) == L.SSD_E_SHAPE
    assert dec(one, state=None) == L.SSD_E_NULL
    assert dec(one, Y=None) == L.SSD_E_NULL
    assert dec(one, state=MIS) == L.SSD_E_ALIGN
    assert dec(one, scales=None) == L.SSD_E_NULL
    assert dec(one, path=4) == L.SSD_E_UNSUPPORTED
    assert dec(shape(seqlen=1, dstate=256)) == L.SSD_E_UNSUPPORTED
    # empty batch: nothing to do
    assert dec(shape(seqlen=1, batch=0)) == L.SSD_OK


def test_ablation_paths_validate():
    b = ctypes.byref
    sh = shape()
    for path in (L.SSD_PATH_ABL_QX, L.SSD_PATH_ABL_RECON):
        assert L.LIB.ssd_workspace_bytes(b(sh), path) > 0
        # scales are required
        assert fwd(sh, path=path, scales=None) == L.SSD_E_NULL
        # no initial state on the ablation rows
        full = L.SsdScales(*([A16] * 10))
        assert fwd(sh, path=path, scales=b(full), init=A16) == L.SSD_E_UNSUPPORTED
    # "Q(X) only" reads only s_Xq and inv_Xq; the recon row also needs s_X
    qx_only = L.SsdScales(*([None] * 8 + [A16, A16]))
    assert fwd(sh, path=L.SSD_PATH_ABL_QX, scales=b(qx_only), ws=None, wsb=0) == L.SSD_E_WORKSPACE
    no_sx = L.SsdScales(*([A16] * 7 + [None, A16, A16]))
    assert fwd(sh, path=L.SSD_PATH_ABL_RECON, scales=b(no_sx)) == L.SSD_E_NULL
    # the module calls and the decode step run the float and INT8 paths only
    assert L.LIB.ssd_chunk_state(b(sh), 2, A16, A16, A16, None, A16, None, None) == L.SSD_E_UNSUPPORTED
    assert fwd(sh, path=4) == L.SSD_E_UNSUPPORTED


def test_epilogue_calls_validate():
    b = ctypes.byref
    sh = shape()
    assert L.LIB.ssd_epilogue(b(sh), None, None, 0.15, A16, 1e-5, A16, None) == L.SSD_E_NULL
    assert L.LIB.ssd_epilogue(b(sh), A16, MIS, 0.15, A16, 1e-5, A16, None) == L.SSD_E_ALIGN
    assert L.LIB.ssd_epilogue(b(sh), A16, None, 0.15, A16, -1.0, A16, None) == L.SSD_E_SHAPE
    assert L.LIB.ssd_epilogue(b(sh), A16, None, float("nan"), A16, 1e-5, A16, None) == L.SSD_E_SHAPE
    assert L.LIB.ssd_epilogue(b(shape(batch=0)), A16, None, 0.15, A16, 1e-5, A16, None) == L.SSD_OK
    assert L.LIB.ssd_mean_correction(b(sh), A16, None, A16, None) == L.SSD_E_NULL
    assert L.LIB.ssd_mean_correction(b(shape(seqlen=0)), A16, A16, A16, None) == L.SSD_E_SHAPE
