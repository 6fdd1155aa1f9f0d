"""GPU parity of every C-ABI call against the CPU oracle.

Module tests feed each GPU module the oracle's upstream values, so every stage
is checked on its own: integer outputs bit for bit, floating outputs within
the stated tolerance. Pipeline tests then run the GPU path from the raw inputs.

Tolerances (floating outputs): max over output channels (h, p) of
max|y - y_ref| / RMS(y_ref on that channel) <= 2e-2 (float path, against the
float64 definition) and <= 5e-2 (INT8 path, against the INT8 method).
"""
import functools

import numpy as np
import pytest

from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

CASE_NAMES = list(H.CASES)


@functools.lru_cache(maxsize=None)
def case_data(name):
    c = H.make_case(H.CASES[name])
    e = c.ev64
    r8 = O.forward_int8(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], c.scales,
                        c.w.chunk)
    yf, hf, S, Hs = O.chunked(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"],
                              c.w.chunk)
    return c, r8, (yf, hf, S, Hs)


def _setup(L, name):
    import torch
    c, r8, fl = case_data(name)
    d = H.dev_inputs(c)
    sh = H.shape_of(L, c.w)
    sc = L.ScalePack(c.scales)
    return torch, c, r8, fl, d, sh, sc


def _i8(t, a):
    return t.from_numpy(np.ascontiguousarray(a.astype(np.int8))).cuda()


def _dev(a, dtype):
    """numpy -> dense device tensor (oracle arrays are often transposed views)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


@pytest.mark.parametrize("name", CASE_NAMES)
def test_quantize_bc(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    qB = torch.empty(d["B"].shape, dtype=torch.int8, device="cuda")
    qC = torch.empty_like(qB)
    L.ssd_quantize_bc(sh, d["B"], d["C"], sc, qB, qC)
    torch.cuda.synchronize()
    assert np.array_equal(qB.cpu().numpy(), r8["qB"])
    assert np.array_equal(qC.cpu().numpy(), r8["qC"])


@pytest.mark.parametrize("name", CASE_NAMES)
def test_chunk_cumsum(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    w = c.w
    n = (w.batch, w.nheads, w.nchunks, w.chunk)
    dAcs = torch.empty(n, dtype=torch.float32, device="cuda")
    lut = torch.empty(n, dtype=torch.float32, device="cuda")
    qd = torch.empty(n[:3], dtype=torch.uint8, device="cuda")
    L.ssd_chunk_cumsum(sh, d["dt"], d["A"], dAcs, lut, qd)
    torch.cuda.synchronize()
    cs = r8["cumsum"]
    # same float64 additions in the same order: bit-exact
    assert np.array_equal(dAcs.cpu().numpy(), cs["dAcs"].astype(np.float32))
    assert np.array_equal(qd.cpu().numpy(), cs["qdecay"])
    # LUT goes through exp(): at most one float32 ulp apart, almost always equal
    ud = H.ulp_diff_f32(lut.cpu().numpy(), cs["lut"].astype(np.float32))
    assert ud.max() <= 1 and (ud > 0).mean() < 1e-4


@pytest.mark.parametrize("name", CASE_NAMES)
def test_chunk_state_int8(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    w = c.w
    lut = _dev(r8["cumsum"]["lut"], np.float32)
    qB = _i8(torch, r8["qB"])
    st = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    qxs = torch.empty(d["x"].shape, dtype=torch.int8, device="cuda")
    s32 = torch.empty(st.shape, dtype=torch.int32, device="cuda")
    L.ssd_chunk_state(sh, L.SSD_PATH_INT8, d["x"], lut, qB, sc, st, taps={"q_xs": qxs, "s32": s32})
    torch.cuda.synchronize()
    assert np.array_equal(qxs.cpu().numpy(), r8["qxs"])
    assert np.array_equal(s32.cpu().numpy(), r8["s32"])
    assert np.array_equal(st.cpu().numpy(), r8["s8"])


@pytest.mark.parametrize("name", CASE_NAMES)
def test_state_passing_int8(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    st = _i8(torch, r8["s8"])
    qd = _dev(r8["cumsum"]["qdecay"], np.uint8)
    fin = torch.empty(st[:, 0].shape, dtype=torch.int8, device="cuda")
    L.ssd_state_passing(sh, L.SSD_PATH_INT8, st, None, qd, fin)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), r8["passed"])
    assert np.array_equal(fin.cpu().numpy(), r8["passed"][:, -1])


@pytest.mark.parametrize("nchunks,with_init", [(1, False), (1, True), (7, False), (33, True), (45, False),
                                               (80, True)])
def test_state_passing_int8_chain_lengths(gpu_lib, nchunks, with_init):
    """Eq. 6 over chains of 1 to 80 chunks (both group sizes of the kernel and
    their ragged last groups), with Q(Decay) rows starting at every byte
    offset, saturating states and decays of 0 and 128 included: bit-exact
    against the oracle's chain, the final state too."""
    import torch
    L = gpu_lib
    rng = np.random.default_rng(1000 + nchunks)
    B, H, P, N, l = 2, 3, 16, 32, 64
    s8 = rng.integers(-127, 128, size=(B, nchunks, H, P, N)).astype(np.int64)
    qd = rng.integers(0, 129, size=(B, H, nchunks)).astype(np.int64)
    qd[0, 0, ::5] = 128
    qd[1, 2, ::7] = 0
    h0 = rng.integers(-127, 128, size=(B, H, P, N)).astype(np.int64) if with_init else None
    ref = O.state_passing_int(s8, qd, 8, h0)
    sh = L.make_shape(B, nchunks * l, H, P, N, 1, l, "fp16")
    st = _i8(torch, s8)
    fin = torch.empty((B, H, P, N), dtype=torch.int8, device="cuda")
    L.ssd_state_passing(sh, L.SSD_PATH_INT8, st, None, _dev(qd, np.uint8), fin,
                        initial_state=None if h0 is None else _i8(torch, h0))
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), ref)
    assert np.array_equal(fin.cpu().numpy(), ref[:, -1])
    assert (np.abs(ref) == 127).any()  # the chain saturates somewhere


@pytest.mark.parametrize("name", CASE_NAMES)
def test_chunk_bmm_int8(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    w = c.w
    cb = torch.empty((w.batch, w.nchunks, w.ngroups, w.chunk, w.chunk), dtype=torch.int32, device="cuda")
    L.ssd_chunk_bmm(sh, L.SSD_PATH_INT8, _i8(torch, r8["qC"]), _i8(torch, r8["qB"]), cb)
    torch.cuda.synchronize()
    ref = np.tril(r8["cb"])
    assert np.array_equal(cb.cpu().numpy(), ref)


@pytest.mark.parametrize("name", CASE_NAMES)
def test_chunk_scan_int8(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, _, d, sh, sc = _setup(L, name)
    cs = r8["cumsum"]
    dAcs = _dev(cs["dAcs"], np.float32)
    cb = _dev(np.tril(r8["cb"]), np.int32)
    y = torch.empty_like(d["x"])
    L.ssd_chunk_scan(sh, L.SSD_PATH_INT8, d["x"], d["dt"], dAcs, _i8(torch, r8["qC"]), cb,
                     _i8(torch, r8["passed"]), d["D"], sc, y)
    torch.cuda.synchronize()
    assert H.chan_err(H.f64(y), r8["y"], c.w.dtype) <= 5e-2


@pytest.mark.parametrize("name", CASE_NAMES)
def test_float_modules(gpu_lib, name):
    """Float path modules: ChunkState, StatePassing, ChunkBMM, ChunkScan."""
    L = gpu_lib
    torch, c, r8, (yf, hf, S, Hs), d, sh, sc = _setup(L, name)
    w = c.w
    cs = r8["cumsum"]
    lut = _dev(cs["lut"], np.float32)
    dAcs = _dev(cs["dAcs"], np.float32)
    st = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    L.ssd_chunk_state(sh, L.SSD_PATH_FLOAT, d["x"], lut, d["B"], None, st)
    torch.cuda.synchronize()
    Sg = st.cpu().numpy().astype(np.float64)
    tol = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 1.5e-2}[w.dtype]
    assert np.abs(Sg - S).max() <= tol * np.abs(S).max()
    # passing on the oracle's float64 local states (cast to fp32)
    st2 = _dev(S, np.float32)
    fin = torch.empty(st2[:, 0].shape, dtype=torch.float32, device="cuda")
    L.ssd_state_passing(sh, L.SSD_PATH_FLOAT, st2, dAcs, None, fin)
    torch.cuda.synchronize()
    Hg = st2.cpu().numpy().astype(np.float64)
    assert np.abs(Hg - Hs).max() <= 1e-4 * np.abs(Hs).max()
    assert np.array_equal(fin.cpu().numpy(), st2[:, -1].cpu().numpy())
    # ChunkBMM against C B^T of the stored inputs
    cb = torch.empty((w.batch, w.nchunks, w.ngroups, w.chunk, w.chunk), dtype=torch.float32, device="cuda")
    L.ssd_chunk_bmm(sh, L.SSD_PATH_FLOAT, d["C"], d["B"], cb)
    torch.cuda.synchronize()
    e = c.ev64
    Lp = w.nchunks * w.chunk
    pad = lambda a: np.concatenate([a, np.zeros((a.shape[0], Lp - a.shape[1]) + a.shape[2:])], 1)  # noqa: E731
    Cp = pad(e["C"]).reshape(w.batch, w.nchunks, w.chunk, w.ngroups, w.dstate)
    Bp = pad(e["B"]).reshape(w.batch, w.nchunks, w.chunk, w.ngroups, w.dstate)
    ref = np.tril(np.einsum("bkign,bkjgn->bkgij", Cp, Bp))
    cbg = cb.cpu().numpy().astype(np.float64)
    assert np.abs(cbg - ref).max() <= {"fp32": 1e-5, "fp16": 1e-3, "bf16": 1e-3}[w.dtype] * np.abs(ref).max()
    # ChunkScan with the oracle's passed states
    y = torch.empty_like(d["x"])
    L.ssd_chunk_scan(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], dAcs, d["C"], cb,
                     _dev(Hs, np.float32), d["D"], None, y)
    torch.cuda.synchronize()
    assert H.chan_err(H.f64(y), yf, c.w.dtype) <= 2e-2


def _modular_int8(L, torch, c, d, sh, sc):
    """The INT8 path through the six module calls (GPU outputs feed GPU modules)."""
    w = c.w
    qB = torch.empty(d["B"].shape, dtype=torch.int8, device="cuda")
    qC = torch.empty_like(qB)
    L.ssd_quantize_bc(sh, d["B"], d["C"], sc, qB, qC)
    n = (w.batch, w.nheads, w.nchunks, w.chunk)
    dAcs = torch.empty(n, dtype=torch.float32, device="cuda")
    lut = torch.empty_like(dAcs)
    qd = torch.empty(n[:3], dtype=torch.uint8, device="cuda")
    L.ssd_chunk_cumsum(sh, d["dt"], d["A"], dAcs, lut, qd)
    st = torch.empty((w.batch, w.nchunks, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    L.ssd_chunk_state(sh, L.SSD_PATH_INT8, d["x"], lut, qB, sc, st)
    L.ssd_state_passing(sh, L.SSD_PATH_INT8, st, None, qd)
    cb = torch.empty((w.batch, w.nchunks, w.ngroups, w.chunk, w.chunk), dtype=torch.int32, device="cuda")
    L.ssd_chunk_bmm(sh, L.SSD_PATH_INT8, qC, qB, cb)
    y = torch.empty_like(d["x"])
    L.ssd_chunk_scan(sh, L.SSD_PATH_INT8, d["x"], d["dt"], dAcs, qC, cb, st, d["D"], sc, y)
    torch.cuda.synchronize()
    return {"passed": st.cpu().numpy(), "y": H.f64(y)}


@pytest.mark.parametrize("sched", list(H.SCHEDULES))
@pytest.mark.parametrize("name", CASE_NAMES)
def test_forward_int8(gpu_lib, name, sched):
    L = gpu_lib
    torch, c, r8, (yf, _, _, _), d, _, sc = _setup(L, name)
    w = c.w
    sh = H.shape_of(L, w, schedule=sched)
    y = torch.empty_like(d["x"])
    stshape = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    taps = {"q_xs": torch.empty(d["x"].shape, dtype=torch.int8, device="cuda"),
            "s32": torch.empty(stshape, dtype=torch.int32, device="cuda"),
            "s8_local": torch.empty(stshape, dtype=torch.int8, device="cuda"),
            "passed": torch.empty(stshape, dtype=torch.int8, device="cuda")}
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], sc, y,
                  final_state=fin, taps=taps)
    torch.cuda.synchronize()
    assert np.array_equal(taps["q_xs"].cpu().numpy(), r8["qxs"])
    assert np.array_equal(taps["s32"].cpu().numpy(), r8["s32"])
    assert np.array_equal(taps["s8_local"].cpu().numpy(), r8["s8"])
    assert np.array_equal(taps["passed"].cpu().numpy(), r8["passed"])
    assert np.array_equal(fin.cpu().numpy(), r8["passed"][:, -1])
    e = c.ev64
    err = H.chan_err(H.f64(y), r8["y"], c.w.dtype)
    bud = H.int8_budget(H.f64(y), r8, e["x"], e["dt"], c.consts["D"], c.scales, w.chunk, w.dtype)
    H.report(f"int8 {name} {sched}", chan_err=err, budget=bud)
    assert err <= 5e-2
    assert bud <= 1.0
    # determinism: a second run (without taps) is bitwise identical, final state too
    y2 = torch.empty_like(y)
    fin2 = torch.empty_like(fin)
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], sc, y2,
                  final_state=fin2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(fin, fin2)
    # and the module-by-module composition gives the same integers, and a Y held
    # to the same bars against the oracle
    ym = _modular_int8(L, torch, c, d, sh, sc)
    assert np.array_equal(ym["passed"], r8["passed"])
    assert H.chan_err(ym["y"], r8["y"], c.w.dtype) <= 5e-2
    assert H.int8_budget(ym["y"], r8, e["x"], e["dt"], c.consts["D"], c.scales, w.chunk, w.dtype) <= 1.0


@pytest.mark.parametrize("name", CASE_NAMES)
def test_int8_schedules_agree(gpu_lib, name):
    """The head-persistent and chunk-parallel schedules do the same arithmetic
    per output element, so they give the same final state and Y bit for bit."""
    L = gpu_lib
    torch, c, _, _, d, _, sc = _setup(L, name)
    w = c.w
    out = {}
    for sched in H.SCHEDULES:
        y = torch.empty_like(d["x"])
        fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
        L.ssd_forward(H.shape_of(L, w, schedule=sched), L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"],
                      d["C"], d["D"], sc, y, final_state=fin)
        torch.cuda.synchronize()
        out[sched] = (y.cpu(), fin.cpu().numpy())
    (yh, fh), (yc, fc) = out["head"], out["chunk"]
    assert np.array_equal(fh, fc)
    print(f"{name}: head vs chunk Y max channel error {H.chan_err(H.f64(yc), H.f64(yh)):.3g}", flush=True)
    assert torch.equal(H.bits(yh), H.bits(yc))


@pytest.mark.parametrize("name", CASE_NAMES)
def test_forward_float(gpu_lib, name):
    L = gpu_lib
    torch, c, r8, (yf, hf, _, _), d, sh, sc = _setup(L, name)
    w = c.w
    y = torch.empty_like(d["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    L.ssd_forward(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, y,
                  final_state=fin)
    torch.cuda.synchronize()
    e = c.ev64
    fg = fin.cpu().numpy().astype(np.float64)
    err = H.chan_err(H.f64(y), yf, c.w.dtype)
    serr = H.state_chan_err(fg, hf)
    by, bh = H.float_budget(H.f64(y), fg, e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"],
                            w.chunk, w.dtype, yf, hf)
    H.report(f"float {name}", chan_err=err, state_chan_err=serr, budget_y=by, budget_state=bh)
    assert err <= 2e-2
    assert serr <= 1e-2
    assert by <= 1.0 and bh <= 1.0


@pytest.mark.parametrize("name", CASE_NAMES)
def test_calibrate_amax(gpu_lib, name):
    import torch
    L = gpu_lib
    c, _, _ = case_data(name)
    w = c.w
    cal = H.synth.calibration_sequences(w, c.consts)
    A = torch.from_numpy(c.consts["A"]).cuda()
    G, HP = w.ngroups, w.nheads * w.headdim
    amax = torch.zeros(2 * G + 2 * HP, dtype=torch.float32, device="cuda")
    for s in cal:
        ds = {k: H.to_dev(v, w.dtype) for k, v in s.items()}
        L.ssd_calibrate_amax(H.shape_of(L, w, batch=1), ds["x"], ds["dt"], A, ds["B"], ds["C"], amax)
    torch.cuda.synchronize()
    a = amax.cpu().numpy().astype(np.float64)
    ref = O.calibrate([H.synth.as_f64(s, w.dtype) for s in cal], c.consts["A"], G, w.chunk)
    assert np.array_equal(a[:G], ref["B"]) and np.array_equal(a[G:2 * G], ref["C"])
    ax = a[2 * G:2 * G + HP].reshape(ref["Xs"].shape)
    assert np.abs(ax - ref["Xs"]).max() <= 1e-6 * ref["Xs"].max()
    asx = a[2 * G + HP:].reshape(ref["S"].shape)
    tol = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 5e-2}[w.dtype]
    assert np.all(np.abs(asx - ref["S"]) <= tol * ref["S"] + 1e-6)


# ---------------------------------------------------------------------------
# Initial state (chunked-prefill continuation)
# ---------------------------------------------------------------------------
def _init_int8(w, seed=7):
    rng = np.random.default_rng(seed)
    return rng.integers(-127, 128, size=(w.batch, w.nheads, w.headdim, w.dstate)).astype(np.int8)


@pytest.mark.parametrize("sched", list(H.SCHEDULES))
@pytest.mark.parametrize("name", CASE_NAMES)
def test_forward_int8_initial_state(gpu_lib, name, sched):
    L = gpu_lib
    torch, c, _, _, d, _, sc = _setup(L, name)
    w, e = c.w, c.ev64
    sh = H.shape_of(L, w, schedule=sched)
    h0 = _init_int8(w)
    r = O.forward_int8(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], c.scales, w.chunk,
                       h_init=h0.astype(np.int64))
    y = torch.empty_like(d["x"])
    fin = torch.empty(h0.shape, dtype=torch.int8, device="cuda")
    stshape = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
    taps = {"passed": torch.empty(stshape, dtype=torch.int8, device="cuda")}
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], sc, y,
                  final_state=fin, taps=taps, initial_state=_i8(torch, h0))
    torch.cuda.synchronize()
    assert np.array_equal(taps["passed"].cpu().numpy(), r["passed"])
    assert np.array_equal(fin.cpu().numpy(), r["passed"][:, -1])
    err = H.chan_err(H.f64(y), r["y"], w.dtype)
    bud = H.int8_budget(H.f64(y), r, e["x"], e["dt"], c.consts["D"], c.scales, w.chunk, w.dtype,
                        h_init=h0.astype(np.float64))
    H.report(f"int8 initial state {name} {sched}", chan_err=err, budget=bud)
    assert err <= 5e-2
    assert bud <= 1.0


@pytest.mark.parametrize("name", CASE_NAMES)
def test_forward_float_initial_state(gpu_lib, name):
    L = gpu_lib
    torch, c, _, (yf, hf, _, _), d, sh, sc = _setup(L, name)
    w, e = c.w, c.ev64
    h0 = hf[:, ::-1].copy()  # a state of realistic size (the heads' final states, reordered)
    yr, hr = O.chunked(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], w.chunk, h0=h0)[:2]
    y = torch.empty_like(d["x"])
    fin = torch.empty(h0.shape, dtype=torch.float32, device="cuda")
    L.ssd_forward(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, y,
                  final_state=fin, initial_state=_dev(h0, np.float32))
    torch.cuda.synchronize()
    fg = fin.cpu().numpy().astype(np.float64)
    err = H.chan_err(H.f64(y), yr, w.dtype)
    serr = H.state_chan_err(fg, hr)
    by, bh = H.float_budget(H.f64(y), fg, e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"],
                            w.chunk, w.dtype, yr, hr, h_init=h0)
    H.report(f"float initial state {name}", chan_err=err, state_chan_err=serr, budget_y=by, budget_state=bh)
    assert err <= 2e-2
    assert serr <= 1e-2
    assert by <= 1.0 and bh <= 1.0


@pytest.mark.parametrize("path", ["int8-head", "int8-chunk", "float"])
@pytest.mark.parametrize("name", ["f16_ragged", "bf16_n64_l128", "w0"])
def test_continuation_at_a_chunk_boundary(gpu_lib, name, path):
    """Two calls (the second starting from the first's final state) give bitwise
    the outputs and final state of one call over the whole sequence."""
    L = gpu_lib
    torch, c, _, _, d, _, sc = _setup(L, name)
    w = c.w
    i8 = path != "float"
    sched = path.split("-")[1] if i8 else 0
    sh = H.shape_of(L, w, schedule=sched)
    p = L.SSD_PATH_INT8 if i8 else L.SSD_PATH_FLOAT
    scales = sc if i8 else None
    fdt = torch.int8 if i8 else torch.float32
    fshape = (w.batch, w.nheads, w.headdim, w.dstate)
    y = torch.empty_like(d["x"])
    fin = torch.empty(fshape, dtype=fdt, device="cuda")
    L.ssd_forward(sh, p, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], scales, y, final_state=fin)
    L1 = w.chunk
    part = lambda t, a_, b_: t[:, a_:b_].contiguous()  # noqa: E731
    sh1 = H.shape_of(L, w, seqlen=L1, schedule=sched)
    sh2 = H.shape_of(L, w, seqlen=w.seqlen - L1, schedule=sched)
    y1 = torch.empty_like(part(d["x"], 0, L1))
    y2 = torch.empty_like(part(d["x"], L1, None))
    f1 = torch.empty(fshape, dtype=fdt, device="cuda")
    f2 = torch.empty(fshape, dtype=fdt, device="cuda")
    L.ssd_forward(sh1, p, part(d["x"], 0, L1), part(d["dt"], 0, L1), d["A"], part(d["B"], 0, L1),
                  part(d["C"], 0, L1), d["D"], scales, y1, final_state=f1)
    L.ssd_forward(sh2, p, part(d["x"], L1, None), part(d["dt"], L1, None), d["A"], part(d["B"], L1, None),
                  part(d["C"], L1, None), d["D"], scales, y2, final_state=f2, initial_state=f1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=1), y)
    assert torch.equal(f2, fin)


def _cumsum_dt_A(dtype, L, H, seed):
    """dt [1, L, H] and A [H] with three kinds of heads: ordinary draws (h % 5 in
    0, 3, 4); a spread of about 2^30 in dt within each chunk (h % 5 == 1); and a
    sum that needs 52 of float64's 53 bits when added exactly (h % 5 == 2: A
    with a full float32 significand, one dt of 2^-24, the rest 0.1 or 0.2)."""
    from mamba_ssd_chunked_amd import synth
    rng = np.random.default_rng(seed)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(1, L, H)))
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    s = np.arange(L)
    for h in range(H):
        if h % 5 == 1:
            dt[0, :, h] = np.where(s % 7 == 0, 2.0 ** -24, rng.uniform(1.0, 60.0, size=L))
        elif h % 5 == 2:
            dt[0, :, h] = 0.1 if h % 2 == 0 else 0.2
            dt[0, 3::97, h] = 2.0 ** -24
            A[h] = np.float32(-(1.0 + 2.0 ** -23))
    stored = synth.cast(dt, dtype)
    return stored, synth.to_f64(stored, dtype), A


@pytest.mark.parametrize("dtype,chunk", [("fp16", 256), ("fp16", 64), ("bf16", 128)])
def test_chunk_cumsum_exact_scan_and_chain(gpu_lib, dtype, chunk):
    """dAcs must equal the sequential float64 sums bit for bit whether a head is
    summed by the exact wave scan or by the sequential chain; the heads above
    sit on both sides of the exactness bound (20 heads: a full and a partial
    block of 16; a ragged last chunk)."""
    import torch
    L = gpu_lib
    nh, Lseq = 20, 3 * chunk - 37
    stored, dt64, A = _cumsum_dt_A(dtype, Lseq, nh, seed=11 + chunk)
    nc = (Lseq + chunk - 1) // chunk
    sh = L.make_shape(1, Lseq, nh, 64, 64, 1, chunk, dtype)
    dt_d = torch.from_numpy(np.ascontiguousarray(stored)).cuda()
    A_d = torch.from_numpy(A).cuda()
    dAcs = torch.empty((1, nh, nc, chunk), dtype=torch.float32, device="cuda")
    lut = torch.empty_like(dAcs)
    qd = torch.empty((1, nh, nc), dtype=torch.uint8, device="cuda")
    L.ssd_chunk_cumsum(sh, dt_d, A_d, dAcs, lut, qd)
    torch.cuda.synchronize()
    cs = O.chunk_cumsum(dt64, A, chunk)
    assert np.array_equal(dAcs.cpu().numpy(), cs["dAcs"].astype(np.float32))
    assert np.array_equal(qd.cpu().numpy(), cs["qdecay"])
    ud = H.ulp_diff_f32(lut.cpu().numpy(), cs["lut"].astype(np.float32))
    assert ud.max() <= 1 and (ud > 0).mean() < 1e-3
