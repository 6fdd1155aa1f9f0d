"""GPU parity of ssd_decode_step (one position per call) against the oracle's
decode steps.

A prefill runs ssd_forward over the first L0 positions of a seeded sequence
and leaves its final state; T decode steps then consume positions L0..L0+T-1
one at a time on that state. The oracle does the same with its own forward
and its decode steps. INT8: the prefill's final state and the state after
every step match bit for bit; Y of all steps within the INT8 tolerance
(5e-2 of the channel RMS, against the INT8 method). FLOAT: Y within 2e-2 of
the float64 recurrence, the state within the float path's state bound.
"""
import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

T_STEPS = 6
CASES = {
    "f16_ragged": 200,      # L0 not a multiple of the chunk
    "bf16_l128": 256,
    "f16_g_eq_h": 64,
    "f32_l256": 256,
    "bf16_n64_l128": 100,
    "w0": 64,
}


def _case(name):
    w = H.CASES[name]
    L0 = CASES[name]
    c = H.make_case(w, seqlen=L0 + T_STEPS)
    return c, L0


def _slice(a, lo, hi):
    return np.ascontiguousarray(a[:, lo:hi])


def _step(a, t):
    return np.ascontiguousarray(a[:, t])


def _prefill(L, torch, c, L0, path, h_dev):
    w = c.w
    d = {k: H.to_dev(_slice(v, 0, L0), w.dtype) for k, v in c.ev.items()}
    A = torch.from_numpy(c.consts["A"]).cuda()
    D = torch.from_numpy(c.consts["D"]).cuda()
    sh = H.shape_of(L, w, seqlen=L0)
    y = torch.empty_like(d["x"])
    sc = L.ScalePack(c.scales) if path == L.SSD_PATH_INT8 else None
    L.ssd_forward(sh, path, d["x"], d["dt"], A, d["B"], d["C"], D, sc, y, final_state=h_dev)
    return A, D, sc


def _decode(L, torch, c, path, A, D, sc, h_dev, t):
    w = c.w
    sh = H.shape_of(L, w, seqlen=1)
    x = H.to_dev(_step(c.ev["x"], t), w.dtype)
    dt = H.to_dev(_step(c.ev["dt"], t), w.dtype)
    B = H.to_dev(_step(c.ev["B"], t), w.dtype)
    C = H.to_dev(_step(c.ev["C"], t), w.dtype)
    y = torch.empty_like(x)
    L.ssd_decode_step(sh, path, x, dt, A, B, C, D, sc, h_dev, y)
    return y


@pytest.mark.parametrize("name", list(CASES))
def test_decode_int8_steps(gpu_lib, name):
    import torch
    L = gpu_lib
    c, L0 = _case(name)
    w, e = c.w, c.ev64
    print(f"decode int8 {name}", flush=True)
    h_dev = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    A, D, sc = _prefill(L, torch, c, L0, L.SSD_PATH_INT8, h_dev)
    torch.cuda.synchronize()
    r = O.forward_int8(_slice(e["x"], 0, L0), _slice(e["dt"], 0, L0), c.consts["A"],
                       _slice(e["B"], 0, L0), _slice(e["C"], 0, L0), c.consts["D"], c.scales,
                       w.chunk)
    h = r["passed"][:, -1]
    assert np.array_equal(h_dev.cpu().numpy(), h)
    ys, refs = [], []
    for t in range(L0, L0 + T_STEPS):
        y = _decode(L, torch, c, L.SSD_PATH_INT8, A, D, sc, h_dev, t)
        s = O.decode_step_int8(_step(e["x"], t), _step(e["dt"], t), c.consts["A"],
                               _step(e["B"], t), _step(e["C"], t), c.consts["D"], c.scales, h)
        h = s["h"]
        torch.cuda.synchronize()
        assert np.array_equal(h_dev.cpu().numpy(), h), t
        ys.append(H.f64(y))
        refs.append(s["y"])
    err = H.chan_err(np.stack(ys, 1), np.stack(refs, 1), w.dtype)
    assert err <= 5e-2, err


@pytest.mark.parametrize("name", list(CASES))
def test_decode_float_steps(gpu_lib, name):
    import torch
    L = gpu_lib
    c, L0 = _case(name)
    w, e = c.w, c.ev64
    print(f"decode float {name}", flush=True)
    h_dev = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                        device="cuda")
    A, D, _ = _prefill(L, torch, c, L0, L.SSD_PATH_FLOAT, h_dev)
    yf, hf = O.chunked(_slice(e["x"], 0, L0), _slice(e["dt"], 0, L0), c.consts["A"],
                       _slice(e["B"], 0, L0), _slice(e["C"], 0, L0), c.consts["D"], w.chunk)[:2]
    h = hf
    ys, refs = [], []
    for t in range(L0, L0 + T_STEPS):
        y = _decode(L, torch, c, L.SSD_PATH_FLOAT, A, D, None, h_dev, t)
        yr, h = O.decode_step_float(_step(e["x"], t), _step(e["dt"], t), c.consts["A"],
                                    _step(e["B"], t), _step(e["C"], t), c.consts["D"], h)
        ys.append(H.f64(y))
        refs.append(yr)
    torch.cuda.synchronize()
    err = H.chan_err(np.stack(ys, 1), np.stack(refs, 1), w.dtype)
    assert err <= 2e-2, err
    hg = h_dev.cpu().numpy().astype(np.float64)
    assert np.abs(hg - h).max() <= 2e-1 * np.sqrt(np.mean(h * h))


@pytest.mark.parametrize("name", ["f16_ragged", "bf16_n64_l128"])
def test_decode_int8_equals_a_one_position_forward(gpu_lib, name):
    """A decode step and ssd_forward over one position continuing from the
    same initial state leave the same INT8 state (the one-position chunk)."""
    import torch
    L = gpu_lib
    c, L0 = _case(name)
    w = c.w
    h_dev = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    A, D, sc = _prefill(L, torch, c, L0, L.SSD_PATH_INT8, h_dev)
    h_prev = h_dev.clone()
    h_fwd = torch.empty_like(h_dev)
    d = {k: H.to_dev(_slice(v, L0, L0 + 1), w.dtype) for k, v in c.ev.items()}
    y_fwd = torch.empty_like(d["x"])
    L.ssd_forward(H.shape_of(L, w, seqlen=1), L.SSD_PATH_INT8, d["x"], d["dt"], A, d["B"], d["C"],
                  D, sc, y_fwd, final_state=h_fwd, initial_state=h_prev)
    y = _decode(L, torch, c, L.SSD_PATH_INT8, A, D, sc, h_dev, L0)
    torch.cuda.synchronize()
    assert torch.equal(h_dev, h_fwd)
    r = O.decode_step_int8(_step(c.ev64["x"], L0), _step(c.ev64["dt"], L0), c.consts["A"],
                           _step(c.ev64["B"], L0), _step(c.ev64["C"], L0), c.consts["D"],
                           c.scales, h_prev.cpu().numpy().astype(np.int64))
    assert np.array_equal(h_dev.cpu().numpy(), r["h"])
    assert H.chan_err(H.f64(y)[:, None], r["y"][:, None], w.dtype) <= 5e-2
    assert H.chan_err(H.f64(y_fwd), r["y"][:, None], w.dtype) <= 5e-2


def _layer_step_inputs(w, batch):
    """One decode position of the layer workload at a given batch, with a
    seeded state drawn uniformly from the int8 range."""
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts, batch=batch, seqlen=1)
    return consts, ev, synth.int8_state(w, batch)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("batch", [8, 1024])
def test_decode_layer_shape(gpu_lib, batch):
    """The 2.7B-shaped layer (H=80, P=64, N=128) at the two timed decode
    batches: every batch row at batch 8, sampled rows at batch 1024."""
    import torch
    L = gpu_lib
    w = synth.WORKLOADS[2]
    print(f"decode layer shape batch {batch}", flush=True)
    consts, ev, h0 = _layer_step_inputs(w, batch)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts, seqlen=512)]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    sc_np = O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads)
    sc = L.ScalePack(sc_np)
    d = {k: H.to_dev(np.ascontiguousarray(v[:, 0]), w.dtype) for k, v in ev.items()}
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    sh = L.make_shape(batch, 1, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
    h_dev = torch.from_numpy(h0).cuda()
    y = torch.empty_like(d["x"])
    L.ssd_decode_step(sh, L.SSD_PATH_INT8, d["x"], d["dt"], A, d["B"], d["C"], D, sc, h_dev, y)
    hf_dev = torch.from_numpy(h0.astype(np.float32)).cuda()
    yf = torch.empty_like(d["x"])
    L.ssd_decode_step(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], A, d["B"], d["C"], D, None, hf_dev, yf)
    torch.cuda.synchronize()
    rows = list(range(batch)) if batch <= 8 else sorted({0, 1, batch // 2, batch - 1})
    e = synth.as_f64(ev, w.dtype)
    y8, r8, y32, r32 = [], [], [], []
    for b in rows:
        s = O.decode_step_int8(e["x"][b:b + 1, 0], e["dt"][b:b + 1, 0], consts["A"],
                               e["B"][b:b + 1, 0], e["C"][b:b + 1, 0], consts["D"], sc_np,
                               h0[b:b + 1].astype(np.int64))
        assert np.array_equal(h_dev[b].cpu().numpy(), s["h"][0]), b
        yr, hr = O.decode_step_float(e["x"][b:b + 1, 0], e["dt"][b:b + 1, 0], consts["A"],
                                     e["B"][b:b + 1, 0], e["C"][b:b + 1, 0], consts["D"],
                                     h0[b:b + 1].astype(np.float64))
        hg = hf_dev[b].cpu().numpy().astype(np.float64)
        assert np.abs(hg - hr[0]).max() <= 1e-5 * np.abs(hr).max(), b
        y8.append(H.f64(y[b]))
        r8.append(s["y"][0])
        y32.append(H.f64(yf[b]))
        r32.append(yr[0])
    err8 = H.chan_err(np.stack(y8)[:, None], np.stack(r8)[:, None], w.dtype)
    err32 = H.chan_err(np.stack(y32)[:, None], np.stack(r32)[:, None], w.dtype)
    assert err8 <= 5e-2 and err32 <= 2e-2, (err8, err32)


def test_decode_empty_batch_is_a_noop(gpu_lib):
    import torch
    L = gpu_lib
    sh = L.make_shape(0, 1, 4, 16, 16, 1, 64, "fp16")
    z = torch.empty(16, dtype=torch.float16, device="cuda")
    st = torch.zeros(16, dtype=torch.int8, device="cuda")
    A = torch.zeros(4, dtype=torch.float32, device="cuda")
    sc = L.ScalePack({k: np.ones(64, np.float32) for k in L.ScalePack.ORDER})
    L.ssd_decode_step(sh, L.SSD_PATH_INT8, z, z, A, z, z, A, sc, st, z)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0


@pytest.mark.parametrize("path", ["int8", "float"])
def test_decode_steps_replayed_from_a_graph(gpu_lib, path):
    """Three decode steps captured in one HIP graph and replayed twice, with
    eager work between the replays, leave the states three and six eager
    steps leave (bitwise: the same kernels on the same inputs)."""
    import torch
    L = gpu_lib
    c, L0 = _case("f16_ragged")
    w = c.w
    i8 = path == "int8"
    p = L.SSD_PATH_INT8 if i8 else L.SSD_PATH_FLOAT
    h_dev = torch.empty((w.batch, w.nheads, w.headdim, w.dstate),
                        dtype=torch.int8 if i8 else torch.float32, device="cuda")
    A, D, sc = _prefill(L, torch, c, L0, p, h_dev)
    sh = H.shape_of(L, w, seqlen=1)
    t = L0
    x = H.to_dev(_step(c.ev["x"], t), w.dtype)
    dt = H.to_dev(_step(c.ev["dt"], t), w.dtype)
    B = H.to_dev(_step(c.ev["B"], t), w.dtype)
    C = H.to_dev(_step(c.ev["C"], t), w.dtype)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    ref = h_dev.clone()
    st = h_dev.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        L.ssd_decode_step(sh, p, x, dt, A, B, C, D, sc, st.clone(), y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            L.ssd_decode_step(sh, p, x, dt, A, B, C, D, sc, st, y)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for _ in range(3):
            L.ssd_decode_step(sh, p, x, dt, A, B, C, D, sc, ref, y)
        torch.cuda.synchronize()
        assert torch.equal(st, ref), rep
        _ = (ref.float() * 2).sum().item()  # eager work between the replays
