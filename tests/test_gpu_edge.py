"""Edge cases of ssd_forward on the GPU against the oracle: degenerate decays,
the shortest sequences around a chunk boundary, and the empty problem.

Degenerate decays: heads with A = 0 (every decay is 1: Q(Decay) = 128, so Eq. 6
is the saturating prefix sum of the local states) and heads with A = -1e4
(every decay underflows to 0: Q(Decay) = 0, the passed state is the local one
and the output memoryless), beside ordinary heads. INT8 integers bit for bit,
outputs within the paths' tolerances (2e-2 float against float64, 5e-2 INT8
against the INT8 method).
"""
import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu


def _run_both(L, torch, w, consts, ev, sched=0):
    e = synth.as_f64(ev, w.dtype)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts, seqlen=max(w.seqlen, 64))]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    sc = O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads)
    r8 = O.forward_int8(e["x"], e["dt"], consts["A"], e["B"], e["C"], consts["D"], sc, w.chunk)
    yf = O.chunked(e["x"], e["dt"], consts["A"], e["B"], e["C"], consts["D"], w.chunk)[0]
    d = {k: H.to_dev(v, w.dtype) for k, v in ev.items()}
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    sh = H.shape_of(L, w, schedule=sched)
    y8 = torch.empty_like(d["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    stshape = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
    taps = {"passed": torch.empty(stshape, dtype=torch.int8, device="cuda")}
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], A, d["B"], d["C"], D, L.ScalePack(sc), y8,
                  final_state=fin, taps=taps)
    y32 = torch.empty_like(d["x"])
    L.ssd_forward(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], A, d["B"], d["C"], D, None, y32)
    torch.cuda.synchronize()
    return r8, yf, y8, fin, taps, y32


@pytest.mark.parametrize("sched", list(H.SCHEDULES))
@pytest.mark.parametrize("name", ["f16_ragged", "w0", "bf16_n64_l128"])
def test_degenerate_decays(gpu_lib, name, sched):
    import torch
    L = gpu_lib
    w = H.CASES[name]
    print(f"degenerate decays {name} {sched}", flush=True)
    consts = synth.layer_constants(w)
    A = consts["A"].copy()
    A[0] = 0.0
    A[-1] = -1e4
    consts = dict(consts, A=A)
    ev = synth.evaluation_batch(w, consts)
    r8, yf, y8, fin, taps, y32 = _run_both(L, torch, w, consts, ev, sched)
    qd = r8["cumsum"]["qdecay"]
    assert (qd[:, 0] == 128).all() and (qd[:, -1] == 0).all()
    assert np.array_equal(taps["passed"].cpu().numpy(), r8["passed"])
    assert np.array_equal(fin.cpu().numpy(), r8["passed"][:, -1])
    assert H.chan_err(H.f64(y8), r8["y"], w.dtype) <= 5e-2
    assert H.chan_err(H.f64(y32), yf, w.dtype) <= 2e-2


@pytest.mark.parametrize("sched", list(H.SCHEDULES))
@pytest.mark.parametrize("seqlen", [1, 17, 255, 256, 257])
def test_short_sequences(gpu_lib, seqlen, sched):
    """One position, a partial chunk, exactly one chunk, one past it (the
    fused kernels at chunk 256)."""
    import torch
    L = gpu_lib
    w = H.CASES["f16_ragged"].replace(seqlen=seqlen)
    print(f"short sequence L={seqlen} {sched}", flush=True)
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts)
    r8, yf, y8, fin, taps, y32 = _run_both(L, torch, w, consts, ev, sched)
    assert np.array_equal(taps["passed"].cpu().numpy(), r8["passed"])
    assert np.array_equal(fin.cpu().numpy(), r8["passed"][:, -1])
    assert H.chan_err(H.f64(y8), r8["y"], w.dtype) <= 5e-2
    assert H.chan_err(H.f64(y32), yf, w.dtype) <= 2e-2


def test_empty_problem_writes_nothing(gpu_lib):
    import torch
    L = gpu_lib
    w = H.CASES["f16_ragged"]
    for batch, seqlen in ((0, 640), (2, 0)):
        sh = L.make_shape(batch, seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
        buf = torch.full((64,), 7.0, dtype=torch.float16, device="cuda")
        A = torch.zeros(w.nheads, dtype=torch.float32, device="cuda")
        for path in (L.SSD_PATH_FLOAT, L.SSD_PATH_INT8):
            sc = L.ScalePack({k: np.ones(1024, np.float32) for k in L.ScalePack.ORDER})
            L.ssd_forward(sh, path, buf, buf, A, buf, buf, A, sc, buf)
        torch.cuda.synchronize()
        assert bool((buf == 7.0).all())


def test_zero_length_carries_the_state(gpu_lib):
    """seqlen 0 with batch > 0: no position is processed, so the final state is
    the initial state (zeros without one), for ssd_forward and
    ssd_state_passing on both paths; Y is not touched."""
    import torch
    L = gpu_lib
    w = H.CASES["f16_ragged"]
    nb = 2
    sh = L.make_shape(nb, 0, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
    n = (nb, w.nheads, w.headdim, w.dstate)
    rng = np.random.default_rng(5)
    buf = torch.full((64,), 7.0, dtype=torch.float16, device="cuda")
    A = torch.zeros(w.nheads, dtype=torch.float32, device="cuda")
    sc = L.ScalePack({k: np.ones(1024, np.float32) for k in L.ScalePack.ORDER})
    for path, dt, ref in ((L.SSD_PATH_INT8, torch.int8, rng.integers(-127, 128, size=n).astype(np.int8)),
                          (L.SSD_PATH_FLOAT, torch.float32, rng.standard_normal(n).astype(np.float32))):
        init = torch.from_numpy(ref).cuda()
        for with_init in (True, False):
            expect = ref if with_init else np.zeros_like(ref)
            fin = torch.full(n, 5, dtype=dt, device="cuda")
            L.ssd_forward(sh, path, buf, buf, A, buf, buf, A, sc, buf, final_state=fin,
                          initial_state=init if with_init else None)
            torch.cuda.synchronize()
            assert np.array_equal(fin.cpu().numpy(), expect)
            fin2 = torch.full(n, 5, dtype=dt, device="cuda")
            L.ssd_state_passing(sh, path, buf, dAcs=A, qdecay=buf, initial_state=init if with_init else None,
                                final_state=fin2)
            torch.cuda.synchronize()
            assert np.array_equal(fin2.cpu().numpy(), expect)
    assert bool((buf == 7.0).all())


@pytest.mark.parametrize("name", ["f16_ragged", "bf16_n64_l128", "w0"])
def test_forward_replayed_from_a_graph(gpu_lib, name):
    """ssd_forward captured in one HIP graph (workspace allocated before the
    capture) and replayed three times, with an eager forward on other buffers
    and a synchronisation between the replays: every replay's Y and final state
    equal an eager call's bit for bit, on both paths (the fused kernels for the
    fp16 and bf16 cases, the module kernels for the fp32 one)."""
    import torch
    L = gpu_lib
    w = H.CASES[name]
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts, seqlen=max(w.seqlen, 64))]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    sc = L.ScalePack(O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads))
    d = {k: H.to_dev(v, w.dtype) for k, v in ev.items()}
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    n = (w.batch, w.nheads, w.headdim, w.dstate)
    for path, sched in ((L.SSD_PATH_INT8, "head"), (L.SSD_PATH_INT8, "chunk"), (L.SSD_PATH_FLOAT, 0)):
        sh = H.shape_of(L, w, schedule=sched)
        i8 = path == L.SSD_PATH_INT8
        scp = sc if i8 else None
        fdt = torch.int8 if i8 else torch.float32
        nws = max(1, L.ssd_workspace_bytes(sh, path))

        def fwd(y, fin, ws):
            L.ssd_forward(sh, path, d["x"], d["dt"], A, d["B"], d["C"], D, scp, y, final_state=fin, workspace=ws)

        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        y_ref, f_ref = torch.empty_like(d["x"]), torch.empty(n, dtype=fdt, device="cuda")
        fwd(y_ref, f_ref, ws)
        torch.cuda.synchronize()
        y, fin = torch.zeros_like(d["x"]), torch.zeros(n, dtype=fdt, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd(y, fin, ws)
        y_e, f_e = torch.empty_like(d["x"]), torch.empty(n, dtype=fdt, device="cuda")
        ws_e = torch.empty(nws, dtype=torch.uint8, device="cuda")
        for rep in range(3):
            y.zero_()
            fin.zero_()
            g.replay()
            fwd(y_e, f_e, ws_e)  # eager work between the replays
            torch.cuda.synchronize()
            assert torch.equal(H.bits(y), H.bits(y_ref)), (path, sched, rep)
            assert torch.equal(H.bits(fin), H.bits(f_ref)), (path, sched, rep)
            assert torch.equal(H.bits(y_e), H.bits(y_ref)), (path, sched, rep)
        del g
