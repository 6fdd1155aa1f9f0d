"""ssd_forward_noalloc (the forward on the library's fixed device workspace)
against ssd_forward on a caller-allocated workspace: two calls in a row, the
second with a smaller input, on both paths and both INT8 schedules. The
outputs (Y, final state, every INT8 tap) must equal ssd_forward's bit for bit,
which is stricter than the parity bar both are held to against the oracle."""
import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

BIG = synth.Workload(31, 2, 700, 8, 64, 128, 2, 256, "fp16", True)
SMALL = synth.Workload(32, 1, 300, 4, 64, 128, 2, 256, "fp16", True)
BIG_BF16 = synth.Workload(33, 2, 520, 6, 64, 64, 1, 128, "bf16", True)
SMALL_BF16 = synth.Workload(34, 1, 130, 6, 64, 64, 1, 128, "bf16", True)


def _inputs(L, w):
    import torch
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts)]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    sc = L.ScalePack(O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads))
    d = {k: H.to_dev(v, w.dtype) for k, v in ev.items()}
    d["A"] = torch.from_numpy(consts["A"]).cuda()
    d["D"] = torch.from_numpy(consts["D"]).cuda()
    return d, sc


def _outputs(torch, w, d, i8):
    fdt = torch.int8 if i8 else torch.float32
    o = {"y": torch.full_like(d["x"], float("nan")),
         "fin": torch.zeros((w.batch, w.nheads, w.headdim, w.dstate), dtype=fdt, device="cuda")}
    if i8:
        st = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
        o["taps"] = {"q_xs": torch.zeros(d["x"].shape, dtype=torch.int8, device="cuda"),
                     "s32": torch.zeros(st, dtype=torch.int32, device="cuda"),
                     "s8_local": torch.zeros(st, dtype=torch.int8, device="cuda"),
                     "passed": torch.zeros(st, dtype=torch.int8, device="cuda")}
    return o


def _same(torch, a, b, what):
    assert torch.equal(H.bits(a["y"]), H.bits(b["y"])), f"{what}: Y"
    assert torch.equal(a["fin"], b["fin"]), f"{what}: final state"
    for k in a.get("taps", {}):
        assert torch.equal(a["taps"][k], b["taps"][k]), f"{what}: tap {k}"


@pytest.mark.parametrize("mode", ["int8-head", "int8-chunk", "int8-auto", "float"])
@pytest.mark.parametrize("pair", ["fp16", "bf16"])
def test_noalloc_matches_forward(gpu_lib, pair, mode):
    import torch
    L = gpu_lib
    i8 = mode != "float"
    path = L.SSD_PATH_INT8 if i8 else L.SSD_PATH_FLOAT
    sched = {"int8-head": 1, "int8-chunk": 2}.get(mode, 0)
    big, small = (BIG, SMALL) if pair == "fp16" else (BIG_BF16, SMALL_BF16)
    for w in (big, small):  # the second call is smaller; the array keeps the first call's bytes
        print(f"noalloc {pair} {mode} B={w.batch} L={w.seqlen} H={w.nheads}", flush=True)
        d, sc = _inputs(L, w)
        sh = H.shape_of(L, w, schedule=sched)
        assert L.ssd_workspace_bytes(sh, path) <= L.NOALLOC_SCRATCH_BYTES
        scp = sc if i8 else None
        ref = _outputs(torch, w, d, i8)
        L.ssd_forward(sh, path, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], scp, ref["y"],
                      final_state=ref["fin"], taps=ref.get("taps"))
        got = _outputs(torch, w, d, i8)
        L.ssd_forward_noalloc(sh, path, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], scp, got["y"],
                              final_state=got["fin"], taps=got.get("taps"))
        torch.cuda.synchronize()
        assert not torch.isnan(got["y"].float()).any()
        _same(torch, got, ref, f"{pair} {mode} {w.batch}x{w.seqlen}")


def test_noalloc_continues_a_sequence(gpu_lib):
    """initial_state through the allocation-free call: two halves (split at a
    chunk boundary) give bitwise the Y and final state of one ssd_forward."""
    import torch
    L = gpu_lib
    w = BIG
    d, sc = _inputs(L, w)
    for path in (L.SSD_PATH_INT8, L.SSD_PATH_FLOAT):
        i8 = path == L.SSD_PATH_INT8
        scp = sc if i8 else None
        ref = _outputs(torch, w, d, i8)
        L.ssd_forward(H.shape_of(L, w), path, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], scp, ref["y"],
                      final_state=ref["fin"])
        L1 = 2 * w.chunk
        part = lambda t, a_, b_: t[:, a_:b_].contiguous()  # noqa: E731
        y1 = torch.empty_like(part(d["x"], 0, L1))
        y2 = torch.empty_like(part(d["x"], L1, None))
        f1 = torch.empty_like(ref["fin"])
        f2 = torch.empty_like(ref["fin"])
        L.ssd_forward_noalloc(H.shape_of(L, w, seqlen=L1), path, part(d["x"], 0, L1), part(d["dt"], 0, L1),
                              d["A"], part(d["B"], 0, L1), part(d["C"], 0, L1), d["D"], scp, y1, final_state=f1)
        L.ssd_forward_noalloc(H.shape_of(L, w, seqlen=w.seqlen - L1), path, part(d["x"], L1, None),
                              part(d["dt"], L1, None), d["A"], part(d["B"], L1, None), part(d["C"], L1, None),
                              d["D"], scp, y2, final_state=f2, initial_state=f1)
        torch.cuda.synchronize()
        assert torch.equal(H.bits(torch.cat([y1, y2], dim=1)), H.bits(ref["y"])), path
        assert torch.equal(f2, ref["fin"]), path


def test_noalloc_rejects_a_problem_beyond_its_array(gpu_lib):
    """A problem whose workspace exceeds the array returns SSD_E_TOO_LARGE and
    writes nothing; the automatic schedule falls back to the head-persistent one
    when only the chunk-parallel workspace is too large."""
    import torch
    L = gpu_lib
    big = L.make_shape(4, 4096, 128, 64, 128, 8, 256, "bf16", L.SSD_SCHED_CHUNK)
    assert L.ssd_workspace_bytes(big, L.SSD_PATH_INT8) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.SSDError) as e:
        L.ssd_forward_noalloc(big, L.SSD_PATH_INT8, x, x, x, x, x, x, None, x)
    assert e.value.status == L.SSD_E_TOO_LARGE
    torch.cuda.synchronize()
    assert not x.any()


def test_noalloc_auto_falls_back_to_the_head_schedule(gpu_lib):
    """A long single sequence (B*H below twice the CU count, so the automatic
    choice is chunk-parallel) whose chunk-parallel workspace exceeds the array:
    the call runs the head-persistent schedule and equals ssd_forward on it bit
    for bit."""
    import torch
    L = gpu_lib
    B, T, Hh, P, N, G, l = 1, 65536, 80, 64, 128, 1, 256
    auto = L.make_shape(B, T, Hh, P, N, G, l, "fp16", L.SSD_SCHED_AUTO)
    head = L.make_shape(B, T, Hh, P, N, G, l, "fp16", L.SSD_SCHED_HEAD)
    chunk = L.make_shape(B, T, Hh, P, N, G, l, "fp16", L.SSD_SCHED_CHUNK)
    assert L.ssd_workspace_bytes(chunk, L.SSD_PATH_INT8) > L.NOALLOC_SCRATCH_BYTES
    assert L.ssd_workspace_bytes(head, L.SSD_PATH_INT8) <= L.NOALLOC_SCRATCH_BYTES
    print("noalloc auto fallback B=1 L=65536 H=80", flush=True)
    g = torch.Generator(device="cuda").manual_seed(35)
    x = torch.randn((B, T, Hh, P), generator=g, device="cuda").half()
    dt = (torch.rand((B, T, Hh), generator=g, device="cuda") * 0.099 + 0.001).half()
    Bm = torch.randn((B, T, G, N), generator=g, device="cuda").half()
    Cm = torch.randn((B, T, G, N), generator=g, device="cuda").half()
    A = -torch.rand(Hh, generator=g, device="cuda") * 4 - 0.5
    D = torch.rand(Hh, generator=g, device="cuda")
    amax = {"s_B": np.full(G, 4.5 / 127, np.float32), "s_C": np.full(G, 4.5 / 127, np.float32),
            "inv_B": np.full(G, 127 / 4.5, np.float32), "inv_C": np.full(G, 127 / 4.5, np.float32),
            "s_X": np.full(Hh * P, 0.5 / 127, np.float32), "inv_X": np.full(Hh * P, 127 / 0.5, np.float32),
            "s_S": np.full(Hh * P, 40.0 / 127, np.float32)}
    amax["M_req"] = (amax["s_X"].astype(np.float64) * amax["s_B"][0] / amax["s_S"]).astype(np.float32)
    sc = L.ScalePack(amax)
    y_ref = torch.empty_like(x)
    f_ref = torch.empty((B, Hh, P, N), dtype=torch.int8, device="cuda")
    L.ssd_forward(head, L.SSD_PATH_INT8, x, dt, A, Bm, Cm, D, sc, y_ref, final_state=f_ref)
    y = torch.full_like(x, float("nan"))
    fin = torch.zeros_like(f_ref)
    L.ssd_forward_noalloc(auto, L.SSD_PATH_INT8, x, dt, A, Bm, Cm, D, sc, y, final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(H.bits(y), H.bits(y_ref))
    assert torch.equal(fin, f_ref)
