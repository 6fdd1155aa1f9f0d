"""Parity at the full layer sizes: the Mamba-2 1.3B-, 2.7B- and 8B-shaped
layers (the 8B one with bf16 and with fp16 inputs) and the 65,536-token
long-context layer.

ssd_forward runs once over the whole layer through the same call and launch
configuration the benchmark times (caller workspace, no taps). A second call
with the debug taps must give bitwise the same Y and final state. The oracle
then recomputes (batch, head) pairs from the raw inputs, with the static scales
it calibrated itself on the two full-length calibration sequences: every head
of the first and the last sequence on the 2.7B- and 1.3B-shaped layers (all
XCD slots, whole-head and split-head workgroups), sampled heads on the larger
layers. On those heads:
  INT8   Q(Xs), S32, local S8, the passed states (all chunks: 256 of them on
         the long-context layer) and the final state bit for bit; Y within the
         INT8 bar (5e-2 per channel) and within its rounding budget (the
         per-element bound from the kernels' own operand roundings);
  float  Y within 2e-2 per channel of the float64 definition, the fp32 final
         state within 1e-2 of each channel's own RMS, both within their
         rounding budgets.
Each case prints its measured errors: the per-channel metric, the global
max|err| / RMS and the budget ratio (<= 1 passes).
"""
import functools

import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = {"1": synth.WORKLOADS[1], "2": synth.WORKLOADS[2], "3": synth.WORKLOADS[3],
        "3-fp16": synth.WORKLOADS[3].replace(dtype="fp16"), "4": synth.WORKLOADS[4]}
# every head of these sequences; sampled heads elsewhere
ALL_HEADS = {"1": (0,), "2": (0, 7)}
_GROUP_KEYS = ("s_B", "s_C", "inv_B", "inv_C")
_HEAD_KEYS = ("s_X", "inv_X", "s_S", "M_req")


@functools.lru_cache(maxsize=2)
def full_case(key):
    w = FULL[key]
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts)]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    del cal
    sc = O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads)
    return w, consts, ev, sc


def units(key, w, consts):
    """(batch, heads) units the oracle recomputes: all heads of the listed
    sequences, or the first and last heads, the head holding the largest X
    channel scale (an outlier channel) and one in the middle, of the first
    and last sequence."""
    if key in ALL_HEADS:
        return [(b, list(range(w.nheads))) for b in ALL_HEADS[key]]
    hmax = int(np.argmax(consts["xscale"].max(axis=1)))
    heads = sorted({0, w.nheads // 2 + 1, hmax, w.nheads - 1})
    return [(b, [h]) for b in sorted({0, w.batch - 1}) for h in heads]


def unit_inputs(w, consts, ev, sc, b, heads):
    """Oracle inputs of sequence b restricted to `heads` (a contiguous range
    of whole groups, or one head with its group)."""
    hpg = w.nheads // w.ngroups
    h0, h1 = heads[0], heads[-1] + 1
    g0, g1 = h0 // hpg, (h1 - 1) // hpg + 1
    assert len(heads) == 1 or (h0 % hpg == 0 and h1 % hpg == 0)
    e = {k: synth.to_f64(v[b:b + 1], w.dtype) for k, v in ev.items()}
    x, dt = e["x"][:, :, h0:h1], e["dt"][:, :, h0:h1]
    Bm, Cm = e["B"][:, :, g0:g1], e["C"][:, :, g0:g1]
    s1 = {"bits": sc["bits"]}
    s1.update({k: sc[k][g0:g1] for k in _GROUP_KEYS})
    s1.update({k: sc[k][h0:h1] for k in _HEAD_KEYS})
    return x, dt, consts["A"][h0:h1], Bm, Cm, consts["D"][h0:h1], s1


def _run(L, torch, w, consts, ev, sc, path):
    print(f"full-size {path} forward: {w.name}", flush=True)
    d = {k: H.to_dev(v, w.dtype) for k, v in ev.items()}
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    sh = H.shape_of(L, w)
    int8 = path == "int8"
    p = L.SSD_PATH_INT8 if int8 else L.SSD_PATH_FLOAT
    scales = L.ScalePack(sc) if int8 else None
    ws = torch.empty(max(1, L.ssd_workspace_bytes(sh, p)), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    fdt = torch.int8 if int8 else torch.float32
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=fdt, device="cuda")
    L.ssd_forward(sh, p, d["x"], d["dt"], A, d["B"], d["C"], D, scales, y, final_state=fin,
                  workspace=ws)
    torch.cuda.synchronize()
    return d, A, D, sh, p, scales, ws, y, fin


class _Worst:
    """Largest value of each metric over the units of a case."""

    def __init__(self):
        self.m = {}
        self.num = 0.0   # global max |err|
        self.den = []    # squares of the reference, for the global RMS

    def add(self, **kw):
        for k, v in kw.items():
            self.m[k] = max(self.m.get(k, 0.0), v)

    def add_global(self, y, ref):
        self.num = max(self.num, float(np.abs(y - ref).max()))
        self.den.append(float(np.mean(ref * ref)))

    def report(self, tag):
        H.report(tag, global_err=self.num / np.sqrt(np.mean(self.den)), **self.m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", list(FULL))
def test_full_size_int8(gpu_lib, key):
    import torch
    L = gpu_lib
    w, consts, ev, sc = full_case(key)
    d, A, D, sh, p, scales, ws, y, fin = _run(L, torch, w, consts, ev, sc, "int8")
    stshape = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
    taps = {"q_xs": torch.empty(d["x"].shape, dtype=torch.int8, device="cuda"),
            "s32": torch.empty(stshape, dtype=torch.int32, device="cuda"),
            "s8_local": torch.empty(stshape, dtype=torch.int8, device="cuda"),
            "passed": torch.empty(stshape, dtype=torch.int8, device="cuda")}
    y2 = torch.empty_like(y)
    fin2 = torch.empty_like(fin)
    L.ssd_forward(sh, p, d["x"], d["dt"], A, d["B"], d["C"], D, scales, y2, final_state=fin2,
                  workspace=ws, taps=taps)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(fin, fin2)
    worst = _Worst()
    for b, heads in units(key, w, consts):
        hs = slice(heads[0], heads[-1] + 1)
        x, dt, Ah, Bm, Cm, Dh, s1 = unit_inputs(w, consts, ev, sc, b, heads)
        r = O.forward_int8(x, dt, Ah, Bm, Cm, Dh, s1, w.chunk)
        assert np.array_equal(taps["q_xs"][b:b + 1, :, hs].cpu().numpy(), r["qxs"]), (b, heads)
        assert np.array_equal(taps["s32"][b:b + 1, :, hs].cpu().numpy(), r["s32"]), (b, heads)
        assert np.array_equal(taps["s8_local"][b:b + 1, :, hs].cpu().numpy(), r["s8"]), (b, heads)
        assert np.array_equal(taps["passed"][b:b + 1, :, hs].cpu().numpy(), r["passed"]), (b, heads)
        assert np.array_equal(fin[b:b + 1, hs].cpu().numpy(), r["passed"][:, -1]), (b, heads)
        yg = H.f64(y[b:b + 1, :, hs])
        err = H.chan_err(yg, r["y"], w.dtype)
        bud = H.int8_budget(yg, r, x, dt, Dh, s1, w.chunk, w.dtype)
        worst.add(chan_err=err, budget=bud)
        worst.add_global(yg, r["y"])
        assert err <= 5e-2, (b, heads, err)
        assert bud <= 1.0, (b, heads, bud)
    worst.report(f"full-size int8 {key} {w.name}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", list(FULL))
def test_full_size_float(gpu_lib, key):
    import torch
    L = gpu_lib
    w, consts, ev, sc = full_case(key)
    d, A, D, sh, p, scales, ws, y, fin = _run(L, torch, w, consts, ev, sc, "float")
    worst = _Worst()
    for b, heads in units(key, w, consts):
        hs = slice(heads[0], heads[-1] + 1)
        x, dt, Ah, Bm, Cm, Dh, _ = unit_inputs(w, consts, ev, sc, b, heads)
        yf, hf = O.chunked(x, dt, Ah, Bm, Cm, Dh, w.chunk)[:2]
        yg = H.f64(y[b:b + 1, :, hs])
        fg = fin[b:b + 1, hs].cpu().numpy().astype(np.float64)
        err = H.chan_err(yg, yf, w.dtype)
        serr = H.state_chan_err(fg, hf)
        by, bh = H.float_budget(yg, fg, x, dt, Ah, Bm, Cm, Dh, w.chunk, w.dtype, yf, hf)
        worst.add(chan_err=err, state_chan_err=serr, budget_y=by, budget_state=bh)
        worst.add_global(yg, yf)
        assert err <= 2e-2, (b, heads, err)
        assert serr <= 1e-2, (b, heads, serr)
        assert by <= 1.0 and bh <= 1.0, (b, heads, by, bh)
    worst.report(f"full-size float {key} {w.name}")
