"""GPU parity of the fused kernels' whole-head workgroups at every chunk length
and state size they cover.

With 128 < B*H < 256 heads on 256 CUs the launcher runs every head as one
workgroup (no p-half split), so these shapes take the whole-head code path
(all four 16-wide p tiles per workgroup) at l = 128 and N = 64, which the
other cases reach only through the half-head path. The INT8 cases run under
both schedules (head-persistent and chunk-parallel). INT8: every tap (Q(Xs),
S32, S8, passed states) bit-exact against the oracle, the final state too, Y
within 5e-2 and within its rounding budget; float: Y within 2e-2 of the
float64 definition, the final state within 1e-2 of each channel's RMS, both
within their rounding budgets.
"""
import functools

import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

SHAPES = {
    "f16_l128_n128": synth.Workload(21, 2, 300, 80, 64, 128, 2, 128, "fp16", True),
    "bf16_l128_n64": synth.Workload(22, 2, 260, 72, 64, 64, 1, 128, "bf16", True),
    "f16_l256_n64": synth.Workload(23, 2, 520, 80, 64, 64, 2, 256, "fp16", True),
}


@functools.lru_cache(maxsize=None)
def _case(name):
    c = H.make_case(SHAPES[name])
    e = c.ev64
    r8 = O.forward_int8(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], c.scales,
                        c.w.chunk)
    yf, hf, _, _ = O.chunked(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], c.w.chunk)
    return c, r8, yf, hf


@pytest.mark.parametrize("sched", list(H.SCHEDULES))
@pytest.mark.parametrize("name", list(SHAPES))
def test_whole_head_int8(gpu_lib, name, sched):
    import torch
    L = gpu_lib
    print(f"whole-head int8 {name} {sched}", flush=True)
    c, r8, _, _ = _case(name)
    w = c.w
    assert 128 < w.batch * w.nheads < 256
    d = H.dev_inputs(c)
    sh = H.shape_of(L, w, schedule=sched)
    y = torch.empty_like(d["x"])
    stshape = (w.batch, w.nchunks, w.nheads, w.headdim, w.dstate)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.int8, device="cuda")
    taps = {"q_xs": torch.empty(d["x"].shape, dtype=torch.int8, device="cuda"),
            "s32": torch.empty(stshape, dtype=torch.int32, device="cuda"),
            "s8_local": torch.empty(stshape, dtype=torch.int8, device="cuda"),
            "passed": torch.empty(stshape, dtype=torch.int8, device="cuda")}
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                  L.ScalePack(c.scales), y, final_state=fin, taps=taps)
    torch.cuda.synchronize()
    assert np.array_equal(taps["q_xs"].cpu().numpy(), r8["qxs"])
    assert np.array_equal(taps["s32"].cpu().numpy(), r8["s32"])
    assert np.array_equal(taps["s8_local"].cpu().numpy(), r8["s8"])
    assert np.array_equal(taps["passed"].cpu().numpy(), r8["passed"])
    assert np.array_equal(fin.cpu().numpy(), r8["passed"][:, -1])
    e = c.ev64
    err = H.chan_err(H.f64(y), r8["y"], w.dtype)
    bud = H.int8_budget(H.f64(y), r8, e["x"], e["dt"], c.consts["D"], c.scales, w.chunk, w.dtype)
    H.report(f"whole-head int8 {name} {sched}", chan_err=err, budget=bud)
    assert err <= 5e-2
    assert bud <= 1.0
    # the instantiation without taps gives the same output and final state
    y2 = torch.empty_like(y)
    fin2 = torch.empty_like(fin)
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                  L.ScalePack(c.scales), y2, final_state=fin2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(fin, fin2)


@pytest.mark.parametrize("name", list(SHAPES))
def test_whole_head_float(gpu_lib, name):
    import torch
    L = gpu_lib
    print(f"whole-head float {name}", flush=True)
    c, _, yf, hf = _case(name)
    w = c.w
    d = H.dev_inputs(c)
    sh = H.shape_of(L, w)
    y = torch.empty_like(d["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    L.ssd_forward(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, y,
                  final_state=fin)
    torch.cuda.synchronize()
    e = c.ev64
    fg = fin.cpu().numpy().astype(np.float64)
    err = H.chan_err(H.f64(y), yf, w.dtype)
    serr = H.state_chan_err(fg, hf)
    by, bh = H.float_budget(H.f64(y), fg, e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"],
                            w.chunk, w.dtype, yf, hf)
    H.report(f"whole-head float {name}", chan_err=err, state_chan_err=serr, budget_y=by, budget_state=bh)
    assert err <= 2e-2
    assert serr <= 1e-2
    assert by <= 1.0 and bh <= 1.0
