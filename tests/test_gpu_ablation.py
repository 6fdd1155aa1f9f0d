"""GPU parity of the two Table 5 ablation rows run by ssd_forward
(SSD_PATH_ABL_QX "Q(X) only", SSD_PATH_ABL_RECON "reconstruction + B,C
quantisation") against the oracle's forward_qx and forward_recon.

Both rows carry floating-point states, so their outputs are checked within
tolerance: Q(X) only against its float64 oracle at the float path's bar (2e-2
of the channel RMS; the Q(X) codes themselves bit for bit, read back from Y with
C = 0 and D = 1, where Y is Q(X) s_Xq rounded once), the recon row at the INT8 bar (5e-2; its ChunkScan1 quantises an fp32 state whose
last bits differ from the oracle's float64 one).
"""
import functools

import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

NAMES = ["w0", "f16_ragged", "bf16_l128", "f16_g_eq_h", "f32_l256", "bf16_n64_l128"]


@functools.lru_cache(maxsize=None)
def case(name):
    c = H.make_case(H.CASES[name])
    cal = [synth.as_f64(s, c.w.dtype) for s in synth.calibration_sequences(c.w, c.consts)]
    sx = O.scale_pack_x(O.calibrate_x(cal))
    sc = dict(c.scales)
    sc.update(sx)
    return c, sc


def _run(L, torch, c, sc, path):
    d = H.dev_inputs(c)
    sh = H.shape_of(L, c.w)
    y = torch.empty_like(d["x"])
    w = c.w
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    L.ssd_forward(sh, path, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], L.ScalePack(sc), y,
                  final_state=fin)
    torch.cuda.synchronize()
    return y, fin


@pytest.mark.parametrize("name", NAMES)
def test_ablation_qx_only(gpu_lib, name):
    import torch
    L = gpu_lib
    c, sc = case(name)
    e = c.ev64
    print(f"ablation Q(X) only {name}", flush=True)
    r = O.forward_qx(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], sc["inv_Xq"],
                     sc["s_Xq"], c.w.chunk)
    y, fin = _run(L, torch, c, sc, L.SSD_PATH_ABL_QX)
    err = H.chan_err(H.f64(y), r["y"], c.w.dtype)
    assert err <= 2e-2, err
    hf = r["final"]
    assert np.abs(fin.cpu().numpy() - hf).max() <= 2e-1 * np.sqrt(np.mean(hf * hf))


@pytest.mark.parametrize("name", ["f16_ragged", "bf16_l128", "f32_l256"])
def test_ablation_qx_codes(gpu_lib, name):
    """With C = 0 and D = 1 the output is the dequantised input itself,
    Y = Q(X) s_Xq rounded once into the storage type; |Q(X)| <= 127 needs 7
    bits, which even bf16's 8-bit significand keeps, so rint(Y / s_Xq) gives
    back every code, and they must equal the oracle's Q(X) bit for bit."""
    import torch
    L = gpu_lib
    c, sc = case(name)
    w = c.w
    print(f"ablation Q(X) codes {name}", flush=True)
    d = H.dev_inputs(c)
    d["C"] = torch.zeros_like(d["C"])
    d["D"] = torch.ones_like(d["D"])
    y = torch.empty_like(d["x"])
    L.ssd_forward(H.shape_of(L, w), L.SSD_PATH_ABL_QX, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                  L.ScalePack(sc), y)
    torch.cuda.synchronize()
    r = O.forward_qx(c.ev64["x"], c.ev64["dt"], c.consts["A"], c.ev64["B"], np.zeros_like(c.ev64["C"]),
                     np.ones_like(c.consts["D"]), sc["inv_Xq"], sc["s_Xq"], w.chunk)
    s_xq = np.asarray(sc["s_Xq"], np.float64).reshape(w.nheads, w.headdim)
    codes = np.rint(H.f64(y) / s_xq[None, None])
    assert np.array_equal(codes, r["qx"].astype(np.float64))
    assert np.abs(r["qx"]).max() > 64  # the codes span most of the int8 range


@pytest.mark.parametrize("name", NAMES)
def test_ablation_recon(gpu_lib, name):
    import torch
    L = gpu_lib
    c, sc = case(name)
    e = c.ev64
    print(f"ablation recon {name}", flush=True)
    r = O.forward_recon(e["x"], e["dt"], c.consts["A"], e["B"], e["C"], c.consts["D"], sc, c.w.chunk)
    y, fin = _run(L, torch, c, sc, L.SSD_PATH_ABL_RECON)
    err = H.chan_err(H.f64(y), r["y"], c.w.dtype)
    assert err <= 5e-2, err
    hf = r["passed"][:, -1]
    assert np.abs(fin.cpu().numpy() - hf).max() <= 1e-3 * np.abs(hf).max()
