"""GPU parity of the SSD epilogue calls against the oracle (R17, R18).

The float and INT8 paths' outputs of one forward give the quantised output
Y_q and its reference Y_ref; ssd_mean_correction forms c* from them and
ssd_epilogue applies RMSNorm(Y_q + 0.15 c*) * weight. The oracle does the same
on the same stored values in float64: c* within float32 rounding, the
normalised output within half an ulp of its storage type plus 1e-5 relative.
"""
import numpy as np
import pytest

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O
from tests import _helpers as H

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _forward_pair(L, torch, name):
    c = H.make_case(H.CASES[name])
    d = H.dev_inputs(c)
    sh = H.shape_of(L, c.w)
    yf = torch.empty_like(d["x"])
    yq = torch.empty_like(d["x"])
    L.ssd_forward(sh, L.SSD_PATH_FLOAT, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, yf)
    L.ssd_forward(sh, L.SSD_PATH_INT8, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                  L.ScalePack(c.scales), yq)
    return c, sh, yf, yq


def _elem_ok(out, ref, dtype):
    err = np.abs(out - ref) - H.half_ulp(out, dtype)
    return float(np.max(err / (1e-5 * np.abs(ref) + 1e-6)))


@pytest.mark.parametrize("name", ["w0", "f16_ragged", "bf16_l128", "f32_l256", "bf16_n64_l128"])
def test_mean_correction_and_epilogue(gpu_lib, name):
    import torch
    L = gpu_lib
    print(f"epilogue {name}", flush=True)
    c, sh, yf, yq = _forward_pair(L, torch, name)
    w = c.w
    cg = torch.empty((w.nheads, w.headdim), dtype=torch.float32, device="cuda")
    L.ssd_mean_correction(sh, yf, yq, cg)
    wt = torch.from_numpy(synth.norm_weight(w)).cuda()
    out = torch.empty_like(yq)
    L.ssd_epilogue(sh, yq, cg, L.MEAN_CORRECTION_ALPHA, wt, EPS, out)
    torch.cuda.synchronize()
    yf64, yq64 = H.f64(yf), H.f64(yq)
    cref = O.mean_correction(yf64, yq64)
    cgn = cg.cpu().numpy().astype(np.float64)
    assert np.abs(cgn - cref).max() <= 1e-6 * np.abs(cref).max() + 1e-12
    # the epilogue itself, from the library's c (float32 values)
    ref = O.epilogue(yq64, cgn, O.MEAN_CORRECTION_ALPHA, synth.norm_weight(w), EPS)
    assert _elem_ok(H.f64(out), ref, w.dtype) <= 1.0
    # without a correction, and in place
    ref0 = O.epilogue(yq64, None, 0.0, synth.norm_weight(w), EPS)
    L.ssd_epilogue(sh, yq, None, 0.0, wt, EPS, yq)
    torch.cuda.synchronize()
    assert _elem_ok(H.f64(yq), ref0, w.dtype) <= 1.0


@pytest.mark.timeout(600)
def test_epilogue_layer_shape(gpu_lib):
    """The 2.7B-shaped layer (batch 8, L 2048, H*P = 5120, fp16): sampled
    positions of the benchmark's configuration."""
    import torch
    L = gpu_lib
    w = synth.WORKLOADS[2]
    print("epilogue layer shape", flush=True)
    ev = synth.evaluation_batch(w, synth.layer_constants(w))
    y = torch.from_numpy(ev["x"]).cuda()      # an fp16 tensor of the output's shape and spread
    sh = L.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
    rng = np.random.default_rng(5)
    corr = (0.05 * rng.standard_normal((w.nheads, w.headdim))).astype(np.float32)
    wt = synth.norm_weight(w)
    out = torch.empty_like(y)
    L.ssd_epilogue(sh, y, torch.from_numpy(corr).cuda(), L.MEAN_CORRECTION_ALPHA,
                   torch.from_numpy(wt).cuda(), EPS, out)
    torch.cuda.synchronize()
    rows = [(0, 0), (0, w.seqlen - 1), (w.batch - 1, 17), (w.batch // 2, w.seqlen // 2)]
    y64 = synth.as_f64({"x": ev["x"]}, w.dtype)["x"]
    for b, t in rows:
        ref = O.epilogue(y64[b:b + 1, t:t + 1], corr, O.MEAN_CORRECTION_ALPHA, wt, EPS)
        assert _elem_ok(H.f64(out[b:b + 1, t:t + 1]), ref, w.dtype) <= 1.0, (b, t)


@pytest.mark.parametrize("dtype,nh,hp,nb,nl", [("fp16", 8, 64, 1, 37), ("bf16", 16, 64, 2, 45),
                                                ("fp16", 48, 64, 1, 300), ("bf16", 80, 64, 1, 33),
                                                ("fp16", 96, 64, 3, 7)])
def test_epilogue_wave_rows(gpu_lib, dtype, nh, hp, nb, nl):
    """Row widths of 512 * V channels (V = 1, 2, 6, 10, 12) take the wave-per-row
    kernel: every row against the oracle, with and without a correction, row
    counts that leave the last workgroup's waves partly idle."""
    import torch
    L = gpu_lib
    print(f"epilogue wave rows {dtype} H={nh} P={hp} B={nb} L={nl}", flush=True)
    rng = np.random.default_rng(11 + nh)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    y = torch.from_numpy(rng.standard_normal((nb, nl, nh, hp)).astype(np.float32)).to(tdt).cuda()
    corr = (0.05 * rng.standard_normal((nh, hp))).astype(np.float32)
    wt = (1.0 + 0.1 * rng.standard_normal((nh, hp))).astype(np.float32)
    sh = L.make_shape(nb, nl, nh, hp, 16, 1, 64, dtype)
    y64 = H.f64(y)
    for c in (corr, None):
        alpha = L.MEAN_CORRECTION_ALPHA if c is not None else 0.0
        out = torch.empty_like(y)
        L.ssd_epilogue(sh, y, None if c is None else torch.from_numpy(c).cuda(), alpha,
                       torch.from_numpy(wt).cuda(), EPS, out)
        torch.cuda.synchronize()
        ref = O.epilogue(y64, c, alpha, wt, EPS)
        assert _elem_ok(H.f64(out), ref, dtype) <= 1.0, (dtype, nh, c is None)
