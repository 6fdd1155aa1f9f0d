"""Shared test helpers: seeded cases, device upload, oracle runs, metrics."""
from __future__ import annotations

import dataclasses

import numpy as np

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O

# Parity cases the oracle finishes in seconds. Each spans several MFMA tiles;
# most have a ragged last chunk (L % l != 0).
CASES = {
    "w0": synth.WORKLOADS[0],
    "f16_ragged": synth.Workload(11, 2, 640, 8, 64, 128, 2, 256, "fp16", True),
    "bf16_l128": synth.Workload(12, 1, 300, 4, 32, 64, 1, 128, "bf16", True),
    "f16_g_eq_h": synth.Workload(13, 1, 200, 4, 16, 32, 4, 64, "fp16", False),
    "f32_l256": synth.Workload(14, 1, 512, 2, 64, 128, 1, 256, "fp32", True),
    "bf16_n64_l128": synth.Workload(15, 2, 700, 6, 64, 64, 2, 128, "bf16", True),
    "f16_l128": synth.Workload(16, 1, 384, 3, 64, 128, 1, 128, "fp16", True),
}


@dataclasses.dataclass
class Case:
    w: synth.Workload
    consts: dict
    ev: dict          # stored arrays
    ev64: dict        # float64 widenings
    scales: dict      # oracle scale pack (float32 arrays)


def make_case(w: synth.Workload, batch=None, seqlen=None, cal_seqlen=None) -> Case:
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts, batch=batch, seqlen=seqlen)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, consts, seqlen=cal_seqlen)]
    am = O.calibrate(cal, consts["A"], w.ngroups, w.chunk)
    sc = O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads)
    return Case(w, consts, ev, synth.as_f64(ev, w.dtype), sc)


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def dev_inputs(case: Case) -> dict:
    import torch
    d = {k: to_dev(v, case.w.dtype) for k, v in case.ev.items()}
    d["A"] = torch.from_numpy(case.consts["A"]).cuda()
    d["D"] = torch.from_numpy(case.consts["D"]).cuda()
    return d


# INT8 forward schedules the parity tests run (by name -> SSD_SCHED_* value).
SCHEDULES = {"head": 1, "chunk": 2}


def shape_of(L, w: synth.Workload, batch=None, seqlen=None, schedule=0):
    sched = SCHEDULES[schedule] if isinstance(schedule, str) else schedule
    return L.make_shape(w.batch if batch is None else batch, w.seqlen if seqlen is None else seqlen,
                        w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype, sched)


def torch_dtype(dtype: str):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def f64(t) -> np.ndarray:
    """Device tensor -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


_MANT = {"fp32": 23, "fp16": 10, "bf16": 7}
_EMIN = {"fp32": -126, "fp16": -14, "bf16": -126}


def half_ulp(y, dtype: str) -> np.ndarray:
    """Half a unit in the last place of |y| in the storage type (the largest
    error of one round-to-nearest into that type)."""
    a = np.abs(np.asarray(y, np.float64))
    e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), _EMIN[dtype])
    e = np.maximum(e, _EMIN[dtype])
    return np.ldexp(0.5, (e - _MANT[dtype]).astype(np.int64))


def chan_err(y, ref, dtype: str | None = None) -> float:
    """max over channels (h, p) of max_{b,t} |y - ref| / RMS_{b,t}(ref).

    With ``dtype`` (the type y is stored in), each element's final rounding
    into that type is allowed for: the error counted is
    max(|y - ref| - half_ulp(y), 0), which is at most the error of the
    float32 value before that rounding."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=(0, 1)))
    d = np.abs(y - ref)
    if dtype is not None:
        d = np.maximum(d - half_ulp(y, dtype), 0.0)
    err = np.max(d, axis=(0, 1))
    return float(np.max(err / np.maximum(rms, 1e-30)))


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def bits(t):
    """A device or host tensor's stored bits, for bitwise comparison (NaN included)."""
    import torch
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])
