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
    # the preparation launch's block kinds for many (batch, chunk, group)
    # units: two blocks per unit for 32 .. CUs / 2 units (80 and 48 units, at
    # l = 128 and at N = 64), one block per unit above that (144 units)
    "bf16_units_l128": synth.Workload(17, 4, 520, 8, 64, 64, 4, 128, "bf16", True),
    "f16_units_n64": synth.Workload(18, 4, 600, 8, 64, 64, 4, 256, "fp16", True),
    "f16_units_whole": synth.Workload(19, 4, 1100, 4, 64, 128, 4, 128, "fp16", True),
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


# ---------------------------------------------------------------------------
# The rounding budget: a per-element bound on |GPU - oracle| from the roundings
# the kernels make, for the tight regression check beside the tolerance bars.
# Each output is a sum of contributions (Scan2 weights times x, Q(C) times the
# passed state, D x; for the float path also LUT x times B in the state).
# Evaluating the oracle on |inputs| gives A = sum |contribution| per element
# (every map is linear in x, B, C, Q(C), CB, the passed states and D, with
# nonnegative dt, decays and scales). A kernel that rounds each computed MFMA
# operand once (relative u_op), forms decays from fp32 dAcs (u_exp) and
# accumulates in fp32 (u_acc) is then within
#   (u_op + u_exp + u_acc) A + (subnormal steps) + half an ulp of its output.
# ---------------------------------------------------------------------------

# one rounding of a computed operand into the MFMA type, at most 2^-p of its
# value for p significant bits (fp16 11, bf16 8): INT8 kernels round the Scan2
# weight (and cache CB' in fp16 before it); the float kernels round LUT x, the
# Scan2 weight and the 16-bit state copy once each, and carry bf16 operands as
# hi + lo pairs (16 significant bits); fp32 inputs use fp32 arithmetic
U_OP = {("int8", "fp16"): 2.0 ** -10, ("int8", "bf16"): 2.0 ** -8 + 2.0 ** -11,
        ("int8", "fp32"): 2.0 ** -20, ("float", "fp16"): 2.0 ** -10,
        ("float", "bf16"): 2.0 ** -15, ("float", "fp32"): 2.0 ** -20}


def u_exp(a_max: float) -> float:
    """Relative error of a decay factor exp(a_s - a_s') (times dt) when a comes
    from fp32 dAcs (|a| <= a_max), is scaled by log2(e) in fp32, and passes
    through the hardware exp2 and log2: a few fp32 roundings of the exponent,
    each at most 2^-24 of its magnitude, times ln 2, plus the instructions'
    own 1-ulp errors."""
    return 2.0 ** -24 * (4.0 * a_max * 1.4427 + 250.0) * 0.6931 + 2.0 ** -21


def u_acc(l: int) -> float:
    """fp32 accumulation along one output's chain (l / 16 MFMA accumulations,
    the rescale, the Scan1 multiply-adds)."""
    return 2.0 ** -24 * (l / 16 + 16)


def budget_ratio(y, ref, absum, u: float, dtype: str, tiny=0.0) -> float:
    """max over elements of |y - ref| / bound, bound = u * absum + tiny + half
    an ulp of y in its storage type (<= 1 passes)."""
    y = np.asarray(y, np.float64)
    bound = u * np.asarray(absum, np.float64) + tiny + half_ulp(y, dtype) + 1e-300
    return float(np.max(np.abs(y - np.asarray(ref, np.float64)) / bound))


def int8_absum(x, dt, r8, D, scales, chunk, h_init=None):
    """sum |contribution| of every INT8 output element, from the oracle's
    ChunkScan on absolute values of its own intermediates."""
    return O.chunk_scan_int8(np.abs(x), dt, r8["cumsum"]["a"], np.abs(r8["qC"]), np.abs(r8["cb"]),
                             np.abs(r8["passed"]), np.abs(np.asarray(D, np.float64)), scales, chunk,
                             None if h_init is None else np.abs(h_init))


def int8_budget(y, r8, x, dt, D, scales, chunk, dtype, h_init=None) -> float:
    """Rounding-budget ratio of an INT8 output y against the oracle's r8["y"]."""
    a_max = float(np.abs(r8["cumsum"]["a"]).max())
    ab = int8_absum(x, dt, r8, D, scales, chunk, h_init)
    # a Scan2 weight below fp16's normal range is off by at most half its
    # subnormal step, 2^-25, times |x|, for at most `chunk` terms
    tiny = 2.0 ** -25 * chunk * np.abs(np.asarray(x, np.float64)).max(axis=(0, 1))
    return budget_ratio(y, r8["y"], ab, U_OP[("int8", dtype)] + u_exp(a_max) + u_acc(chunk), dtype, tiny)


def float_budget(y, fin, x, dt, A, B, C, D, chunk, dtype, y_ref, h_ref, h_init=None):
    """Rounding-budget ratios (Y, final state) of a float-path output against
    the float64 definition (y_ref, h_ref from oracle.chunked)."""
    cs = O.chunk_cumsum(np.asarray(dt, np.float64), A, chunk)
    a_max = float(np.abs(cs["a"]).max())
    ya, ha = O.chunked(np.abs(x), dt, A, np.abs(B), np.abs(C), np.abs(np.asarray(D, np.float64)), chunk,
                       *(() if h_init is None else (np.abs(h_init),)))[:2]
    u = U_OP[("float", dtype)] + u_exp(a_max) + u_acc(chunk)
    L = np.asarray(x).shape[1]
    c = -(-L // chunk)
    tiny_y = 2.0 ** -25 * chunk * np.abs(np.asarray(x, np.float64)).max(axis=(0, 1))
    ry = budget_ratio(y, y_ref, ya, u, dtype, tiny_y)
    rh = None
    if fin is not None:
        # the state adds one fp32 multiply-add per chunk; a LUT x operand below
        # fp16's normal range is off by 2^-25 |B| per position
        tiny_h = 2.0 ** -25 * L * np.abs(np.asarray(B, np.float64)).max() if dtype == "fp16" else 0.0
        fin = np.asarray(fin, np.float64)
        bound = (u + c * 2.0 ** -23) * ha + tiny_h + 1e-300
        rh = float(np.max(np.abs(fin - h_ref) / bound))
    return ry, rh


def state_chan_err(fin, ref) -> float:
    """max over channels (h, p) of max_{b,n} |fin - ref| / RMS_{b,n}(ref) for
    states [B, H, P, N] (each channel against its own size)."""
    fin = np.asarray(fin, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=(0, 3)))
    err = np.abs(fin - ref).max(axis=(0, 3))
    return float(np.max(err / np.maximum(rms, 1e-30)))


def report(tag: str, **metrics) -> None:
    """One line of measured errors (shown with pytest -s, and in the tail of
    a failing test)."""
    print(tag + ": " + ", ".join(f"{k} {v:.3g}" for k, v in metrics.items() if v is not None), flush=True)
