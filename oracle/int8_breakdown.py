"""Where the INT8 method's error comes from: the forward with one quantiser
switched on at a time (reading R19 of ssd_oracle), then all of them, each
measured against the float64 definition.

TEST INFRASTRUCTURE (a report, CPU only). It runs the oracle alone; scales are
calibrated by the oracle on the two calibration sequences, as everywhere else.

Usage: python -m oracle.int8_breakdown [workload ids...]   (default: 1 2)
Prints one markdown table per workload: the global max|err| / RMS, the RMS of
the error over the RMS of the output, the per-channel metric (max over (h, p)
of max |err| / that channel's RMS) and the share of values each switched-on
quantiser saturated.
"""
from __future__ import annotations

import sys
import time

import numpy as np

from mamba_ssd_chunked_amd import synth
from oracle import ssd_oracle as O

ROWS = (("none (float64 definition)", ()),
        ("Q(B), Q(C)", ("bc",)),
        ("Q(Xs)", ("xs",)),
        ("S8 (local state)", ("s8",)),
        ("S8 + Eq. 6 (passed state)", ("eq6",)),
        ("all (the INT8 method)", O.STAGES))


def metrics(y, ref) -> tuple:
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(y - ref)
    chan_rms = np.sqrt(np.mean(ref * ref, axis=(0, 1)))
    per_chan = float(np.max(err.max(axis=(0, 1)) / np.maximum(chan_rms, 1e-30)))
    return float(err.max()) / rms, float(np.sqrt(np.mean(err * err))) / rms, per_chan


def breakdown(wid: int) -> str:
    w = synth.WORKLOADS[wid]
    c = synth.layer_constants(w)
    ev = synth.as_f64(synth.evaluation_batch(w, c), w.dtype)
    cal = [synth.as_f64(s, w.dtype) for s in synth.calibration_sequences(w, c)]
    am = O.calibrate(cal, c["A"], w.ngroups, w.chunk)
    del cal
    sc = O.scale_pack(am["B"], am["C"], am["Xs"], am["S"], w.nheads)
    ref, _ = O.chunked(ev["x"], ev["dt"], c["A"], ev["B"], ev["C"], c["D"], w.chunk)[:2]
    lines = [f"workload {wid} ({w.name})", "",
             "| quantisers on | max\\|err\\|/RMS | RMS err / RMS | per-channel | saturated |",
             "|---|---|---|---|---|"]
    for label, stages in ROWS:
        t0 = time.perf_counter()
        r = O.forward_stages(ev["x"], ev["dt"], c["A"], ev["B"], ev["C"], c["D"], sc, w.chunk, stages)
        g, rmse, pc = metrics(r["y"], ref)
        sat = ", ".join(f"{k} {100.0 * n / t:.3g}%" for k, (n, t) in r["saturated"].items()) or "-"
        lines.append(f"| {label} | {g:.3g} | {rmse:.3g} | {pc:.3g} | {sat} |")
        print(f"  {label}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    return "\n".join(lines)


def main(argv) -> int:
    wids = [int(a) for a in argv] or [1, 2]
    for wid in wids:
        print(breakdown(wid), flush=True)
        print(flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
