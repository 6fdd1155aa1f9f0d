"""Benchmark of the SSD-layer forward on one MI355X.

A step is one ssd_forward call (the whole hot path: B/C quantisation,
ChunkCumsum, ChunkState, StatePassing, ChunkBMM, ChunkScan) over one batch of
synthetic Mamba-2 2.7B-shaped input (batch 8, L 2048, H 80, P 64, N 128, G 1,
chunk 256, fp16), already resident in HBM. The INT8 path is the headline line;
the float path is measured beside it.

Prints one JSON line. --gpus N with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
WORKLOAD_ID = 2           # Mamba-2 2.7B-shaped layer


def algorithmic_bytes_per_token(w, int8: bool) -> int:
    """X, dt, B, C read once, Y written once, plus one chunk-state exchange
    (each chunk-boundary state written once and read once) at the path's state
    width: int8, or the input dtype for the float path."""
    esz = {"fp32": 4, "fp16": 2, "bf16": 2}[w.dtype]
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    io = esz * (2 * H * P + H + 2 * G * N)
    state = (1 if int8 else esz) * 2 * H * P * N / w.chunk
    return int(round(io + state))


def io_bytes_per_token(w) -> int:
    """X, dt, B, C read once and Y written once (no state exchange)."""
    esz = {"fp32": 4, "fp16": 2, "bf16": 2}[w.dtype]
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    return esz * (2 * H * P + H + 2 * G * N)


def copy_bandwidth(torch, nbytes=1 << 30, reps=10) -> float:
    """Device-to-device copy rate (bytes read + written per second, GB/s)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del a, b
    return gbs


def device_info(torch) -> dict:
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip, "torch": torch.__version__}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def kernel_source_hash() -> str:
    d = os.path.join(ROOT, "mamba_ssd_chunked_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str):
    """HBM bytes per call from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    f = os.path.join(ROOT, "profiles", f"traffic_{workload}_{path}.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_call")


DECODE_BATCHES = (8, 1024)   # the layer's batch (latency) and a serving batch (bandwidth)


def decode_bytes_per_step(w, batch: int, int8: bool) -> int:
    """One decode position: the state read and written once (int8, or fp32 on
    the float path), x, dt, B, C read and y written once."""
    esz = {"fp32": 4, "fp16": 2, "bf16": 2}[w.dtype]
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    state = (1 if int8 else 4) * 2 * H * P * N
    return batch * (state + esz * (2 * H * P + H + 2 * G * N))


def bench_decode(torch, np, L, synth, w, consts, scales, steps, warmup) -> dict:
    """ssd_decode_step at each batch of DECODE_BATCHES on both paths; inputs
    resident in HBM, the state updated in place each step. us_per_step comes
    from `steps` steps replayed as one HIP graph; eager_us_per_step from the
    same steps called one by one from Python (host-bound at small batch)."""
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    out = {}
    for batch in DECODE_BATCHES:
        ev = synth.evaluation_batch(w, consts, batch=batch, seqlen=1)
        dev = {k: torch.from_numpy(np.ascontiguousarray(v[:, 0])).cuda() for k, v in ev.items()}
        h8 = torch.from_numpy(synth.int8_state(w, batch)).cuda()
        sh = L.make_shape(batch, 1, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
        y = torch.empty_like(dev["x"])
        for path_name in ("int8", "float"):
            i8 = path_name == "int8"
            path = L.SSD_PATH_INT8 if i8 else L.SSD_PATH_FLOAT
            st = h8 if i8 else h8.float()
            sc = scales if i8 else None

            def step():
                L.ssd_decode_step(sh, path, dev["x"], dev["dt"], A, dev["B"], dev["C"], D, sc, st, y)

            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            eager_us = e0.elapsed_time(e1) * 1e3 / steps
            # the same steps captured in one HIP graph: a serving loop's launch
            # path, without the host cost of one Python call per step
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(steps):
                    step()
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            del g
            nbytes = decode_bytes_per_step(w, batch, i8)
            gbs = nbytes / (us * 1e-6) / 1e9
            rec = {
                "us_per_step": us, "eager_us_per_step": eager_us, "tokens_per_s": batch / (us * 1e-6),
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": nbytes,
                             "traffic": measured_traffic(f"decode_b{batch}", path_name)}}
            if nbytes < LLC_BYTES:
                # the state stays in the last-level cache between back-to-back
                # steps; single steps after a 512 MB write give the rate from HBM
                # (the write is enqueued first, so the step's events bracket GPU
                # time only)
                scratch = torch.empty(2 * LLC_BYTES // 4, dtype=torch.float32, device="cuda")
                reps = min(steps, 20)
                cs = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
                ce = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
                for i in range(reps):
                    scratch.fill_(float(i))
                    cs[i].record()
                    step()
                    ce[i].record()
                torch.cuda.synchronize()
                cold_us = float(np.median([a_.elapsed_time(b_) for a_, b_ in zip(cs, ce)])) * 1e3
                del scratch
                rec["cache"] = "warm (back-to-back steps; working set under the 256 MB last-level cache)"
                rec["cold_us_per_step"] = cold_us
                rec["cold_roofline_frac"] = nbytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS
            else:
                rec["cache"] = "working set over the last-level cache"
            out[f"{path_name}_b{batch}"] = rec
            del st
        del h8, dev, y
        torch.cuda.empty_cache()
    return out


# Table 5 of the SSDi8 notes page: SSD latency (ms) of Mamba-2 2.7B at W4A8 for
# the float SSD, "+ Q(X) only", "+ reconstruction + B,C quantisation" and the
# full method (persistent INT8 state + INT8 ChunkBMM). Another machine's
# numbers: their ratios are the comparison, not the values.
PAGES_TABLE5_MS = (8.63, 8.58, 8.05, 6.53)


def bench_ablation(torch, np, L, synth, w, consts, dev, A, D, scales, cal_dev, steps, warmup) -> dict:
    """The Table 5 ladder on this GPU: every row run through the module
    kernels (one launch per module, states and CB through HBM, as the pages'
    modules do), and the two rows the fused kernels cover through ssd_forward."""
    sh = L.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
    # step of Q(X) by the library's pack rule, from amax |x| on the calibration sequences
    amx = torch.stack([s["x"].abs().amax(dim=(0, 1)).float() for s in cal_dev]).amax(0)
    G, HP = w.ngroups, w.nheads * w.headdim
    am = np.concatenate([np.ones(2 * G, np.float32), amx.cpu().numpy().reshape(-1),
                         np.ones(HP, np.float32)])
    px = L.ssd_scales_from_amax(G, w.nheads, w.headdim, am)
    sc_host = {k: v for k, v in scales.host.items()}
    sc_host.update({"s_Xq": px["s_X"], "inv_Xq": px["inv_X"]})
    sc_all = L.ScalePack(sc_host)
    y = torch.empty_like(dev["x"])
    c = sh.nchunks
    cs = (w.batch, w.nheads, c, w.chunk)
    dAcs = torch.empty(cs, dtype=torch.float32, device="cuda")
    lut = torch.empty_like(dAcs)
    qd = torch.empty(cs[:3], dtype=torch.uint8, device="cuda")
    st_shape = (w.batch, c, w.nheads, w.headdim, w.dstate)
    st8 = torch.empty(st_shape, dtype=torch.int8, device="cuda")
    st32 = torch.empty(st_shape, dtype=torch.float32, device="cuda")
    cb = torch.empty((w.batch, c, w.ngroups, w.chunk, w.chunk), dtype=torch.float32, device="cuda")
    qB = torch.empty(dev["B"].shape, dtype=torch.int8, device="cuda")
    qC = torch.empty_like(qB)

    def modules_float():
        L.ssd_chunk_cumsum(sh, dev["dt"], A, dAcs, lut)
        L.ssd_chunk_state(sh, L.SSD_PATH_FLOAT, dev["x"], lut, dev["B"], None, st32)
        L.ssd_state_passing(sh, L.SSD_PATH_FLOAT, st32, dAcs)
        L.ssd_chunk_bmm(sh, L.SSD_PATH_FLOAT, dev["C"], dev["B"], cb)
        L.ssd_chunk_scan(sh, L.SSD_PATH_FLOAT, dev["x"], dev["dt"], dAcs, dev["C"], cb, st32, D, None, y)

    def modules_int8():
        L.ssd_quantize_bc(sh, dev["B"], dev["C"], scales, qB, qC)
        L.ssd_chunk_cumsum(sh, dev["dt"], A, dAcs, lut, qd)
        L.ssd_chunk_state(sh, L.SSD_PATH_INT8, dev["x"], lut, qB, scales, st8)
        L.ssd_state_passing(sh, L.SSD_PATH_INT8, st8, dAcs, qd)
        L.ssd_chunk_bmm(sh, L.SSD_PATH_INT8, qC, qB, cb)
        L.ssd_chunk_scan(sh, L.SSD_PATH_INT8, dev["x"], dev["dt"], dAcs, qC, cb, st8, D, scales, y)

    wss = {p: torch.empty(max(1, L.ssd_workspace_bytes(sh, p)), dtype=torch.uint8, device="cuda")
           for p in (L.SSD_PATH_ABL_QX, L.SSD_PATH_ABL_RECON, L.SSD_PATH_FLOAT, L.SSD_PATH_INT8)}

    def forward(p, sc):
        return lambda: L.ssd_forward(sh, p, dev["x"], dev["dt"], A, dev["B"], dev["C"], D, sc, y,
                                     workspace=wss[p])

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    rows = [
        {"row": "SSD all floating point (fp16)", "module_ms": timed(modules_float),
         "fused_ms": timed(forward(L.SSD_PATH_FLOAT, None))},
        {"row": "+ Q(X) only", "module_ms": timed(forward(L.SSD_PATH_ABL_QX, sc_all))},
        {"row": "+ reconstruction + B,C quantisation", "module_ms": timed(forward(L.SSD_PATH_ABL_RECON, sc_all))},
        {"row": "+ persistent INT8 state + INT8 ChunkBMM (the full method)", "module_ms": timed(modules_int8),
         "fused_ms": timed(forward(L.SSD_PATH_INT8, scales))},
    ]
    base = rows[0]["module_ms"]
    for r, pg in zip(rows, PAGES_TABLE5_MS):
        r["module_speedup_vs_float_modules"] = base / r["module_ms"]
        r["pages_ms"] = pg
        r["pages_speedup"] = PAGES_TABLE5_MS[0] / pg
    return {"workload": w.name, "rows": rows}


def bench_epilogue(torch, np, L, synth, w, y, y_ref, steps, warmup) -> dict:
    """ssd_epilogue (RMSNorm with the 0.15 mean correction) on the layer's
    output: Y read once and the result written once per call."""
    sh = L.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
    c = torch.empty((w.nheads, w.headdim), dtype=torch.float32, device="cuda")
    L.ssd_mean_correction(sh, y_ref, y, c)
    wt = torch.from_numpy(synth.norm_weight(w)).cuda()
    out = torch.empty_like(y)

    def step():
        L.ssd_epilogue(sh, y, c, L.MEAN_CORRECTION_ALPHA, wt, 1e-5, out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    esz = {"fp32": 4, "fp16": 2, "bf16": 2}[w.dtype]
    nbytes = 2 * w.batch * w.seqlen * w.nheads * w.headdim * esz
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": us, "tokens_per_s": w.batch * w.seqlen / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nbytes}}


CPU_SEQUENCES = 4   # sequences of the batch the CPU baseline runs (a bounded sample)


def cpu_baseline(w, consts, ev) -> dict:
    """The float64 recurrence oracle timed on host cores, on the first
    CPU_SEQUENCES sequences of the batch (all heads, full length), split by
    (sequence, head block) over a process pool that is started before timing."""
    import concurrent.futures as cf
    import multiprocessing as mp

    from mamba_ssd_chunked_amd import synth

    nb = min(CPU_SEQUENCES, w.batch)
    x = synth.to_f64(ev["x"][:nb], w.dtype)
    dt = synth.to_f64(ev["dt"][:nb], w.dtype)
    B = synth.to_f64(ev["B"][:nb], w.dtype)
    C = synth.to_f64(ev["C"][:nb], w.dtype)
    ncpu = len(os.sched_getaffinity(0))
    workers = max(1, min(16, ncpu))
    hpg = w.nheads // w.ngroups
    nblk = max(1, -(-workers // nb))
    per = -(-w.nheads // nblk)
    jobs = []
    for b in range(nb):
        for h0 in range(0, w.nheads, per):
            h1 = min(w.nheads, h0 + per)
            g0, g1 = h0 // hpg, (h1 - 1) // hpg + 1
            # a head block inside whole groups keeps the head -> group map
            jobs.append((x[b:b + 1, :, h0:h1], dt[b:b + 1, :, h0:h1], consts["A"][h0:h1],
                         B[b:b + 1, :, g0:g1], C[b:b + 1, :, g0:g1], consts["D"][h0:h1], h0, hpg, g0))
    # one BLAS thread per worker process, so the workers are the threads used
    threads = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in threads}
    os.environ.update({k: "1" for k in threads})
    try:
        with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            list(ex.map(_warm, range(workers)))          # workers started and imported
            t0 = time.perf_counter()
            list(ex.map(_recurrence_job, jobs))
            t1 = time.perf_counter()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    tokens_per_s = nb * w.seqlen / (t1 - t0)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 recurrence on {nb} of {w.batch} sequences (all {w.nheads} heads, "
                      f"L={w.seqlen}); {t1 - t0:.2f} s wall on {workers} single-threaded processes",
            "seconds": t1 - t0, "cpu": cpu_model(),
            "host_cpus_available": ncpu, "host_cpus_total": os.cpu_count()}


def _warm(_):
    from oracle import ssd_oracle  # noqa: F401
    return 0


def _recurrence_job(job):
    import numpy as np

    from oracle import ssd_oracle as O
    x, dt, A, B, C, D, h0, hpg, g0 = job
    H = x.shape[2]
    # remap the block's heads onto its local groups
    g_local = (np.arange(h0, h0 + H) // hpg) - g0
    Bh = B[:, :, g_local]
    Ch = C[:, :, g_local]
    y, _ = O.recurrence(x, dt, A, Bh, Ch, D)
    return float(y[0, -1, 0, 0])


def schedule_of(w, cus: int) -> str:
    """The INT8 schedule the library's automatic choice takes for a layer."""
    return "chunk" if w.batch * w.nheads < 2 * cus else "head"


LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def time_forward(torch, np, L, w, sh, path, dev, A, D, scales, y, steps, warmup, copy_gbs,
                 traffic=None, spread=True, cold=False) -> dict:
    """Tokens/s and HBM roofline fraction of ssd_forward on resident inputs:
    `warmup` untimed calls, then `steps` back-to-back calls bracketed by one
    pair of events on the stream the kernels run on (events between the calls
    would add their own packets); optionally the spread of single calls from a
    second, untimed pass, and (cold) single calls each after a 512 MB write
    that evicts the inputs from the last-level cache."""
    ws = torch.empty(max(1, L.ssd_workspace_bytes(sh, path)), dtype=torch.uint8, device="cuda")
    sc = scales if path == L.SSD_PATH_INT8 else None

    def step():
        L.ssd_forward(sh, path, dev["x"], dev["dt"], A, dev["B"], dev["C"], D, sc, y, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tokens = w.batch * w.seqlen
    ms_per_step = (t1 - t0) * 1e3 / steps
    avg_call_s = e0.elapsed_time(e1) * 1e-3 / steps
    call_ms = {"timed_mean": avg_call_s * 1e3}
    if spread:
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            ev_s[i].record()
            step()
            ev_e[i].record()
        torch.cuda.synchronize()
        per_call_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_s, ev_e)])
        call_ms.update({"mean": float(per_call_ms.mean()), "median": float(np.median(per_call_ms)),
                        "p10": float(np.percentile(per_call_ms, 10)),
                        "p90": float(np.percentile(per_call_ms, 90))})
    if cold:
        scratch = torch.empty(2 * LLC_BYTES // 4, dtype=torch.float32, device="cuda")
        reps = min(steps, 20)
        cs = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            scratch.fill_(float(i))
            cs[i].record()
            step()
            ce[i].record()
        torch.cuda.synchronize()
        cold_ms = np.array([a.elapsed_time(b) for a, b in zip(cs, ce)])
        call_ms["cold_median"] = float(np.median(cold_ms))
        del scratch
    del ws
    bpt = algorithmic_bytes_per_token(w, path == L.SSD_PATH_INT8)
    bytes_per_call = bpt * tokens
    achieved = bytes_per_call / avg_call_s / 1e9
    return {
        "value": tokens / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "call_ms": call_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "ssd_forward (all kernels of one call)",
                     "algorithmic_bytes_per_call": bytes_per_call,
                     "algorithmic_bytes_per_token": bpt,
                     "io_only_frac": io_bytes_per_token(w) * tokens / avg_call_s / 1e9 / HBM_PEAK_GBS,
                     "frac_of_copy": achieved / copy_gbs},
    }


CONFIG_IDS = (1, 2, 3, 4)   # every single-GPU layer of the workload table


def bench_configs(torch, np, L, synth, steps, warmup, copy_gbs, head=None) -> dict:
    """Both paths on each workload of the table, on its own seeded inputs and
    static scales (calibrated on the GPU from its two calibration sequences);
    the headline layer's figures are reused when given."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for wid in CONFIG_IDS:
        w = synth.WORKLOADS[wid]
        rec = {"workload": wid, "int8_schedule": schedule_of(w, cus)}
        if head is not None and head[0] == wid:
            res = head[1]
        else:
            consts = synth.layer_constants(w)
            ev = synth.evaluation_batch(w, consts)
            dev = {k: torch.from_numpy(v).cuda() for k, v in ev.items()}
            del ev
            A = torch.from_numpy(consts["A"]).cuda()
            D = torch.from_numpy(consts["D"]).cuda()
            sh = L.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
            cal = [{k: torch.from_numpy(v).cuda() for k, v in s.items()}
                   for s in synth.calibration_sequences(w, consts)]
            scales = L.calibrate(lambda s: L.make_shape(1, w.seqlen, w.nheads, w.headdim, w.dstate,
                                                        w.ngroups, w.chunk, w.dtype), cal, A)
            del cal
            y = torch.empty_like(dev["x"])
            res = {}
            for name, path in (("int8", L.SSD_PATH_INT8), ("float", L.SSD_PATH_FLOAT)):
                small = algorithmic_bytes_per_token(w, path == L.SSD_PATH_INT8) * w.batch * w.seqlen < LLC_BYTES
                res[name] = time_forward(torch, np, L, w, sh, path, dev, A, D, scales, y, steps, warmup,
                                         copy_gbs, traffic=measured_traffic(w.name, name), spread=False,
                                         cold=small)
            del dev, y
            torch.cuda.empty_cache()
        for name, r in res.items():
            rec[name] = {"tokens_per_s": r["value"], "call_ms": r["call_ms"]["timed_mean"],
                         "roofline_frac": r["roofline"]["frac"],
                         "achieved_gbs": r["roofline"]["achieved"],
                         "traffic": r["roofline"]["traffic"]}
            if "cold_median" in r["call_ms"]:
                # back-to-back calls keep this working set in the last-level
                # cache: the figures above are warm; the cold ones follow a
                # 512 MB write before each call
                cm = r["call_ms"]["cold_median"]
                rec[name]["cache"] = "warm (working set under the 256 MB last-level cache)"
                rec[name]["cold_call_ms"] = cm
                rec[name]["cold_roofline_frac"] = r["roofline"]["frac"] * r["call_ms"]["timed_mean"] / cm
        if "int8" in rec and "float" in rec:
            rec["int8_speedup"] = rec["float"]["call_ms"] / rec["int8"]["call_ms"]
        out[w.name] = rec
        print(f"# config {wid}: " + ", ".join(f"{k} {rec[k]['call_ms']:.4f} ms ({rec[k]['roofline_frac']:.3f})"
                                              + (f" cold {rec[k]['cold_call_ms']:.4f} ms" if "cold_call_ms" in rec[k] else "")
                                              for k in ("int8", "float") if k in rec),
              file=sys.stderr, flush=True)
    return out


TREND_BATCHES = (1, 8, 32)
TREND_SEQLENS = (256, 2048, 8192)


def device_sequence(torch, w, consts, batch, seqlen, seed):
    """One sequence drawn on the GPU with the input recipe of the workload
    table (X = N(0, 1) x the per-(h, p) scale, dt = softplus(0.5 N(0, 1) +
    dt_bias), B, C ~ N(0, 1)), cast once to the storage dtype. For shapes too
    large to draw on the host in reasonable time."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt_t = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype]
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    xs = torch.from_numpy(consts["xscale"]).cuda()
    bias = torch.from_numpy(consts["dt_bias"]).cuda()
    x = (torch.randn((batch, seqlen, H, P), generator=g, device="cuda") * xs).to(dt_t)
    dt = torch.nn.functional.softplus(
        0.5 * torch.randn((batch, seqlen, H), generator=g, device="cuda", dtype=torch.float64) + bias).to(dt_t)
    Bm = torch.randn((batch, seqlen, G, N), generator=g, device="cuda").to(dt_t)
    Cm = torch.randn((batch, seqlen, G, N), generator=g, device="cuda").to(dt_t)
    return {"x": x, "dt": dt, "B": Bm, "C": Cm}


def bench_trend(torch, np, L, synth, steps, warmup, copy_gbs) -> dict:
    """The INT8-over-float speed-up of ssd_forward on the 2.7B layer's head
    shape (H 80, P 64, N 128, G 1, chunk 256, fp16) over batch x length."""
    base = synth.WORKLOADS[2]
    consts = synth.layer_constants(base)
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cal = [device_sequence(torch, base, consts, 1, 2048, 7001 + r) for r in range(2)]
    scales = L.calibrate(lambda s: L.make_shape(1, 2048, base.nheads, base.headdim, base.dstate,
                                                base.ngroups, base.chunk, base.dtype), cal, A)
    del cal
    points = []
    for b in TREND_BATCHES:
        for seqlen in TREND_SEQLENS:
            w = base.replace(batch=b, seqlen=seqlen)
            dev = device_sequence(torch, w, consts, b, seqlen, 7100 + 10 * b + seqlen)
            sh = L.make_shape(b, seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype)
            y = torch.empty_like(dev["x"])
            r8 = time_forward(torch, np, L, w, sh, L.SSD_PATH_INT8, dev, A, D, scales, y, steps, warmup,
                              copy_gbs, spread=False)
            rf = time_forward(torch, np, L, w, sh, L.SSD_PATH_FLOAT, dev, A, D, None, y, steps, warmup,
                              copy_gbs, spread=False)
            del dev, y
            t8, tf = r8["call_ms"]["timed_mean"], rf["call_ms"]["timed_mean"]
            warm = algorithmic_bytes_per_token(w, False) * b * seqlen < LLC_BYTES
            points.append({"batch": b, "seqlen": seqlen, "int8_schedule": schedule_of(w, cus),
                           "int8_ms": t8, "float_ms": tf, "int8_speedup": tf / t8,
                           "int8_frac": r8["roofline"]["frac"], "float_frac": rf["roofline"]["frac"],
                           "cache": "warm (back-to-back calls; working set under the 256 MB last-level cache)"
                           if warm else "working set over the last-level cache"})
            print(f"# trend B={b} L={seqlen}: int8 {t8:.4f} ms, float {tf:.4f} ms, x{tf / t8:.2f}",
                  file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    return {"shape": "H80 P64 N128 G1 chunk256 fp16 (2.7B layer heads), inputs drawn on the GPU",
            "points": points}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paths", default="int8,float")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-epilogue", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode step (prints its JSON object)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload figures")
    ap.add_argument("--no-trend", action="store_true", help="skip the batch x length speed-up ladder")
    ap.add_argument("--schedule", choices=("auto", "head", "chunk"), default="auto",
                    help="INT8 schedule of the headline layer (default: the library's automatic choice)")
    ap.add_argument("--workload", type=int, default=WORKLOAD_ID,
                    help="workload id of the headline line (default: the 2.7B-shaped layer)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the SSD layer runs on a single MI355X here "
              "(no multi-GPU path is built); run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mamba_ssd_chunked_amd import _lib as L
    from mamba_ssd_chunked_amd import synth

    w = synth.WORKLOADS[args.workload]
    consts = synth.layer_constants(w)
    ev = synth.evaluation_batch(w, consts)
    dev = {k: torch.from_numpy(v).cuda() for k, v in ev.items()}
    A = torch.from_numpy(consts["A"]).cuda()
    D = torch.from_numpy(consts["D"]).cuda()
    sched = {"auto": L.SSD_SCHED_AUTO, "head": L.SSD_SCHED_HEAD, "chunk": L.SSD_SCHED_CHUNK}[args.schedule]
    sh = L.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, w.dtype, sched)

    # static scales from the two calibration sequences, on the GPU
    cal = synth.calibration_sequences(w, consts)
    cal_dev = [{k: torch.from_numpy(v).cuda() for k, v in s.items()} for s in cal]
    scales = L.calibrate(lambda s: L.make_shape(1, w.seqlen, w.nheads, w.headdim, w.dstate,
                                                w.ngroups, w.chunk, w.dtype), cal_dev, A)
    if args.decode_only:
        copy_bandwidth(torch)  # the 1 GiB copy that counter runs scale against
        dec = bench_decode(torch, np, L, synth, w, consts, scales, args.steps, args.warmup)
        print(json.dumps({"decode": dec, "kernel_source_hash": kernel_source_hash()}), flush=True)
        return 0
    y = torch.empty_like(dev["x"])
    copy_gbs = copy_bandwidth(torch)
    results = {}
    for path_name in args.paths.split(","):
        path = L.SSD_PATH_INT8 if path_name == "int8" else L.SSD_PATH_FLOAT
        results[path_name] = time_forward(torch, np, L, w, sh, path, dev, A, D, scales, y, args.steps,
                                          args.warmup, copy_gbs, traffic=measured_traffic(w.name, path_name))
    head_path = "int8" if "int8" in results else next(iter(results))
    head = results[head_path]
    out = {
        "metric": "SSD-layer tokens/s (INT8 & fp16) at 1 MI355X; % of HBM/int8-MFMA roofline",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if "int8" in results else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk": w.chunk, "input_dtype": w.dtype, "path": head_path,
                   "int8_schedule": (schedule_of(w, torch.cuda.get_device_properties(0).multi_processor_count)
                                     if args.schedule == "auto" else args.schedule)},
        "roofline": head["roofline"],
        "paths": results,
        "kernel_source_hash": kernel_source_hash(),
        "device": device_info(torch),
        "copy_gbs": copy_gbs,
    }
    if not args.no_decode:
        out["decode"] = bench_decode(torch, np, L, synth, w, consts, scales, args.steps, args.warmup)
    if not args.no_epilogue and "int8" in results:
        y8 = torch.empty_like(dev["x"])
        yf = torch.empty_like(dev["x"])
        L.ssd_forward(sh, L.SSD_PATH_INT8, dev["x"], dev["dt"], A, dev["B"], dev["C"], D, scales, y8)
        L.ssd_forward(sh, L.SSD_PATH_FLOAT, dev["x"], dev["dt"], A, dev["B"], dev["C"], D, None, yf)
        out["epilogue"] = bench_epilogue(torch, np, L, synth, w, y8, yf, args.steps, args.warmup)
    if not args.no_ablation:
        out["ablation"] = bench_ablation(torch, np, L, synth, w, consts, dev, A, D, scales, cal_dev,
                                         args.steps, args.warmup)
    if not args.no_configs:
        out["configs"] = bench_configs(torch, np, L, synth, min(args.steps, 20), min(args.warmup, 3), copy_gbs,
                                       head=(args.workload, results) if len(results) == 2 else None)
    if not args.no_trend:
        out["trend"] = bench_trend(torch, np, L, synth, min(args.steps, 10), min(args.warmup, 2), copy_gbs)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, consts, ev)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
