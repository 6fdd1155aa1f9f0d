"""Seeded synthetic inputs for the SSD layer workloads.

This module draws random tensors and casts them to the storage dtype. It holds
none of the SSD method's arithmetic, so both the HIP path (through the tests
and the benchmark) and the CPU oracle may consume what it returns.

Workloads are Mamba-2-shaped single SSD layers:

  id  shape (batch, L, H, P, N, G, chunk)   dtype  notes
  0   1, 256, 4, 16, 16, 1, 64               fp32   tiny, correctness only
  1   1, 2048, 64, 64, 128, 1, 256           fp16   1.3B-shaped layer
  2   8, 2048, 80, 64, 128, 1, 256           fp16   2.7B-shaped layer (headline)
  3   4, 4096, 128, 64, 128, 8, 256          bf16   8B-shaped, 16 heads per group
  4   1, 65536, 80, 64, 128, 1, 256          fp16   long context, small dt

Recipe (per workload id ``w``; ``Generator(PCG64(1000*w + role))``):
  role 0 - layer constants: dt_bias[h] = log(expm1(u_h)) with u_h log-uniform
           on [1e-3, 0.1] ([1e-3, 1e-2] for w=4); A[h] = -exp(U(0, ln 16));
           D[h] ~ N(0, 1); from w=1 on, a per-head X scale ~ LogNormal(0, 0.5)
           and max(1, round(0.01*H*P)) (h, p) outlier channels scaled x20.
  role 1, 2 - calibration sequences (batch 1 each).
  role 3 - evaluation batch.
  Per sequence: X = N(0,1) * xscale[h,p]; dt = softplus(0.5*N(0,1) + dt_bias[h]);
  B, C ~ N(0, 1). Draws are fp32/fp64 and cast once (round to nearest even)
  to the storage dtype. dt is handed to the SSD already through softplus.

Storage: fp32 -> np.float32, fp16 -> np.float16, bf16 -> np.uint16 holding
the bf16 bit pattern (NumPy has no bfloat16). ``to_f64`` widens any of them
exactly.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str
    outliers: bool
    dt_lo: float = 1e-3
    dt_hi: float = 1e-1

    @property
    def name(self) -> str:
        return (f"ssd_b{self.batch}_L{self.seqlen}_H{self.nheads}_P{self.headdim}"
                f"_N{self.dstate}_G{self.ngroups}_l{self.chunk}_{self.dtype}")

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    0: Workload(0, 1, 256, 4, 16, 16, 1, 64, "fp32", False),
    1: Workload(1, 1, 2048, 64, 64, 128, 1, 256, "fp16", True),
    2: Workload(2, 8, 2048, 80, 64, 128, 1, 256, "fp16", True),
    3: Workload(3, 4, 4096, 128, 64, 128, 8, 256, "bf16", True),
    4: Workload(4, 1, 65536, 80, 64, 128, 1, 256, "fp16", True, 1e-3, 1e-2),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def cast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float draws once to the storage representation of ``dtype``."""
    if dtype == "fp32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(a, dtype=np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def layer_constants(w: Workload, seed_base: int | None = None) -> dict:
    """Per-layer constants (role 0): A, D (fp32), dt_bias, X channel scale."""
    base = 1000 * w.wid if seed_base is None else seed_base
    rng = np.random.Generator(np.random.PCG64(base + 0))
    H, P = w.nheads, w.headdim
    u = np.exp(rng.uniform(math.log(w.dt_lo), math.log(w.dt_hi), size=H))
    dt_bias = np.log(np.expm1(u))
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    xscale = np.ones((H, P), dtype=np.float64)
    if w.outliers:
        xscale *= rng.lognormal(0.0, 0.5, size=H)[:, None]
        n_out = max(1, int(round(0.01 * H * P)))
        idx = rng.choice(H * P, size=n_out, replace=False)
        xscale.reshape(-1)[idx] *= 20.0
    return {"A": A, "D": D, "dt_bias": dt_bias, "xscale": xscale.astype(np.float32)}


def sequence(w: Workload, role: int, batch: int | None = None, consts: dict | None = None,
             seqlen: int | None = None, seed_base: int | None = None) -> dict:
    """Draw X, dt, B, C for one role (1, 2: calibration; 3: evaluation).

    Returns the stored (cast) arrays: x [b,L,H,P], dt [b,L,H], B, C [b,L,G,N].
    """
    base = 1000 * w.wid if seed_base is None else seed_base
    consts = layer_constants(w, seed_base) if consts is None else consts
    rng = np.random.Generator(np.random.PCG64(base + role))
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    x = rng.standard_normal((b, L, H, P), dtype=np.float32)
    x *= consts["xscale"][None, None]
    z = rng.standard_normal((b, L, H), dtype=np.float32).astype(np.float64)
    dt = _softplus(0.5 * z + consts["dt_bias"][None, None, :])
    Bm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    Cm = rng.standard_normal((b, L, G, N), dtype=np.float32)
    return {
        "x": cast(x, w.dtype),
        "dt": cast(dt, w.dtype),
        "B": cast(Bm, w.dtype),
        "C": cast(Cm, w.dtype),
    }


def calibration_sequences(w: Workload, consts: dict | None = None, seqlen: int | None = None,
                          seed_base: int | None = None) -> list:
    """The two calibration sequences (roles 1 and 2, batch 1 each)."""
    consts = layer_constants(w, seed_base) if consts is None else consts
    return [sequence(w, r, 1, consts, seqlen, seed_base) for r in (1, 2)]


def evaluation_batch(w: Workload, consts: dict | None = None, batch: int | None = None,
                     seqlen: int | None = None, seed_base: int | None = None) -> dict:
    consts = layer_constants(w, seed_base) if consts is None else consts
    return sequence(w, 3, batch, consts, seqlen, seed_base)


def int8_state(w: Workload, batch: int, seed: int | None = None) -> np.ndarray:
    """A persistent INT8 state [batch, H, P, N], uniform over [-127, 127]
    (seeded; role 4 of the workload unless a seed is given)."""
    rng = np.random.Generator(np.random.PCG64(1000 * w.wid + 4 if seed is None else seed))
    return rng.integers(-127, 128, size=(batch, w.nheads, w.headdim, w.dstate), dtype=np.int8)


def norm_weight(w: Workload, seed: int | None = None) -> np.ndarray:
    """RMSNorm weight [H, P] for the epilogue, 1 + 0.1 N(0, 1) (seeded; role 5)."""
    rng = np.random.Generator(np.random.PCG64(1000 * w.wid + 5 if seed is None else seed))
    return (1.0 + 0.1 * rng.standard_normal((w.nheads, w.headdim))).astype(np.float32)


def as_f64(seq: dict, dtype: str) -> dict:
    """Widen every stored tensor of a sequence dict to float64 (exact)."""
    return {k: to_f64(v, dtype) for k, v in seq.items()}
