"""Python binding of libssd.so (the SSD C ABI declared in include/ssd.h).

Argument marshalling only: every step of the SSD forward runs in the HIP
kernels behind the C ABI. torch tensors supply device memory and the current
stream. The functions keep the C names and argument order; device buffers are
passed as torch tensors (or None for optional ones), the shape as an
``SsdShape`` and the INT8 scales as a ``ScalePack``.

Importing this module loads libssd.so and raises if it is missing: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_OK = 0
SSD_E_NULL = 1
SSD_E_SHAPE = 2
SSD_E_UNSUPPORTED = 3
SSD_E_ALIGN = 4
SSD_E_WORKSPACE = 5
SSD_E_HIP = 6
SSD_E_INTERNAL = 7
SSD_E_VALUE = 8
SSD_E_TOO_LARGE = 9
NOALLOC_SCRATCH_BYTES = 128 << 20

SSD_DTYPE_F32 = 0
SSD_DTYPE_F16 = 1
SSD_DTYPE_BF16 = 2
SSD_PATH_FLOAT = 0
SSD_PATH_INT8 = 1
SSD_PATH_ABL_QX = 2
SSD_PATH_ABL_RECON = 3
SSD_SCHED_AUTO = 0
SSD_SCHED_HEAD = 1
SSD_SCHED_CHUNK = 2

DTYPE_CODE = {torch.float32: SSD_DTYPE_F32, torch.float16: SSD_DTYPE_F16,
              torch.bfloat16: SSD_DTYPE_BF16}
DTYPE_NAME = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


class SsdShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("schedule", ctypes.c_int32)]

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)


class SsdScales(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("s_B", "s_C", "inv_B", "inv_C", "inv_X", "s_S", "M_req", "s_X", "s_Xq", "inv_Xq")]


class SsdTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q_xs", "s32", "s8_local", "passed")]


class SSDError(RuntimeError):
    def __init__(self, name: str, rc: int):
        super().__init__(f"{name} failed: {status_string(rc)} (status {rc})")
        self.status = rc


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -m mamba_ssd_chunked_amd.csrc.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    SP = ctypes.POINTER(SsdShape)
    sig = {
        "ssd_quantize_bc": [SP, P, P, ctypes.POINTER(SsdScales), P, P, P],
        "ssd_chunk_cumsum": [SP, P, P, P, P, P, P],
        "ssd_chunk_state": [SP, ctypes.c_int, P, P, P, ctypes.POINTER(SsdScales), P,
                            ctypes.POINTER(SsdTaps), P],
        "ssd_state_passing": [SP, ctypes.c_int, P, P, P, P, P, P],
        "ssd_chunk_bmm": [SP, ctypes.c_int, P, P, P, P],
        "ssd_chunk_scan": [SP, ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.POINTER(SsdScales), P, P],
        "ssd_forward": [SP, ctypes.c_int, P, P, P, P, P, P, ctypes.POINTER(SsdScales), P, P, P, P,
                        ctypes.c_size_t, ctypes.POINTER(SsdTaps), P],
        "ssd_forward_noalloc": [SP, ctypes.c_int, P, P, P, P, P, P, ctypes.POINTER(SsdScales), P, P, P,
                                ctypes.POINTER(SsdTaps), P],
        "ssd_decode_step": [SP, ctypes.c_int, P, P, P, P, P, P, ctypes.POINTER(SsdScales), P, P,
                            P],
        "ssd_epilogue": [SP, P, P, ctypes.c_float, P, ctypes.c_float, P, P],
        "ssd_mean_correction": [SP, P, P, P, P],
        "ssd_calibrate_amax": [SP, P, P, P, P, P, P, P, ctypes.c_size_t, P],
        "ssd_scales_from_amax": [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name in ("ssd_workspace_bytes",):
        f = getattr(lib, name)
        f.argtypes = [SP, ctypes.c_int]
        f.restype = ctypes.c_size_t
    lib.ssd_calibrate_workspace_bytes.argtypes = [SP]
    lib.ssd_calibrate_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    return lib


LIB = _load()

EXPORTED = ("ssd_quantize_bc", "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing",
            "ssd_chunk_bmm", "ssd_chunk_scan", "ssd_forward", "ssd_forward_noalloc", "ssd_decode_step",
            "ssd_epilogue", "ssd_mean_correction",
            "ssd_workspace_bytes",
            "ssd_calibrate_amax", "ssd_calibrate_workspace_bytes", "ssd_scales_from_amax",
            "ssd_status_string")


def status_string(rc: int) -> str:
    return LIB.ssd_status_string(rc).decode()


def _check(name: str, rc: int) -> None:
    if rc != SSD_OK:
        raise SSDError(name, rc)


def _p(t):
    """Device address of a tensor; the C ABI takes dense row-major buffers only."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("SSD buffers must be contiguous (row-major, no strides)")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
               schedule=0) -> SsdShape:
    code = dtype if isinstance(dtype, int) else DTYPE_CODE[DTYPE_NAME.get(dtype, dtype)]
    return SsdShape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, code, schedule)


class ScalePack:
    """Device copy of the static scale pack, each array 256-byte aligned.

    ``arrays`` holds float32 numpy arrays s_B, s_C, inv_B, inv_C ([G]) and
    s_X, inv_X, s_S, M_req ([H, P] or [H*P]); optionally s_Xq, inv_Xq ([H, P],
    the step of X itself, read only by the "Q(X) only" ablation path).
    """

    ORDER = ("s_B", "s_C", "inv_B", "inv_C", "s_X", "inv_X", "s_S", "M_req")
    OPTIONAL = ("s_Xq", "inv_Xq")

    def __init__(self, arrays: dict, device="cuda"):
        names = [k for k in self.ORDER if k in arrays] + [k for k in self.OPTIONAL if k in arrays]
        flat = [np.ascontiguousarray(arrays[k], dtype=np.float32).reshape(-1) for k in names]
        offs, cur = [], 0
        for a in flat:
            offs.append(cur)
            cur += -(-a.size // 64) * 64
        host = np.zeros(max(cur, 64), dtype=np.float32)
        for o, a in zip(offs, flat):
            host[o:o + a.size] = a
        self.host = {k: a for k, a in zip(names, flat)}
        self.tensor = torch.from_numpy(host).to(device)
        base = self.tensor.data_ptr()
        ptr = {k: base + 4 * o for k, o in zip(names, offs)}
        self.struct = SsdScales(*[ptr.get(k) for k in ("s_B", "s_C", "inv_B", "inv_C", "inv_X",
                                                       "s_S", "M_req", "s_X", "s_Xq", "inv_Xq")])


def _scales(sc):
    if sc is None:
        return None
    if isinstance(sc, ScalePack):
        return ctypes.byref(sc.struct)
    return ctypes.byref(sc)


def _taps(taps):
    if taps is None:
        return None
    return ctypes.byref(SsdTaps(_p(taps.get("q_xs")), _p(taps.get("s32")),
                                _p(taps.get("s8_local")), _p(taps.get("passed"))))


# ---------------------------------------------------------------------------
# the C calls, same names and argument order
# ---------------------------------------------------------------------------

def ssd_quantize_bc(shape, B, C, scales, qB, qC, stream=None):
    _check("ssd_quantize_bc", LIB.ssd_quantize_bc(ctypes.byref(shape), _p(B), _p(C),
                                                  _scales(scales), _p(qB), _p(qC),
                                                  _stream(stream)))


def ssd_chunk_cumsum(shape, dt, A, dAcs, lut=None, qdecay=None, stream=None):
    _check("ssd_chunk_cumsum", LIB.ssd_chunk_cumsum(ctypes.byref(shape), _p(dt), _p(A),
                                                    _p(dAcs), _p(lut), _p(qdecay),
                                                    _stream(stream)))


def ssd_chunk_state(shape, path, X, lut, Bq, scales, states, taps=None, stream=None):
    _check("ssd_chunk_state", LIB.ssd_chunk_state(ctypes.byref(shape), path, _p(X), _p(lut),
                                                  _p(Bq), _scales(scales), _p(states),
                                                  _taps(taps), _stream(stream)))


def ssd_state_passing(shape, path, states, dAcs=None, qdecay=None, final_state=None,
                      stream=None, initial_state=None):
    _check("ssd_state_passing", LIB.ssd_state_passing(ctypes.byref(shape), path, _p(states),
                                                      _p(dAcs), _p(qdecay), _p(initial_state),
                                                      _p(final_state), _stream(stream)))


def ssd_chunk_bmm(shape, path, Cq, Bq, CB, stream=None):
    _check("ssd_chunk_bmm", LIB.ssd_chunk_bmm(ctypes.byref(shape), path, _p(Cq), _p(Bq), _p(CB),
                                              _stream(stream)))


def ssd_chunk_scan(shape, path, X, dt, dAcs, Cq, CB, states, D, scales, Y, stream=None,
                   initial_state=None):
    _check("ssd_chunk_scan", LIB.ssd_chunk_scan(ctypes.byref(shape), path, _p(X), _p(dt),
                                                _p(dAcs), _p(Cq), _p(CB), _p(states),
                                                _p(initial_state), _p(D), _scales(scales), _p(Y),
                                                _stream(stream)))


def ssd_workspace_bytes(shape, path) -> int:
    return int(LIB.ssd_workspace_bytes(ctypes.byref(shape), path))


def ssd_forward(shape, path, X, dt, A, B, C, D, scales, Y, final_state=None, workspace=None,
                taps=None, stream=None, initial_state=None):
    """Whole forward. ``workspace`` (a uint8 device tensor) is allocated here if None.
    ``initial_state`` continues a sequence from a previous call's final state."""
    need = ssd_workspace_bytes(shape, path)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ssd_forward", LIB.ssd_forward(ctypes.byref(shape), path, _p(X), _p(dt), _p(A), _p(B),
                                          _p(C), _p(D), _scales(scales), _p(Y),
                                          _p(initial_state), _p(final_state), _p(workspace), wsb,
                                          _taps(taps),
                                          _stream(stream)))
    return workspace


def ssd_forward_noalloc(shape, path, X, dt, A, B, C, D, scales, Y, final_state=None, taps=None,
                        stream=None, initial_state=None):
    """Whole forward on the library's fixed device workspace (allocates nothing;
    calls that may overlap on one device race)."""
    _check("ssd_forward_noalloc",
           LIB.ssd_forward_noalloc(ctypes.byref(shape), path, _p(X), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                   _scales(scales), _p(Y), _p(initial_state), _p(final_state),
                                   _taps(taps), _stream(stream)))


def ssd_decode_step(shape, path, X, dt, A, B, C, D, scales, state, Y, stream=None):
    """One position: ``state`` [B,H,P,N] (int8 or fp32) is updated in place,
    Y [B,H,P] receives the output. ``shape.seqlen`` must be 1."""
    _check("ssd_decode_step", LIB.ssd_decode_step(ctypes.byref(shape), path, _p(X), _p(dt), _p(A),
                                                  _p(B), _p(C), _p(D), _scales(scales),
                                                  _p(state), _p(Y), _stream(stream)))


# "Key design 4": the mean correction's coefficient fixed by "Training strategy"
MEAN_CORRECTION_ALPHA = 0.15


def ssd_epilogue(shape, Y, corr, alpha, weight, eps, out, stream=None):
    """RMSNorm over the H*P channels of every position of Y, after adding
    alpha * corr (corr may be None)."""
    _check("ssd_epilogue", LIB.ssd_epilogue(ctypes.byref(shape), _p(Y), _p(corr), float(alpha),
                                            _p(weight), float(eps), _p(out), _stream(stream)))


def ssd_mean_correction(shape, Y_ref, Y_q, c, stream=None):
    """c = per-channel mean of Y_ref - Y_q over all positions."""
    _check("ssd_mean_correction", LIB.ssd_mean_correction(ctypes.byref(shape), _p(Y_ref), _p(Y_q),
                                                          _p(c), _stream(stream)))


def ssd_calibrate_workspace_bytes(shape) -> int:
    return int(LIB.ssd_calibrate_workspace_bytes(ctypes.byref(shape)))


def ssd_calibrate_amax(shape, X, dt, A, B, C, amax, workspace=None, stream=None):
    need = ssd_calibrate_workspace_bytes(shape)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ssd_calibrate_amax", LIB.ssd_calibrate_amax(ctypes.byref(shape), _p(X), _p(dt), _p(A),
                                                        _p(B), _p(C), _p(amax), _p(workspace),
                                                        wsb, _stream(stream)))


def ssd_scales_from_amax(ngroups: int, nheads: int, headdim: int, amax: np.ndarray) -> dict:
    """Host call: the static scale pack from calibration maxima (numpy in, numpy out)."""
    G, HP = ngroups, nheads * headdim
    a = np.ascontiguousarray(amax, dtype=np.float32).reshape(-1)
    if a.size != 2 * G + 2 * HP:
        raise ValueError("amax must hold 2*G + 2*H*P values")
    pack = np.zeros(4 * G + 4 * HP, dtype=np.float32)
    _check("ssd_scales_from_amax", LIB.ssd_scales_from_amax(
        ngroups, nheads, headdim, a.ctypes.data, pack.ctypes.data))
    out, o = {}, 0
    for k, n in (("s_B", G), ("s_C", G), ("inv_B", G), ("inv_C", G),
                 ("s_X", HP), ("inv_X", HP), ("s_S", HP), ("M_req", HP)):
        out[k] = pack[o:o + n].copy()
        o += n
    return out


def calibrate(shape_of, seqs, A, device="cuda") -> ScalePack:
    """Static scales from calibration sequences, on the GPU.

    ``seqs``: iterable of dicts of device tensors x, dt, B, C (one batch each);
    ``shape_of(seq)`` returns the SsdShape of a sequence.
    """
    seqs = list(seqs)
    s0 = shape_of(seqs[0])
    G, H, P = s0.ngroups, s0.nheads, s0.headdim
    amax = torch.zeros(2 * G + 2 * H * P, dtype=torch.float32, device=device)
    for sq in seqs:
        ssd_calibrate_amax(shape_of(sq), sq["x"], sq["dt"], A, sq["B"], sq["C"], amax)
    host = amax.cpu().numpy()
    return ScalePack(ssd_scales_from_amax(G, H, P, host), device)
