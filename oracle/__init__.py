"""TAH-Quant reference oracle (ctypes loader) — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never does. It loads ``liboracle_tah.so`` built
from ``tah_ref.c`` (plain C, single thread) and wraps it for numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtahref.so")
SRC_PATH = os.path.join(_HERE, "tah_ref.c")

F32 = 0
BF16 = 1

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "BUFFER_TOO_SMALL", 4: "BUDGET_INFEASIBLE", 5: "BAD_PAYLOAD"}


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {STATUS.get(code, code)}")
        self.code = code


class _Params(ctypes.Structure):
    _fields_ = [
        ("tile", ctypes.c_int32),
        ("tokens_per_sample", ctypes.c_int32),
        ("bit_budget", ctypes.c_float),
        ("n_candidates", ctypes.c_int32),
        ("candidates", ctypes.c_uint8 * 4),
        ("tau", ctypes.c_float),
        ("alloc_tile", ctypes.c_int32),
        ("allocator", ctypes.c_int32),
    ]


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("tokens", "hidden", "S", "nsamples", "M", "tiles", "tiles_per_sample", "nblocks")] + [
        (n, ctypes.c_int32) for n in ("G", "log2G", "b_lo", "b_hi")
    ] + [(n, ctypes.c_int64) for n in ("k", "off_table", "off_bitmap", "off_side", "off_scale", "off_zero", "off_codes", "code_bytes", "total",
                                  "A", "kA", "MA", "atiles", "atiles_per_sample", "allocator", "R")]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: no fast-math and no FMA contraction, so each
    fp32 operation rounds once in the written order."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, SRC_PATH, "-lm"]
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.tahref_plan_make.argtypes = [ctypes.c_int64, ctypes.c_int64, P(_Params), P(_Plan)]
        L.tahref_log2s.argtypes = [ctypes.c_float]
        L.tahref_log2s.restype = ctypes.c_float
        L.tahref_fwht.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.tahref_entropy.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.tahref_entropy.restype = ctypes.c_float
        L.tahref_alloc_entropy.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        L.tahref_alloc_entropy.restype = ctypes.c_float
        L.tahref_outlier.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float, P(ctypes.c_int), P(ctypes.c_float), P(ctypes.c_float)]
        L.tahref_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, P(ctypes.c_float), P(ctypes.c_float), ctypes.c_void_p]
        L.tahref_dequantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.tahref_allocate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.tahref_greedy_lambda.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.tahref_allocate_greedy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.tahref_encode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P(_Params), ctypes.c_void_p, ctypes.c_size_t]
        L.tahref_decode.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int64, P(_Params), ctypes.c_void_p, ctypes.c_int]
        L.tahref_tile_stats.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P(_Params)] + [ctypes.c_void_p] * 6
        L.tahref_naive_payload_bytes.argtypes = [ctypes.c_int64, ctypes.c_int, P(ctypes.c_size_t)]
        L.tahref_naive_quantize.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_float, P(ctypes.c_int32)]
        L.tahref_naive_dequantize.argtypes = [ctypes.c_int32, ctypes.c_int, ctypes.c_float]
        L.tahref_naive_dequantize.restype = ctypes.c_float
        L.tahref_naive_encode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t]
        L.tahref_naive_decode.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        _lib = L
    return _lib


def _params(p) -> _Params:
    c = _Params()
    c.tile = int(p.tile)
    c.tokens_per_sample = int(p.tokens_per_sample)
    c.bit_budget = float(p.bit_budget)
    cands = tuple(p.candidates)
    c.n_candidates = len(cands)
    for i in range(4):
        c.candidates[i] = int(cands[i]) if i < len(cands) else 0
    c.tau = float(p.tau)
    c.alloc_tile = int(getattr(p, "alloc_tile", 0))
    c.allocator = int(getattr(p, "allocator", 0))
    return c


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("input must be float32 or uint16 (bf16 bits)")


def plan(tokens: int, hidden: int, p) -> dict:
    pl = _Plan()
    cp = _params(p)
    rc = lib().tahref_plan_make(tokens, hidden, ctypes.byref(cp), ctypes.byref(pl))
    if rc:
        raise OracleError(rc, "plan")
    return {n: getattr(pl, n) for n, _ in _Plan._fields_}


def log2s(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.float32).ravel()
    f = lib().tahref_log2s
    return np.array([f(float(v)) for v in u], dtype=np.float32)


def fwht(v: np.ndarray) -> np.ndarray:
    v = np.array(v, dtype=np.float32, copy=True)
    lib().tahref_fwht(_ptr(v), v.size)
    return v


def entropy(alpha: np.ndarray) -> float:
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    return float(np.float32(lib().tahref_entropy(_ptr(a), a.size)))


def alloc_entropy(alpha: np.ndarray, G: int) -> float:
    """Entropy of one allocation tile of alpha.size = kA * G channels."""
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    assert a.size % G == 0
    return float(np.float32(lib().tahref_alloc_entropy(_ptr(a), a.size, int(G))))


def outlier(alpha: np.ndarray, tau: float):
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    d = ctypes.c_int()
    m1 = ctypes.c_float()
    m2 = ctypes.c_float()
    f = lib().tahref_outlier(_ptr(a), a.size, float(tau), ctypes.byref(d), ctypes.byref(m1), ctypes.byref(m2))
    return bool(f), d.value, np.float32(m1.value), np.float32(m2.value)


def quantize(y: np.ndarray, b: int):
    y = np.ascontiguousarray(y, dtype=np.float32)
    q = np.zeros(y.size, dtype=np.uint32)
    lo = ctypes.c_float()
    s = ctypes.c_float()
    lib().tahref_quantize(_ptr(y), y.size, int(b), ctypes.byref(lo), ctypes.byref(s), _ptr(q))
    return np.float32(lo.value), np.float32(s.value), q


def dequantize(q: np.ndarray, s: float, lo: float, flag: bool, d: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint32)
    out = np.zeros(q.size, dtype=np.float32)
    lib().tahref_dequantize(_ptr(q), q.size, float(s), float(lo), int(bool(flag)), int(d), _ptr(out))
    return out


def allocate(H: np.ndarray, k: int) -> np.ndarray:
    H = np.ascontiguousarray(H, dtype=np.float32)
    hi = np.zeros(H.size, dtype=np.uint8)
    rc = lib().tahref_allocate(_ptr(H), H.size, int(k), _ptr(hi))
    if rc:
        raise OracleError(rc, "allocate")
    return hi


def greedy_lambda(cands) -> np.ndarray:
    """The n-1 per-upgrade constants lambda_j of the greedy allocator (fp32)."""
    c = np.ascontiguousarray(cands, dtype=np.uint8)
    lam = np.zeros(max(c.size - 1, 1), np.float32)
    rc = lib().tahref_greedy_lambda(c.size, _ptr(c), _ptr(lam))
    if rc:
        raise OracleError(rc, "greedy_lambda")
    return lam[: c.size - 1]


def allocate_greedy(H: np.ndarray, cands, R: int) -> np.ndarray:
    """Candidate index of each of the H.size allocation tiles of one sample."""
    H = np.ascontiguousarray(H, dtype=np.float32)
    c = np.ascontiguousarray(cands, dtype=np.uint8)
    level = np.zeros(H.size, dtype=np.uint8)
    rc = lib().tahref_allocate_greedy(_ptr(H), H.size, c.size, _ptr(c), int(R), _ptr(level))
    if rc:
        raise OracleError(rc, "allocate_greedy")
    return level


def encode(x: np.ndarray, p) -> np.ndarray:
    x = np.ascontiguousarray(x)
    tokens, hidden = x.shape
    pl = plan(tokens, hidden, p)
    out = np.zeros(pl["total"], dtype=np.uint8)
    cp = _params(p)
    rc = lib().tahref_encode(_ptr(x), _dtype_of(x), tokens, hidden, ctypes.byref(cp), _ptr(out), out.size)
    if rc:
        raise OracleError(rc, "encode")
    return out


def decode(payload: np.ndarray, tokens: int, hidden: int, p, y_dtype: int = F32) -> np.ndarray:
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    y = np.zeros((tokens, hidden), dtype=np.float32 if y_dtype == F32 else np.uint16)
    cp = _params(p)
    rc = lib().tahref_decode(_ptr(payload), payload.size, tokens, hidden, ctypes.byref(cp), _ptr(y), int(y_dtype))
    if rc:
        raise OracleError(rc, "decode")
    return y


def tile_stats(x: np.ndarray, p) -> dict:
    x = np.ascontiguousarray(x)
    tokens, hidden = x.shape
    pl = plan(tokens, hidden, p)
    n = pl["tiles"]
    H = np.zeros(pl["atiles"], np.float32)
    flag = np.zeros(n, np.uint8)
    piv = np.zeros(n, np.uint8)
    hi = np.zeros(n, np.uint8)
    lo = np.zeros(n, np.float32)
    sc = np.zeros(n, np.float32)
    cp = _params(p)
    rc = lib().tahref_tile_stats(_ptr(x), _dtype_of(x), tokens, hidden, ctypes.byref(cp), _ptr(H), _ptr(flag), _ptr(piv), _ptr(hi), _ptr(lo), _ptr(sc))
    if rc:
        raise OracleError(rc, "tile_stats")
    return dict(H=H, flag=flag, pivot=piv, hi=hi, lo=lo, scale=sc)


# ---------------------------------------------------------------- backward compressor (Q_Naive) ----
def naive_payload_bytes(n: int, bits: int) -> int:
    out = ctypes.c_size_t()
    rc = lib().tahref_naive_payload_bytes(int(n), int(bits), ctypes.byref(out))
    if rc:
        raise OracleError(rc, "naive_payload_bytes")
    return out.value


def naive_quantize(g, bits: int, c: float) -> np.ndarray:
    g = np.asarray(g, dtype=np.float32).ravel()
    q = ctypes.c_int32()
    out = np.zeros(g.size, dtype=np.int32)
    f = lib().tahref_naive_quantize
    for i, v in enumerate(g):
        rc = f(float(v), int(bits), float(np.float32(c)), ctypes.byref(q))
        if rc:
            raise OracleError(rc, "naive_quantize")
        out[i] = q.value
    return out


def naive_dequantize(q, bits: int, c: float) -> np.ndarray:
    q = np.asarray(q, dtype=np.int32).ravel()
    f = lib().tahref_naive_dequantize
    return np.array([f(int(v), int(bits), float(np.float32(c))) for v in q], dtype=np.float32)


def naive_encode(g: np.ndarray, bits: int, c: float) -> np.ndarray:
    g = np.ascontiguousarray(g)
    out = np.zeros(naive_payload_bytes(g.size, bits), dtype=np.uint8)
    rc = lib().tahref_naive_encode(_ptr(g), _dtype_of(g), g.size, int(bits), float(np.float32(c)), _ptr(out), out.size)
    if rc:
        raise OracleError(rc, "naive_encode")
    return out


def naive_decode(payload: np.ndarray, n: int, bits: int, c: float, y_dtype: int = F32) -> np.ndarray:
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    y = np.zeros(n, dtype=np.float32 if y_dtype == F32 else np.uint16)
    rc = lib().tahref_naive_decode(_ptr(payload), payload.size, int(n), int(bits), float(np.float32(c)), _ptr(y), int(y_dtype))
    if rc:
        raise OracleError(rc, "naive_decode")
    return y
