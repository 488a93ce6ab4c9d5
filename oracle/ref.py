"""ctypes front end of the C oracle (oracle.c).  Test infrastructure only.

Every function takes and returns NumPy arrays.  Failing argument checks raise
ValueError (the C side returns -2 for bad sizes, -3 for an expert id outside
[0, E)).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the front end at another build of oracle.c (the mutation
# check of the pins runs the pin suite against deliberately broken copies).
lib_path = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            from . import build as _b
            _b.build()
        L = C.CDLL(lib_path)
        P = C.c_void_p
        i = C.c_int
        L.oracle_e4m3_value.restype = C.c_double
        L.oracle_e4m3_value.argtypes = [C.c_uint8]
        L.oracle_e8m0_value.restype = C.c_double
        L.oracle_e8m0_value.argtypes = [C.c_uint8]
        L.oracle_dequant.restype = C.c_double
        L.oracle_dequant.argtypes = [C.c_uint8, C.c_uint8]
        L.oracle_e4m3_table.argtypes = [P]
        L.oracle_e8m0_table.argtypes = [P]
        L.oracle_bf16_value.restype = C.c_double
        L.oracle_bf16_value.argtypes = [C.c_uint16]
        L.oracle_round_f32.restype = C.c_float
        L.oracle_round_f32.argtypes = [C.c_double]
        L.oracle_bf16_rne.restype = C.c_uint16
        L.oracle_bf16_rne.argtypes = [C.c_float]
        L.oracle_silu.restype = C.c_double
        L.oracle_silu.argtypes = [C.c_double]
        L.oracle_gate_up.restype = i
        L.oracle_gate_up.argtypes = [P, P, P, P, i, i, i, i, i, P, P, P, i]
        L.oracle_down.restype = i
        L.oracle_down.argtypes = [P, P, P, P, P, i, i, i, i, i, P, i]
        L.oracle_moe_decode.restype = i
        L.oracle_moe_decode.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, P, i]
        L.oracle_max_threads.restype = i
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [C.c_double]
        L.oracle_mxfp8_quantize.argtypes = [P, C.c_long, P, P]
        L.oracle_moe_decode_exact.restype = i
        L.oracle_moe_decode_exact.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i]
        L.oracle_moe_decode_conventional.restype = i
        L.oracle_moe_decode_conventional.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i]
        L.oracle_route.restype = i
        L.oracle_route.argtypes = [P, i, i, i, P, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _rc(rc):
    if rc == -2:
        raise ValueError("oracle: bad sizes (need K>=1, E>=1, H and I multiples of 32)")
    if rc == -3:
        raise ValueError("oracle: expert id outside [0, E)")
    if rc:
        raise ValueError(f"oracle: error {rc}")


def e4m3_table() -> np.ndarray:
    out = np.empty(256, np.float64)
    _load().oracle_e4m3_table(_p(out))
    return out


def e8m0_table() -> np.ndarray:
    out = np.empty(256, np.float64)
    _load().oracle_e8m0_table(_p(out))
    return out


def dequant(code: int, scale: int) -> float:
    return _load().oracle_dequant(code, scale)


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def round_f32(v: float) -> float:
    return _load().oracle_round_f32(v)


def bf16_rne(f: float) -> int:
    return _load().oracle_bf16_rne(f)


def silu(g: float) -> float:
    return _load().oracle_silu(g)


def _dims(layer_arrays, x_or_act_shape=None):
    wgu, sgu, wd, sd = layer_arrays
    E, I2, H = wgu.shape
    return E, H, I2 // 2


def gate_up(x, ids, wgu, sgu, nthreads: int = 0, return_gu: bool = False):
    """act[B,K,I] BF16 bits (and optionally FP64 g, u) from x[B,H] bits."""
    x = _c(x, np.uint16); ids = _c(ids, np.int32)
    wgu = _c(wgu, np.uint8); sgu = _c(sgu, np.uint8)
    E, I2, H = wgu.shape
    I = I2 // 2
    B, K = ids.shape
    assert x.shape == (B, H) and sgu.shape == (E, I2, H // 32)
    act = np.empty((B, K, I), np.uint16)
    g = np.empty((B, K, I), np.float64) if return_gu else None
    u = np.empty((B, K, I), np.float64) if return_gu else None
    _rc(_load().oracle_gate_up(_p(x), _p(ids), _p(wgu), _p(sgu), B, K, E, H, I, _p(act),
                               _p(g) if return_gu else None, _p(u) if return_gu else None, nthreads))
    return (act, g, u) if return_gu else act


def down(act, ids, w, wd, sd, nthreads: int = 0):
    """y[B,H] FP64 from a given intermediate act[B,K,I] (BF16 bits)."""
    act = _c(act, np.uint16); ids = _c(ids, np.int32); w = _c(w, np.float32)
    wd = _c(wd, np.uint8); sd = _c(sd, np.uint8)
    E, H, I = wd.shape
    B, K = ids.shape
    assert act.shape == (B, K, I) and w.shape == (B, K) and sd.shape == (E, H, I // 32)
    y = np.empty((B, H), np.float64)
    _rc(_load().oracle_down(_p(act), _p(ids), _p(w), _p(wd), _p(sd), B, K, E, H, I, _p(y), nthreads))
    return y


def moe_decode(x, ids, w, wgu, sgu, wd, sd, nthreads: int = 0):
    """(y[B,H] FP64, act[B,K,I] BF16 bits) for the whole layer."""
    x = _c(x, np.uint16); ids = _c(ids, np.int32); w = _c(w, np.float32)
    wgu = _c(wgu, np.uint8); sgu = _c(sgu, np.uint8); wd = _c(wd, np.uint8); sd = _c(sd, np.uint8)
    E, I2, H = wgu.shape
    I = I2 // 2
    B, K = ids.shape
    assert wd.shape == (E, H, I)
    act = np.empty((B, K, I), np.uint16)
    y = np.empty((B, H), np.float64)
    _rc(_load().oracle_moe_decode(_p(x), _p(ids), _p(w), _p(wgu), _p(sgu), _p(wd), _p(sd),
                                  B, K, E, H, I, _p(act), _p(y), nthreads))
    return y, act


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(v)


def mxfp8_quantize(v):
    """(codes uint8, scales uint8) of FP64 values along the last axis (OCP MX rule)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.shape[-1] % 32 == 0
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    _load().oracle_mxfp8_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def _layer_call(fn, x, ids, w, wgu, sgu, wd, sd, nthreads):
    x = _c(x, np.uint16); ids = _c(ids, np.int32); w = _c(w, np.float32)
    wgu = _c(wgu, np.uint8); sgu = _c(sgu, np.uint8); wd = _c(wd, np.uint8); sd = _c(sd, np.uint8)
    E, I2, H = wgu.shape
    B, K = ids.shape
    if H > 8192 or I2 // 2 > 16384:
        raise ValueError("oracle: H <= 8192 and I <= 16384 for the accuracy functions")
    y = np.empty((B, H), np.float64)
    _rc(fn(_p(x), _p(ids), _p(w), _p(wgu), _p(sgu), _p(wd), _p(sd), B, K, E, H, I2 // 2, _p(y), nthreads))
    return y


def moe_decode_exact(x, ids, w, wgu, sgu, wd, sd, nthreads: int = 0):
    """Reference y[B,H] in FP64 with no rounding of the intermediate or output."""
    return _layer_call(_load().oracle_moe_decode_exact, x, ids, w, wgu, sgu, wd, sd, nthreads)


def moe_decode_conventional(x, ids, w, wgu, sgu, wd, sd, nthreads: int = 0):
    """y[B,H] (BF16 values) with the conventional path's activation rounding
    (x and the intermediate through MXFP8, per-expert outputs in BF16)."""
    return _layer_call(_load().oracle_moe_decode_conventional, x, ids, w, wgu, sgu, wd, sd, nthreads)


def route(logits, K: int):
    """(ids [B,K] int32, w [B,K] FP64): top-K of each row of logits [B,E]
    (larger first, ties to the lower index) and the softmax over the chosen K."""
    logits = _c(logits, np.float32)
    B, E = logits.shape
    ids = np.empty((B, K), np.int32)
    w = np.empty((B, K), np.float64)
    _rc(_load().oracle_route(_p(logits), B, E, K, _p(ids), _p(w)))
    return ids, w


def max_threads() -> int:
    return _load().oracle_max_threads()


def moe_decode_dense_weights(x, ids, w, gu_of, dn_of):
    """Reference y[B,H] in FP64 of the layer with arbitrary real weights: for
    token b, y[b] = sum_k w[b,k] * Wd_e (SiLU(Wg_e x[b]) * (Wu_e x[b])) with
    e = ids[b,k], no rounding anywhere.  gu_of(e) gives expert e's gate/up
    rows [2I, H] (gate rows first) and dn_of(e) its down rows [H, I], any
    float dtype; each expert's weights are fetched once, for all the slots
    that chose it.  Used with the weights as drawn before MXFP8 quantization,
    it is the full-precision reference of the accuracy experiment."""
    xb = np.asarray(x, np.uint16).astype(np.uint32) << 16
    xf = xb.view(np.float32).astype(np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, np.float64)
    y = None
    for e in np.unique(ids):
        bs, ks = np.nonzero(ids == e)
        gu = np.asarray(gu_of(int(e)), np.float64)
        dn = np.asarray(dn_of(int(e)), np.float64)
        I = gu.shape[0] // 2
        xs = xf[bs]                                   # [n, H], one row per slot
        g = xs @ gu[:I].T
        u = xs @ gu[I:].T
        a = g / (1.0 + np.exp(-g)) * u                # SiLU(g) * u, [n, I]
        if y is None:
            y = np.zeros((ids.shape[0], dn.shape[0]))
        np.add.at(y, bs, w[bs, ks][:, None] * (a @ dn.T))
    return y
