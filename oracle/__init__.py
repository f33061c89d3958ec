"""ctypes wrapper around the plain C++ CPU oracle (oracle/oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may import this package; the HIP library and its Python binding never
do. The oracle shares no code with the HIP path.

Every function takes and returns numpy arrays. bf16 values travel as uint16 bit
patterns; expert weights travel in their logical (unpacked) form:
q uint8 0..15, scale and bias bf16 bits, one (scale, bias) per 64 inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at a deliberately broken build of the oracle.
_LIB = os.environ.get("MOE_ORACLE_LIB", _DEFAULT_LIB)
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ (-O2, OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_DEFAULT_LIB):
        tmp = _DEFAULT_LIB + ".tmp"
        cmd = ["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def _declare(L):
    L.oracle_max_threads.restype = _INT
    L.oracle_dequant.argtypes = [_P, _P, _P, _I64, _I64, _P]
    L.oracle_router_logits.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _INT]
    L.oracle_topk.argtypes = [_P, _I64, _I64, _I64, _INT, _P, _P]
    L.oracle_route_meta.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                    _P, _I64, _P]
    L.oracle_expert_ffn.argtypes = [_P, _I64, _I64] + [_P] * 9 + [_P]
    L.oracle_layer.argtypes = ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P] + [_P] * 9
                               + [_P, _I64, _INT, _P, _P, _P, _P, _INT])
    L.oracle_layer_dense_masked.argtypes = ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P]
                                            + [_P] * 9 + [_P, _INT])
    for name in ("oracle_dequant", "oracle_router_logits", "oracle_topk",
                 "oracle_route_meta", "oracle_expert_ffn", "oracle_layer",
                 "oracle_layer_dense_masked"):
        getattr(L, name).restype = _INT


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def dequant(q, scale, bias):
    """w[n][c] = q[n][c]*scale[n][c//64] + bias[n][c//64], in float64."""
    q = _c(q, np.uint8)
    scale = _c(scale, np.uint16)
    bias = _c(bias, np.uint16)
    rows, cols = q.shape
    w = np.empty((rows, cols), np.float64)
    _check(lib().oracle_dequant(_ptr(q), _ptr(scale), _ptr(bias), rows, cols, _ptr(w)),
           "oracle_dequant")
    return w


def router_logits(x, wr, rbias=None, nthreads=0):
    x = _c(x, np.uint16)
    wr = _c(wr, np.float32)
    rbias = _c(rbias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    _check(lib().oracle_router_logits(_ptr(x), _ptr(wr), _ptr(rbias), T, H, E,
                                      _ptr(out), nthreads), "oracle_router_logits")
    return out


def topk(logits, k, alt_swap=False):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib().oracle_topk(_ptr(logits), T, E, k, int(alt_swap), _ptr(idx), _ptr(w)),
           "oracle_topk")
    return idx, w


def max_blocks(T, k, E, BM):
    return (T * k + BM - 1) // BM + E


def route_meta(idx, E, BM):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    mb = max_blocks(T, k, E, BM)
    hist = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv_perm = np.empty(T * k, np.int32)
    block_map = np.zeros((mb, 3), np.int32)
    nb = np.zeros(1, np.int32)
    _check(lib().oracle_route_meta(_ptr(idx), T, E, k, BM, _ptr(hist), _ptr(offsets),
                                   _ptr(perm), _ptr(inv_perm), _ptr(block_map), mb,
                                   _ptr(nb)), "oracle_route_meta")
    return dict(hist=hist, offsets=offsets, perm=perm, inv_perm=inv_perm,
                block_map=block_map[: int(nb[0])].copy(), num_blocks=int(nb[0]))


def expert_ffn(xrow, gate, up, down):
    """One SwiGLU expert on one token. gate/up/down are (q, scale, bias) tuples."""
    xrow = _c(xrow, np.uint16)
    H = xrow.shape[0]
    I = gate[0].shape[0]
    mats = []
    for (q, s, b) in (gate, up, down):
        mats += [_c(q, np.uint8), _c(s, np.uint16), _c(b, np.uint16)]
    out = np.empty(H, np.float64)
    _check(lib().oracle_expert_ffn(_ptr(xrow), H, I, *[_ptr(m) for m in mats], _ptr(out)),
           "oracle_expert_ffn")
    return out


def _layer_args(w):
    """Flatten a synth.LayerWeights into the oracle's expert arrays (E+1 experts)."""
    mats = []
    for m in ("gate", "up", "down"):
        mats += [_c(w.q[m], np.uint8), _c(w.scale[m], np.uint16), _c(w.bias[m], np.uint16)]
    return mats


def layer(x, w, k=8, tokens=None, alt_swap=False, nthreads=0):
    """The whole layer for the listed tokens (all when None).

    Returns dict(y float64 [n,H], logits float32 [n,E], idx int32 [n,k], w float32 [n,k]).
    """
    x = _c(x, np.uint16)
    T, H = x.shape
    E = w.E
    I = w.I
    toks = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = T if toks is None else toks.shape[0]
    mats = _layer_args(w)
    y = np.empty((n, H), np.float64)
    logits = np.empty((n, E), np.float32)
    idx = np.empty((n, k), np.int32)
    wsel = np.empty((n, k), np.float32)
    wr = _c(w.router_w, np.float32)
    rb = _c(w.router_bias, np.float32)
    _check(lib().oracle_layer(_ptr(x), T, H, I, E, k, _ptr(wr), _ptr(rb),
                              *[_ptr(m) for m in mats], _ptr(toks), n, int(alt_swap),
                              _ptr(logits), _ptr(idx), _ptr(wsel), _ptr(y), nthreads),
           "oracle_layer")
    return dict(y=y, logits=logits, idx=idx, w=wsel)


def layer_dense_masked(x, w, k=8, nthreads=0):
    x = _c(x, np.uint16)
    T, H = x.shape
    mats = _layer_args(w)
    y = np.empty((T, H), np.float64)
    wr = _c(w.router_w, np.float32)
    rb = _c(w.router_bias, np.float32)
    _check(lib().oracle_layer_dense_masked(_ptr(x), T, H, w.I, w.E, k, _ptr(wr), _ptr(rb),
                                           *[_ptr(m) for m in mats], _ptr(y), nthreads),
           "oracle_layer_dense_masked")
    return y
