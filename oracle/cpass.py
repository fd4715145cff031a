"""Build and call the float64 C oracle of the whole pass (collapsed form; oracle/collapsed_pass.c).
TEST INFRASTRUCTURE ONLY: used by the tests and by the benchmark's CPU-baseline leg.

`pass_units` runs score, selection and gather for a list of units held in host arrays, with a given number of
OpenMP threads; the NumPy oracle (oracle/__init__.py) pins its results in tests/test_oracle_cpass.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "collapsed_pass.c")
LIB = os.path.join(HERE, "libcollapsed.so")
CFLAGS = ["-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall"]

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        L.tri_oracle_collapsed_pass.restype = ctypes.c_int
        L.tri_oracle_collapsed_pass.argtypes = [ctypes.c_int, p, p, p, p, p, p, p, p, ctypes.c_int, ctypes.c_double,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                p, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def pass_units(K, V, pos, lengths, u, chat, t, theta, budget, recent, rope="half", threads=0, outputs=True):
    """The pass over n units given as concatenated rows.

    K, V: uint16 [rows, d] bf16 bit patterns; pos int32 [rows]; lengths int [n] (rows of each unit, in order);
    u float64 [n, d]; chat float64 [n, d/2]; t int [n].  Returns a dict with scores (float64 [rows]), keep
    (int32 [n, budget]), k, v ([n, budget, d] uint16), pos ([n, budget] int32), new_len (int32 [n]); with
    outputs=False only new_len (for timing).
    """
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    n, d = lengths.shape[0], K.shape[1]
    row0 = np.ascontiguousarray(np.concatenate([[0], np.cumsum(lengths, dtype=np.int64)[:-1]]), dtype=np.int64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    chat = np.ascontiguousarray(chat, dtype=np.float64)
    t = np.ascontiguousarray(t, dtype=np.int32)
    out = {"new_len": np.zeros(n, dtype=np.int32)}
    if outputs:
        out.update(scores=np.full(K.shape[0], np.nan), keep=np.full((n, budget), -1, dtype=np.int32),
                   k=np.zeros((n, budget, d), dtype=np.uint16), v=np.zeros((n, budget, d), dtype=np.uint16),
                   pos=np.full((n, budget), -1, dtype=np.int32))
    rc = lib().tri_oracle_collapsed_pass(n, _ptr(lengths), _ptr(row0), _ptr(K), _ptr(V), _ptr(pos), _ptr(u),
                                         _ptr(chat), _ptr(t), d, float(theta), 1 if rope == "half" else 0, budget,
                                         recent, threads, _ptr(out.get("scores")), _ptr(out.get("keep")),
                                         _ptr(out.get("k")), _ptr(out.get("v")), _ptr(out.get("pos")),
                                         _ptr(out["new_len"]))
    if rc != 0:
        raise ValueError("tri_oracle_collapsed_pass rejected its arguments")
    return out
