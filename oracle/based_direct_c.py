"""ctypes wrapper of oracle/based_direct.c: the causal Based forward by its definition in plain C (float64).

TEST INFRASTRUCTURE ONLY (see based_oracle.py). The library is compiled by `build()` below (called from
`__graft_entry__.build()`); gcc with OpenMP, -O3 without fast-math and without contracting
a * b + c into one fused operation, so every operation is an IEEE float64 operation in the order the
source states.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .based_oracle import resolve_scale

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "based_direct.c")
LIB = os.path.join(HERE, "libbased_direct.so")

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build() (or oracle.based_direct_c.build())")
        lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.based_direct_rows.restype = ctypes.c_int
        lib.based_direct_rows.argtypes = [p, p, p, i64, i64, i64, i64, i64, ctypes.c_double, p, i64, p]
        _lib = lib
    return _lib


def based_ref_direct_c(qb, kb, vb, scale=None, rows=None):
    """The definition (field spec_md) for bfloat16 bit arrays qb, kb (B, T, H, K) and vb (B, T, H, V) (uint16).
    rows: positions t to evaluate for every (b, h), or None for all. Returns float64 (B, len(rows) or T, H, V)."""
    qb = np.ascontiguousarray(qb, dtype=np.uint16)
    kb = np.ascontiguousarray(kb, dtype=np.uint16)
    vb = np.ascontiguousarray(vb, dtype=np.uint16)
    B, T, H, K = qb.shape
    V = vb.shape[-1]
    assert kb.shape == qb.shape and vb.shape[:3] == (B, T, H)
    sigma = resolve_scale(scale, K)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = T if r is None else len(r)
    out = np.empty((B, n, H, V), dtype=np.float64)
    rc = _load().based_direct_rows(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, B, T, H, K, V, sigma,
                                   None if r is None else r.ctypes.data, n, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"based_direct_rows failed ({rc}: -1 bad arguments, -2 out of memory)")
    return out
