"""CPU fp64 oracle of the token-choice top-k MoE feed-forward layer forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  The product
path (the HIP library and its binding) never imports it, and the two share no
code: the only common module is ``workloads`` (seeded input draws, no layer
arithmetic).

The arithmetic lives in ``moe_oracle.c`` (plain C loops in double precision,
compiled with gcc); this file marshals numpy arrays.  Which passage of the
pages each step follows is written beside that step in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16 = 0, 1
SWIGLU, RELU = 0, 1
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.oracle_forward.argtypes = [I64, I64, I64, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P,
                                       I64, P, P, P, P, P, P, I32]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_combine.argtypes = [I64, I32, I64, I32, I32, P, P, P, P, P]
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_param_count.argtypes = [I64, I64, I32, I32, I32, I32]
        lib.oracle_param_count.restype = ctypes.c_int64
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 bf16 bit patterns, got %s" % a.dtype)


def forward(x, router, gate_up, down, *, top_k, norm=True, act="swiglu", router_bias=None,
            up_bias=None, down_bias=None, tokens=None, forced_sel=None, nthreads=None) -> dict:
    """Layer forward on the CPU in fp64.

    x (T,D), router (E,D), gate_up (E,G*F,D), down (E,D,F) share one dtype:
    float32, or uint16 holding bf16 bits.  Biases are float32 or None.
    ``tokens`` evaluates only those rows of x; ``forced_sel`` (n,K) replays a
    selection.  Returns out (n,D), sel (n,K) int64, weights (n,K), logits
    (n,E), probs (n,E), all float64 except sel.
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    x2 = x.reshape(-1, x.shape[-1])
    T, D = x2.shape
    router, gate_up, down = (np.ascontiguousarray(a) for a in (router, gate_up, down))
    E = router.shape[0]
    G = 2 if act == "swiglu" else 1
    F = down.shape[2]
    dt = _dtype_code(x2)
    for a in (router, gate_up, down):
        if _dtype_code(a) != dt:
            raise TypeError("x and the weights must share a dtype")
    if router.shape != (E, D) or gate_up.shape != (E, G * F, D) or down.shape != (E, D, F):
        raise ValueError("weight shapes do not match router (E,D), gate_up (E,G*F,D), down (E,D,F)")
    rb, ub, db = (None if b is None else np.ascontiguousarray(b, dtype=np.float32)
                  for b in (router_bias, up_bias, down_bias))
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tokens.shape[0]
    else:
        n = T
    if forced_sel is not None:
        forced_sel = np.ascontiguousarray(forced_sel, dtype=np.int64).reshape(n, top_k)
    out = np.empty((n, D), np.float64)
    sel = np.empty((n, top_k), np.int64)
    w = np.empty((n, top_k), np.float64)
    logits = np.empty((n, E), np.float64)
    probs = np.empty((n, E), np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = lib.oracle_forward(T, D, F, E, top_k, int(bool(norm)), SWIGLU if act == "swiglu" else RELU, dt,
                            _ptr(x2), _ptr(router), _ptr(gate_up), _ptr(down), _ptr(rb), _ptr(ub), _ptr(db),
                            _ptr(tokens), n, _ptr(forced_sel), _ptr(out), _ptr(sel), _ptr(w), _ptr(logits),
                            _ptr(probs), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_forward failed with code %d" % rc)
    return dict(out=out, sel=sel, weights=w, logits=logits, probs=probs, nthreads=int(min(nthreads, max(n, 1))))


def forward_inputs(inp: dict, **kw) -> dict:
    """forward() on a dict produced by ``workloads.generate``."""
    c = inp["cfg"]
    return forward(inp["x"], inp["router"], inp["gate_up"], inp["down"], top_k=c["K"], norm=c["norm"],
                   act=c["act"], router_bias=inp.get("router_bias"), up_bias=inp.get("up_bias"),
                   down_bias=inp.get("down_bias"), **kw)


def combine(probs, expert_outs, *, top_k, norm=True) -> dict:
    """Selection, weights and weighted sum from given probs (T,E) and expert outputs (T,E,D)."""
    lib = _load()
    probs = np.ascontiguousarray(probs, dtype=np.float64)
    eo = np.ascontiguousarray(expert_outs, dtype=np.float64)
    T, E = probs.shape
    D = eo.shape[2]
    if eo.shape != (T, E, D):
        raise ValueError("expert_outs must be (T,E,D)")
    sel = np.empty((T, top_k), np.int64)
    w = np.empty((T, top_k), np.float64)
    out = np.empty((T, D), np.float64)
    rc = lib.oracle_combine(T, E, D, top_k, int(bool(norm)), _ptr(probs), _ptr(eo), _ptr(sel), _ptr(w), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_combine failed with code %d" % rc)
    return dict(sel=sel, weights=w, out=out)


def param_count(D, F, E, *, act="swiglu", expert_biases=False, router_bias=False) -> int:
    return int(_load().oracle_param_count(D, F, E, SWIGLU if act == "swiglu" else RELU,
                                          int(bool(expert_biases)), int(bool(router_bias))))
