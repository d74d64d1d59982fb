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
# MOE_ORACLE_LIB selects another build of the same source (the sanitizer
# build of the test suite); it is loaded as it is, never rebuilt here.
_LIB_ENV = os.environ.get("MOE_ORACLE_LIB")
_LIB = _LIB_ENV or os.path.join(_HERE, "libmoe_oracle.so")

# Flags of the AddressSanitizer + UndefinedBehaviorSanitizer build: any report
# aborts the process (no recovery), frames are kept for the report.
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]

F32, BF16 = 0, 1
SWIGLU, RELU = 0, 1
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if _LIB_ENV:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile the same source with AddressSanitizer and UBSan into ``path``
    (host code only; load it with the ASan runtime preloaded)."""
    subprocess.check_call(["gcc", *SANITIZE_FLAGS, "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                           "-shared", "-fPIC", "-pthread", _SRC, "-o", path, "-lm"])
    return path


def _load():
    global _lib
    if _lib is None:
        if not _LIB_ENV and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
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
        lib.oracle_route.argtypes = [I64, I64, I32, I32, I32, I32, P, P, P, P, I64, P, P, ctypes.c_double, P, P, P,
                                     P, P, I32]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_capacity_slots.argtypes = [I64, I32, I32, ctypes.c_double]
        lib.oracle_capacity_slots.restype = ctypes.c_int64
        lib.oracle_capacity.argtypes = [I64, I32, I32, I64, I64, P, P]
        lib.oracle_capacity.restype = ctypes.c_int
        lib.oracle_experts.argtypes = [I64, I64, I64, I32, I32, I32, I32, P, P, P, P, P, P, I64, P, P, P, P, I32]
        lib.oracle_experts.restype = ctypes.c_int
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


# ------------------------------------------------------------ routing options
def route(x, router, *, top_k, norm=True, router_bias=None, tokens=None, replay=None, replay_mask=None,
          threshold=0.0, nthreads=None) -> dict:
    """Router part for the given tokens (default all): logits, probs, sel,
    weights and kept flags, with routing replay (``replay`` (n,K), optional
    ``replay_mask`` (n) bool) and the dynamic threshold.  See oracle_route in
    moe_oracle.c for the passages each option follows."""
    lib = _load()
    x2 = np.ascontiguousarray(x).reshape(-1, np.shape(x)[-1])
    T, D = x2.shape
    router = np.ascontiguousarray(router)
    E = router.shape[0]
    dt = _dtype_code(x2)
    if _dtype_code(router) != dt or router.shape != (E, D):
        raise ValueError("router must be (E,D) in the dtype of x")
    rb = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tokens.shape[0]
    else:
        n = T
    if replay is not None:
        replay = np.ascontiguousarray(replay, dtype=np.int64).reshape(n, top_k)
    if replay_mask is not None:
        replay_mask = np.ascontiguousarray(replay_mask, dtype=np.uint8).reshape(n)
    sel = np.empty((n, top_k), np.int64)
    w = np.empty((n, top_k), np.float64)
    logits = np.empty((n, E), np.float64)
    probs = np.empty((n, E), np.float64)
    kept = np.empty((n, top_k), np.uint8)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = lib.oracle_route(T, D, E, top_k, int(bool(norm)), dt, _ptr(x2), _ptr(router), _ptr(rb), _ptr(tokens), n,
                          _ptr(replay), _ptr(replay_mask), float(threshold), _ptr(sel), _ptr(w), _ptr(logits),
                          _ptr(probs), _ptr(kept), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_route failed with code %d" % rc)
    return dict(sel=sel, weights=w, logits=logits, probs=probs, kept=kept.astype(bool))


def capacity_slots(seq_len, top_k, num_experts, capacity_factor) -> int:
    """Slots per expert per sequence for a capacity factor (oracle_capacity_slots)."""
    return int(_load().oracle_capacity_slots(int(seq_len), int(top_k), int(num_experts), float(capacity_factor)))


def capacity(sel, kept, *, num_experts, seq_len, slots) -> np.ndarray:
    """Capacity drops over whole sequences; returns the updated kept flags (T,K)."""
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    T, K = sel.shape
    k8 = np.ascontiguousarray(kept, dtype=np.uint8).copy()
    rc = _load().oracle_capacity(T, K, int(num_experts), int(seq_len), int(slots), _ptr(sel), _ptr(k8))
    if rc != 0:
        raise ValueError("oracle_capacity failed with code %d" % rc)
    return k8.astype(bool)


def experts(x, gate_up, down, sel, weights, kept=None, *, act="swiglu", up_bias=None, down_bias=None, tokens=None,
            nthreads=None) -> np.ndarray:
    """Expert part for the given tokens with given sel/weights/kept (rows per evaluated token)."""
    lib = _load()
    x2 = np.ascontiguousarray(x).reshape(-1, np.shape(x)[-1])
    T, D = x2.shape
    gate_up, down = np.ascontiguousarray(gate_up), np.ascontiguousarray(down)
    E, _, F = down.shape
    dt = _dtype_code(x2)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    n, K = sel.shape
    weights = np.ascontiguousarray(weights, dtype=np.float64)
    k8 = None if kept is None else np.ascontiguousarray(kept, dtype=np.uint8)
    ub, db = (None if b is None else np.ascontiguousarray(b, dtype=np.float32) for b in (up_bias, down_bias))
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        if tokens.shape[0] != n:
            raise ValueError("one sel row per evaluated token")
    elif n > T:
        raise ValueError("more rows than tokens")
    out = np.empty((n, D), np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = lib.oracle_experts(T, D, F, E, K, SWIGLU if act == "swiglu" else RELU, dt, _ptr(x2), _ptr(gate_up),
                            _ptr(down), _ptr(ub), _ptr(db), _ptr(tokens), n, _ptr(sel), _ptr(weights), _ptr(k8),
                            _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_experts failed with code %d" % rc)
    return out


def balance_stats(probs, sel, weights) -> dict:
    """Router statistics and the four balancing objectives of the ES-MoE "API"
    page, section "Balancing objectives", over the T tokens of one call.

    probs (T,E) is the full softmax; the gate (T,E) holds each token's routing
    weights at its selected experts (the top-k selection renormalised) and 0
    elsewhere.  The usage u is the per-expert mean, normalised to sum to one:
      switch       = E * sum_i mean(probs)_i * mean(gate > 0)_i
      gshard       = E * sum_i u_i^2                   (u from the gate)
      master       = (1/E) * sum_i (u_i - 1/E)^2        (u from the gate)
      gshard_probs = E * sum_i u_i^2                   (u from probs)
    All in float64.
    """
    probs = np.asarray(probs, dtype=np.float64)
    sel = np.asarray(sel, dtype=np.int64)
    weights = np.asarray(weights, dtype=np.float64)
    T, E = probs.shape
    gate = np.zeros((T, E), np.float64)
    for k in range(sel.shape[1]):
        np.add.at(gate, (np.arange(T), sel[:, k]), weights[:, k])
    mean_probs = probs.mean(axis=0)
    mean_gate = gate.mean(axis=0)
    frac_routed = (gate > 0).mean(axis=0)
    u_gate = mean_gate / mean_gate.sum()
    u_probs = mean_probs / mean_probs.sum()
    return dict(mean_probs=mean_probs, mean_gate=mean_gate, frac_routed=frac_routed,
                switch=float(E * np.sum(mean_probs * frac_routed)),
                gshard=float(E * np.sum(u_gate ** 2)),
                master=float(np.sum((u_gate - 1.0 / E) ** 2) / E),
                gshard_probs=float(E * np.sum(u_probs ** 2)))


def forward_routed(inp: dict, *, tokens=None, replay=None, replay_mask=None, threshold=0.0, capacity_factor=None,
                   seq_len=None, nthreads=None) -> dict:
    """The layer with routing options on a ``workloads.generate`` dict.

    Routing (replay, dynamic threshold) and capacity drops are decided over
    all T tokens; the experts are evaluated for ``tokens`` (default all).
    Returns out (n,D) for the evaluated tokens; sel, weights, kept, logits,
    probs for all T tokens; the capacity slot count (or None); stats.
    """
    c = inp["cfg"]
    r = route(inp["x"], inp["router"], top_k=c["K"], norm=c["norm"], router_bias=inp.get("router_bias"),
              replay=replay, replay_mask=replay_mask, threshold=threshold, nthreads=nthreads)
    T = r["sel"].shape[0]
    slots = None
    if capacity_factor is not None:
        L = T if seq_len is None else int(seq_len)
        slots = capacity_slots(L, c["K"], c["E"], capacity_factor)
        r["kept"] = capacity(r["sel"], r["kept"], num_experts=c["E"], seq_len=L, slots=slots)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = experts(inp["x"], inp["gate_up"], inp["down"], r["sel"][tok], r["weights"][tok], r["kept"][tok],
                  act=c["act"], up_bias=inp.get("up_bias"), down_bias=inp.get("down_bias"), tokens=tok,
                  nthreads=nthreads)
    r.update(out=out, slots=slots, stats=balance_stats(r["probs"], r["sel"], r["weights"]))
    return r
