"""Seeded synthetic inputs for the token-choice top-k MoE feed-forward layer.

This module only draws numbers: it holds none of the layer's arithmetic
(no router, no softmax, no expert math).  Both the HIP path's tests and
benchmark and the CPU oracle's tests take their inputs from here, and nowhere
else do the two sides share code.

Recipe (every tensor)
---------------------
* Each tensor has its own integer seed ``1000 * cfg_id + tensor_id`` with
  tensor ids x=0, router=1, router_bias=2, gate_up (or W1)=3, up bias (b1)=4,
  down (or W2)=5, down bias (b2)=6.
* A normal tensor is flattened and cut into chunks of ``CHUNK`` elements;
  chunk ``i`` is ``numpy.random.default_rng([seed, i]).standard_normal(n,
  float32)``, multiplied in float32 by its standard deviation.  Chunks are
  independent streams, so they are drawn on several threads and any prefix
  of a tensor can be drawn alone.
* bf16 tensors are the round-to-nearest-even bf16 of those float32 draws and
  are held as ``uint16`` bit patterns.
* Biases and the router bias are always float32.

The five workloads follow the block described on the mojolearn ``MoEBlock``
page (Hugging Face layouts router (E,D), gate_up_proj (E,2F,D), down_proj
(E,D,F)) and the ReLU-expert exercise of the crackedaicode "Mixture-of-Experts
FFN" page (each expert Dense(F)->ReLU->Dense(D) with biases, router Dense(E)
with bias).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

TID_X, TID_ROUTER, TID_RB, TID_W1, TID_B1, TID_W2, TID_B2 = range(7)

# name -> description.  act "swiglu": gate_up_proj is (E, 2F, D) (gate rows
# [0,F), up rows [F,2F)); act "relu": it is W1 (E, F, D) and biases exist.
CONFIGS = {
    "tiny": dict(cfg_id=1, T=64, x_shape=(4, 16, 64), D=64, F=128, E=8, K=2,
                 norm=True, act="swiglu", dtype="f32", biases=False,
                 x_dist="uniform", desc="Mixtral-style SwiGLU block, fp32, "
                 "x (4,16,64) uniform[0,1) as in the MoEBlock page example"),
    "relu": dict(cfg_id=2, T=4096, D=512, F=2048, E=8, K=2, norm=True,
                 act="relu", dtype="f32", biases=True, x_dist="normal",
                 desc="ReLU experts with biases, fp32, T=4096 D=512 F=2048 E=8 K=2"),
    "prefill": dict(cfg_id=3, T=8192, D=4096, F=14336, E=8, K=2, norm=True,
                    act="swiglu", dtype="bf16", biases=False, x_dist="normal",
                    desc="Mixtral-8x7B-shaped prefill, bf16, T=8192 D=4096 F=14336 E=8 K=2"),
    "decode": dict(cfg_id=3, T=64, D=4096, F=14336, E=8, K=2, norm=True,
                   act="swiglu", dtype="bf16", biases=False, x_dist="normal",
                   desc="Mixtral-8x7B-shaped decode batch, bf16, T=64 (first 64 "
                   "tokens of the prefill workload, same weights)"),
    "fine": dict(cfg_id=5, T=16384, D=2048, F=768, E=128, K=8, norm=True,
                 act="swiglu", dtype="bf16", biases=False, x_dist="normal",
                 router_bias="zipf", desc="fine-grained 128-expert layer, bf16, "
                 "T=16384 D=2048 F=768 E=128 K=8, Zipf-skewed router bias"),
    "fine_zero": dict(cfg_id=5, T=16384, D=2048, F=768, E=128, K=8, norm=True,
                      act="swiglu", dtype="bf16", biases=False, x_dist="normal",
                      router_bias="zipf_zero", desc="as 'fine' with 8 experts "
                      "pushed to zero load (router bias -30)"),
}

W_STD = 0.02   # expert and router weights
B_STD = 0.01   # biases of the ReLU experts and the router


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, n: int, std: float = 1.0) -> np.ndarray:
    """First ``n`` values of the chunked N(0, std^2) stream of ``seed``."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        np.random.default_rng([seed, i]).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        fill(0) if n else None
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    n = u.size
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24

    def conv(i: int) -> None:
        s = flat_u[i:i + step]
        flat_o[i:i + step] = ((s + np.uint32(0x7FFF) + ((s >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(conv, range(0, n, step)))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_rank_bias(E: int, s: float = 1.1) -> np.ndarray:
    """0.5 * ln(P(rank e+1)) under Zipf(s) over ranks 1..E, float32."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return (0.5 * np.log(p)).astype(np.float32)


def zero_load_experts(E: int, n: int = 8, seed: int = 5007) -> np.ndarray:
    return np.sort(np.random.default_rng(seed).choice(E, size=n, replace=False))


def _weight(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    a = normal_f32(seed, int(np.prod(shape)), std).reshape(shape)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def generate(name_or_cfg, *, T: int | None = None, with_weights: bool = True) -> dict:
    """Inputs of a named workload (or of an explicit config dict).

    Returns a dict with x (T,D), router (E,D), gate_up (E,G*F,D), down (E,D,F)
    as float32 (dtype f32) or uint16 bf16 bits (dtype bf16), router_bias (E),
    up_bias (E,G*F), down_bias (E,D) as float32 or None, and the config.
    ``T`` draws only the first T tokens of x.
    """
    cfg = dict(CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cid = cfg["cfg_id"]
    D, F, E = cfg["D"], cfg["F"], cfg["E"]
    G = 2 if cfg["act"] == "swiglu" else 1
    T = cfg["T"] if T is None else T
    cfg["T"] = T
    dt = cfg["dtype"]
    seed = lambda tid: 1000 * cid + tid  # noqa: E731

    if cfg.get("x_dist") == "uniform":
        # The MoEBlock page's example input: default_rng(0).random(shape, float32).
        shape = cfg.get("x_shape", (T, D))
        xf = np.random.default_rng(0).random(shape, dtype=np.float32).reshape(-1, D)[:T]
    else:
        xf = normal_f32(seed(TID_X), T * D).reshape(T, D)
    out = dict(cfg=cfg, x=f32_to_bf16_bits(xf) if dt == "bf16" else xf)
    if not with_weights:
        return out
    out["router"] = _weight(seed(TID_ROUTER), (E, D), W_STD, dt)
    out["gate_up"] = _weight(seed(TID_W1), (E, G * F, D), W_STD, dt)
    out["down"] = _weight(seed(TID_W2), (E, D, F), W_STD, dt)
    rb = None
    if cfg.get("biases"):
        rb = normal_f32(seed(TID_RB), E, B_STD)
        out["up_bias"] = normal_f32(seed(TID_B1), E * G * F, B_STD).reshape(E, G * F)
        out["down_bias"] = normal_f32(seed(TID_B2), E * D, B_STD).reshape(E, D)
    else:
        out["up_bias"] = out["down_bias"] = None
    if cfg.get("router_bias") in ("zipf", "zipf_zero"):
        rb = zipf_rank_bias(E)
        if cfg["router_bias"] == "zipf_zero":
            rb[zero_load_experts(E)] -= np.float32(30.0)
    elif cfg.get("router_bias") == "last_heavy":
        # the highest-index expert is favoured: it takes most of the rows,
        # the other experts share the rest
        rb = np.zeros(E, dtype=np.float32)
        rb[E - 1] = np.float32(2.0)
    out["router_bias"] = rb
    return out


def small_config(T, D, F, E, K, *, act="swiglu", dtype="f32", norm=True, biases=False,
                 cfg_id=100, router_bias=None, x_dist="normal") -> dict:
    """An ad-hoc config (tests: edge cases, ragged tails)."""
    return dict(cfg_id=cfg_id, T=T, D=D, F=F, E=E, K=K, norm=norm, act=act, dtype=dtype,
                biases=biases, router_bias=router_bias, x_dist=x_dist)


def input_sha256(inputs: dict) -> str:
    import hashlib
    h = hashlib.sha256()
    for k in ("x", "router", "gate_up", "down", "router_bias", "up_bias", "down_bias"):
        v = inputs.get(k)
        if v is not None:
            h.update(k.encode())
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["CONFIGS", "generate", "small_config", "normal_f32", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "zipf_rank_bias", "zero_load_experts", "input_sha256",
           "ceil_div"]
