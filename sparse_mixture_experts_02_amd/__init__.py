"""MI355X-native forward pass of a token-choice top-k mixture-of-experts
feed-forward layer.

The layer runs in ``libmoe.so`` (hand-written HIP kernels for gfx950, C ABI in
``include/moe.h``).  This module is a thin ctypes binding: the functions named
like the C entry points (``moe_forward``, ``moe_dispatch``,
``moe_workspace_bytes``, ``moe_status_string``, ``moe_abi_version``) marshal
arguments and nothing else; ``forward`` additionally allocates the outputs and
the workspace with PyTorch, on the device of ``x``, and returns them.  PyTorch
provides device memory and the current stream; every step of the layer runs in
the library's kernels.  There is no fallback: without the built library on a
ROCm device every call raises.

Semantics follow the mojolearn ``MoEBlock`` page (Hugging Face weight layouts
router (E,D), gate_up_proj (E,2F,D), down_proj (E,D,F); output with the shape
of x; selected experts int64 in descending probability; ValueError for a bad
top_k or mismatched shapes, NotImplementedError for another activation,
TypeError for float64) and the ReLU-expert exercise of the crackedaicode
"Mixture-of-Experts FFN" page (biases, 1e-9-guarded renormalisation).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_ETYPE, MOE_EWORKSPACE, MOE_EDEVICE = range(6)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_RELU = 0, 1
MOE_MAX_EXPERTS = 256

_ACTS = {"silu": MOE_ACT_SWIGLU, "swiglu": MOE_ACT_SWIGLU, "relu": MOE_ACT_RELU}


class MoeDesc(ctypes.Structure):
    """Mirror of ``moe_desc`` in include/moe.h."""
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int64), ("F", ctypes.c_int64),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("deterministic", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    """Mirror of ``moe_routing`` in include/moe.h."""
    _fields_ = [("replay_experts", ctypes.c_void_p), ("replay_mask", ctypes.c_void_p),
                ("dynamic_threshold", ctypes.c_float), ("capacity_factor", ctypes.c_double),
                ("seq_len", ctypes.c_int64), ("kept", ctypes.c_void_p), ("stats", ctypes.c_void_p)]


def stats_len(E: int) -> int:
    """Length of the statistics vector (MOE_STATS_LEN)."""
    return 3 * int(E) + 4


class MoEError(RuntimeError):
    """A HIP launch or runtime failure reported by the library."""


_lib = None


def load_library():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built: run `python -m sparse_mixture_experts_02_amd.build` "
                               "(the layer has no non-HIP fallback)")
        # Load torch's HIP runtime first so the library binds to that same
        # runtime instance (one set of streams and allocations per process).
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover
            pass
        lib = ctypes.CDLL(LIB_PATH)
        P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        D = ctypes.POINTER(MoeDesc)
        lib.moe_workspace_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_workspace_bytes.restype = ctypes.c_int
        lib.moe_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.moe_forward.restype = ctypes.c_int
        lib.moe_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.moe_forward_noalloc.restype = ctypes.c_int
        lib.moe_forward_timed.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P, P, I32]
        lib.moe_forward_timed.restype = ctypes.c_int
        lib.moe_dispatch.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.moe_dispatch.restype = ctypes.c_int
        R = ctypes.POINTER(MoeRouting)
        lib.moe_forward_routed.argtypes = [D, R, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.moe_forward_routed.restype = ctypes.c_int
        lib.moe_dispatch_routed.argtypes = [D, R, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.moe_dispatch_routed.restype = ctypes.c_int
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_abi_version.argtypes = []
        lib.moe_abi_version.restype = I32
        lib.moe_probe_mfma.argtypes = [I32, I32, P, P]
        lib.moe_probe_mfma.restype = ctypes.c_int
        lib.moe_probe_mfma_flops.argtypes = [I32, I32]
        lib.moe_probe_mfma_flops.restype = ctypes.c_int64
        lib.moe_probe_read.argtypes = [P, ctypes.c_int64, I32, P, P]
        lib.moe_probe_read.restype = ctypes.c_int
        lib.moe_gemm_plan.argtypes = [D, P]
        lib.moe_gemm_plan.restype = ctypes.c_int
        _lib = lib
    return _lib


# ------------------------------------------------ entry points (C names)
def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(int(status)).decode()


def moe_abi_version() -> int:
    return int(load_library().moe_abi_version())


def moe_probe_mfma(blocks, iters, out, stream) -> int:
    """Raw call of the matrix-core rate probe; returns the status code."""
    return load_library().moe_probe_mfma(int(blocks), int(iters), out, stream)


def moe_probe_mfma_flops(blocks, iters) -> int:
    return int(load_library().moe_probe_mfma_flops(int(blocks), int(iters)))


def moe_probe_read(buf, nbytes, blocks, out, stream) -> int:
    """Raw call of the HBM read-rate probe; returns the status code."""
    return load_library().moe_probe_read(buf, int(nbytes), int(blocks), out, stream)


GEMM_VARIANTS = {0: "generic_m128", 1: "direct_m256_tail", 3: "direct_m32", 4: "generic_m64",
                 5: "stream_m32", 6: "stream_m32_narrow", 7: "stream_m64_narrow"}


def moe_gemm_plan(desc: MoeDesc) -> dict:
    """The two grouped GEMMs a call with `desc` runs (host only, no device
    call): per GEMM the kernel variant, rows and columns per tile, column
    tiles, whether its last round may be split along K, and the work-list
    capacity."""
    buf = (ctypes.c_int32 * 12)()
    _check(load_library().moe_gemm_plan(ctypes.byref(desc), buf))
    out = {}
    for i, name in enumerate(("gate_up", "down")):
        v = list(buf[6 * i:6 * i + 6])
        out[name] = dict(variant=GEMM_VARIANTS.get(v[0], str(v[0])), rows=v[1], cols=v[2], col_tiles=v[3],
                         k_split=bool(v[4]), max_items=v[5])
    return out


def moe_workspace_bytes(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def moe_forward(desc, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                stream) -> int:
    """Raw call: pointers are integers (or None); returns the status code."""
    return load_library().moe_forward(ctypes.byref(desc), x, router, gate_up_proj, down_proj, router_bias, up_bias,
                                      down_bias, out, selected_experts, routing_weights, router_logits,
                                      expert_counts, workspace, workspace_bytes, stream)


MOE_NOALLOC_MAX_BYTES = 128 << 20


def moe_forward_noalloc(desc, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                        selected_experts, routing_weights, router_logits, expert_counts, stream) -> int:
    """Raw call of moe_forward_noalloc (no workspace argument); returns the status code."""
    return load_library().moe_forward_noalloc(ctypes.byref(desc), x, router, gate_up_proj, down_proj, router_bias,
                                              up_bias, down_bias, out, selected_experts, routing_weights,
                                              router_logits, expert_counts, stream)


def moe_forward_timed(desc, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                      selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                      stream, events, n_events) -> int:
    """Raw call of moe_forward_timed; ``events`` is a ctypes array of hipEvent_t handles (or None)."""
    return load_library().moe_forward_timed(ctypes.byref(desc), x, router, gate_up_proj, down_proj, router_bias,
                                            up_bias, down_bias, out, selected_experts, routing_weights,
                                            router_logits, expert_counts, workspace, workspace_bytes, stream,
                                            events, n_events)


def moe_dispatch(desc, x, router, router_bias, selected_experts, routing_weights, router_logits, expert_counts,
                 expert_offsets, sorted_token, sorted_slot, workspace, workspace_bytes, stream) -> int:
    """Raw call: pointers are integers (or None); returns the status code."""
    return load_library().moe_dispatch(ctypes.byref(desc), x, router, router_bias, selected_experts,
                                       routing_weights, router_logits, expert_counts, expert_offsets, sorted_token,
                                       sorted_slot, workspace, workspace_bytes, stream)


def moe_forward_routed(desc, routing, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                       selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                       stream) -> int:
    """Raw call; ``routing`` is a MoeRouting or None."""
    r = ctypes.byref(routing) if routing is not None else None
    return load_library().moe_forward_routed(ctypes.byref(desc), r, x, router, gate_up_proj, down_proj, router_bias,
                                             up_bias, down_bias, out, selected_experts, routing_weights,
                                             router_logits, expert_counts, workspace, workspace_bytes, stream)


def moe_dispatch_routed(desc, routing, x, router, router_bias, selected_experts, routing_weights, router_logits,
                        expert_counts, expert_offsets, sorted_token, sorted_slot, workspace, workspace_bytes,
                        stream) -> int:
    """Raw call; ``routing`` is a MoeRouting or None."""
    r = ctypes.byref(routing) if routing is not None else None
    return load_library().moe_dispatch_routed(ctypes.byref(desc), r, x, router, router_bias, selected_experts,
                                              routing_weights, router_logits, expert_counts, expert_offsets,
                                              sorted_token, sorted_slot, workspace, workspace_bytes, stream)


def _check(status: int) -> None:
    if status == MOE_OK:
        return
    msg = moe_status_string(status)
    if status in (MOE_EINVAL, MOE_EWORKSPACE):
        raise ValueError(msg)
    if status == MOE_ENOTSUP:
        raise NotImplementedError(msg)
    if status == MOE_ETYPE:
        raise TypeError(msg)
    raise MoEError(msg)


# ------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}.get(t, -1)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _aligned16(t):
    """t as a contiguous tensor whose data starts on a 16-byte boundary (a copy
    only when a view starts elsewhere)."""
    t = t.contiguous()
    return t if t.data_ptr() % 16 == 0 else t.clone()


def make_desc(T, D, F, E, K, *, norm_topk_prob=True, act="silu", dtype=None, out_dtype=None,
              deterministic=False) -> MoeDesc:
    return MoeDesc(T=int(T), D=int(D), F=int(F), E=int(E), K=int(K), norm_topk=int(bool(norm_topk_prob)),
                   act=_ACTS.get(act, -1) if isinstance(act, str) else int(act),
                   dtype=_dtype_code(dtype) if dtype is not None else MOE_F32,
                   out_dtype=_dtype_code(out_dtype) if out_dtype is not None else MOE_F32,
                   deterministic=int(bool(deterministic)))


def _prepare(x, router, gate_up_proj, down_proj, top_k, act, biases=(None, None, None)):
    torch = _torch()
    if x.dtype == torch.float64:
        raise TypeError("float64 input is not supported")
    D = x.shape[-1]
    E = router.shape[0]
    if router.dim() != 2 or router.shape[1] != D:
        raise ValueError("router must be (E, D) = (%d, %d), got %s" % (E, D, tuple(router.shape)))
    if down_proj.dim() != 3 or down_proj.shape[0] != E or down_proj.shape[1] != D:
        raise ValueError("down_proj must be (E, D, F), got %s" % (tuple(down_proj.shape),))
    F = down_proj.shape[2]
    G = 1 if act == "relu" else 2
    if gate_up_proj.shape != (E, G * F, D):
        raise ValueError("gate_up_proj must be %s, got %s" % ((E, G * F, D), tuple(gate_up_proj.shape)))
    _check_biases(*biases, D, F, E, act)
    for t in (router, gate_up_proj, down_proj):
        if t.dtype != x.dtype:
            raise TypeError("x and the weights must share one dtype")
        if t.device != x.device:
            raise ValueError("all tensors must be on one device")
    if x.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    return D, F, E


def _check_biases(router_bias, up_bias, down_bias, D, F, E, act):
    """The kernels read router_bias as (E), up_bias as (E, G*F) (the up half
    at +F for SwiGLU) and down_bias as (E, D): any other shape is refused
    before a pointer reaches them."""
    G = 1 if act == "relu" else 2
    for name, b, shape in (("router_bias", router_bias, (E,)), ("up_bias", up_bias, (E, G * F)),
                           ("down_bias", down_bias, (E, D))):
        if b is not None and tuple(b.shape) != shape:
            raise ValueError("%s must be %s, got %s" % (name, shape, tuple(b.shape)))


def _routing(T, top_k, dev, replay, replay_mask, dynamic_threshold, capacity_factor, seq_len, kept, stats):
    """A MoeRouting for the options (None when every option is off), plus the
    device tensors it points to (kept alive by the caller)."""
    torch = _torch()
    if replay is None and not dynamic_threshold and capacity_factor is None and kept is None and stats is None:
        return None, []
    keep = []
    rep = msk = None
    if replay is not None:
        rep = replay.to(device=dev, dtype=torch.int64).reshape(T, top_k).contiguous()
        keep.append(rep)
        if replay_mask is not None:
            msk = replay_mask.to(device=dev).reshape(T).ne(0).to(torch.uint8).contiguous()
            keep.append(msk)
    r = MoeRouting(replay_experts=_ptr(rep), replay_mask=_ptr(msk), dynamic_threshold=float(dynamic_threshold or 0.0),
                   capacity_factor=float(capacity_factor or 0.0), seq_len=int(seq_len or 0), kept=_ptr(kept),
                   stats=_ptr(stats))
    return r, keep


def forward(x, router, gate_up_proj, down_proj, *, top_k, norm_topk_prob=True, act="silu", router_bias=None,
            up_bias=None, down_bias=None, out_dtype=None, deterministic=True, return_logits=False,
            return_counts=False, workspace=None, replay=None, replay_mask=None, dynamic_threshold=0.0,
            capacity_factor=None, seq_len=None, return_kept=False, return_stats=False):
    """Layer forward on the device of x.

    Returns (out with the shape of x, selected_experts int64 (T,K),
    routing_weights fp32 (T,K)) plus, in this order and when requested,
    router_logits (T,E), expert_counts (E), kept (T,K) bool and the
    statistics vector (3E+4) fp32.  ``out_dtype`` defaults to float32.
    ``deterministic`` (default) sums each token's K expert rows in k order;
    False adds them with fp32 atomics instead.  Routing options (see
    ``moe_routing`` in include/moe.h): ``replay`` (T,K) recorded experts with
    an optional ``replay_mask`` (T); ``dynamic_threshold``; ``capacity_factor``
    over sequences of ``seq_len`` tokens (default: all T).
    """
    torch = _torch()
    D, F, E = _prepare(x, router, gate_up_proj, down_proj, top_k, act, (router_bias, up_bias, down_bias))
    lead = x.shape[:-1]
    x2 = x.reshape(-1, D).contiguous()
    T = x2.shape[0]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    desc = make_desc(T, D, F, E, top_k, norm_topk_prob=norm_topk_prob, act=act, dtype=x.dtype,
                     out_dtype=out_dtype, deterministic=deterministic)
    nbytes = moe_workspace_bytes(desc)
    dev = x.device
    out = torch.empty((T, D), dtype=out_dtype, device=dev)
    sel = torch.empty((T, top_k), dtype=torch.int64, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if return_logits else None
    counts = torch.empty((E,), dtype=torch.int32, device=dev) if return_counts else None
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of x (%s), got %s" % (dev, workspace.device))
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    biases = [None if b is None else b.to(device=dev, dtype=torch.float32).contiguous()
              for b in (router_bias, up_bias, down_bias)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    kept = torch.empty((T, top_k), dtype=torch.uint8, device=dev) if return_kept else None
    stats = torch.empty((stats_len(E),), dtype=torch.float32, device=dev) if return_stats else None
    rt, _alive = _routing(T, top_k, dev, replay, replay_mask, dynamic_threshold, capacity_factor, seq_len, kept, stats)
    # contiguous, 16-byte aligned operands, held until the call has been enqueued
    x2, rt_w, gu, dn = (_aligned16(t) for t in (x2, router, gate_up_proj, down_proj))
    if workspace.data_ptr() % 16:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    args = (_ptr(x2), _ptr(rt_w), _ptr(gu), _ptr(dn),
            *(_ptr(b) for b in biases), _ptr(out), _ptr(sel), _ptr(w), _ptr(logits), _ptr(counts), _ptr(workspace),
            nbytes, stream)
    if rt is None:
        _check(moe_forward(desc, *args))
    else:
        _check(moe_forward_routed(desc, rt, *args))
    res = [out.reshape(*lead, D), sel, w]
    if return_logits:
        res.append(logits)
    if return_counts:
        res.append(counts)
    if return_kept:
        res.append(kept.bool())
    if return_stats:
        res.append(stats)
    return tuple(res)


def dispatch(x, router, *, top_k, norm_topk_prob=True, router_bias=None, num_experts=None, F=1, replay=None,
             replay_mask=None, dynamic_threshold=0.0, capacity_factor=None, seq_len=None):
    """Router plus the stable sort into expert order (of the kept slots when
    a routing option drops some).

    Returns dict(selected_experts, routing_weights, router_logits,
    expert_counts, expert_offsets, sorted_token, sorted_slot, kept).
    """
    torch = _torch()
    D = x.shape[-1]
    E = router.shape[0] if num_experts is None else num_experts
    x2 = x.reshape(-1, D).contiguous()
    T = x2.shape[0]
    desc = make_desc(T, D, F, E, top_k, norm_topk_prob=norm_topk_prob, dtype=x.dtype)
    nbytes = moe_workspace_bytes(desc)
    dev = x.device
    M = T * top_k
    r = dict(selected_experts=torch.empty((T, top_k), dtype=torch.int64, device=dev),
             routing_weights=torch.empty((T, top_k), dtype=torch.float32, device=dev),
             router_logits=torch.empty((T, E), dtype=torch.float32, device=dev),
             expert_counts=torch.empty((E,), dtype=torch.int32, device=dev),
             expert_offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
             sorted_token=torch.empty((M,), dtype=torch.int32, device=dev),
             sorted_slot=torch.empty((M,), dtype=torch.int32, device=dev))
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    if router.dim() != 2 or router.shape[1] != D or router.shape[0] != E:
        raise ValueError("router must be (E, D) = (%d, %d), got %s" % (E, D, tuple(router.shape)))
    _check_biases(router_bias, None, None, D, F, E, "silu")
    if router.dtype != x.dtype:
        raise TypeError("x and the router must share one dtype")
    rb = None if router_bias is None else router_bias.to(device=dev, dtype=torch.float32).contiguous()
    stream = torch.cuda.current_stream(dev).cuda_stream
    kept = torch.empty((T, top_k), dtype=torch.uint8, device=dev)
    rt, _alive = _routing(T, top_k, dev, replay, replay_mask, dynamic_threshold, capacity_factor, seq_len, kept, None)
    router_c = router.contiguous()  # held until the call has been enqueued
    _check(moe_dispatch_routed(desc, rt, _ptr(x2), _ptr(router_c), _ptr(rb), _ptr(r["selected_experts"]),
                               _ptr(r["routing_weights"]), _ptr(r["router_logits"]), _ptr(r["expert_counts"]),
                               _ptr(r["expert_offsets"]), _ptr(r["sorted_token"]), _ptr(r["sorted_slot"]),
                               _ptr(ws), nbytes, stream))
    r["kept"] = kept.bool()
    return r


MOE_STAGE_EVENTS = 6

__all__ = ["MoeDesc", "MoeRouting", "MoEError", "load_library", "moe_forward", "moe_forward_noalloc",
           "moe_forward_timed",
           "moe_forward_routed", "moe_dispatch", "moe_dispatch_routed", "moe_workspace_bytes", "moe_status_string",
           "moe_abi_version", "moe_gemm_plan", "GEMM_VARIANTS", "make_desc", "stats_len", "forward", "dispatch",
           "LIB_PATH"]
