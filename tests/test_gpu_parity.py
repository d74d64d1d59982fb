"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (ctypes binding over libmoe.so).  Sizes:
the small workloads are compared token by token in full; the full-size
workloads (the Mixtral-shaped prefill and decode, the 128-expert layer) run
at their real shape in the configuration the benchmark times and are compared
on the tokens of the first and last row of every 64-row strip of every expert
segment (every row tile, tail tile and K-split tile of both GEMMs), plus
properties that hold for every token.
"""
import os

import numpy as np
import pytest

import workloads
from parity import (assert_strata_covered, check, check_full_properties, device_inputs, gpu_forward,
                    stratified_tokens, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no ROCm device", allow_module_level=True)

import sparse_mixture_experts_02_amd as moe  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print("[gpu-parity] " + msg, flush=True)


STRIP = 64  # every row tile of the 256- and 128-row GEMM tiles starts at a multiple of 64 in its segment


def _strata(inp, g, d=None):
    """Compared tokens: the first and last row of every 64-row strip of every
    expert segment of the sorted order (so every row tile of both GEMMs, each
    tail tile and each K-split tile has compared rows), plus tokens 0 and T-1.
    With the device inputs at hand the order is taken from moe.dispatch and
    checked bit-exact against a stable argsort of the layer's selection."""
    c = inp["cfg"]
    T, E, K = c["T"], c["E"], c["K"]
    tok, rows, offs, order = stratified_tokens(g["sel"], E, STRIP)
    if d is not None:
        r = moe.dispatch(d["x"], d["router"], top_k=K, norm_topk_prob=c["norm"], router_bias=d["router_bias"])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r["selected_experts"].cpu().numpy(), g["sel"])
        np.testing.assert_array_equal(r["expert_offsets"].cpu().numpy(), offs)
        np.testing.assert_array_equal(r["sorted_slot"].cpu().numpy(), order)
        np.testing.assert_array_equal(r["sorted_token"].cpu().numpy(), order // K)
    tok = np.unique(np.concatenate([tok, [0, T - 1]]))
    assert_strata_covered(tok, g["sel"], E, STRIP)
    _say("compared tokens %d (rows %d of %d)" % (tok.size, rows.size, T * K))
    return tok


# ------------------------------------------------------------ small, full
@pytest.mark.parametrize("det", [False, True])
def test_tiny_block_fp32(det):
    inp = workloads.generate("tiny")
    _say("tiny det=%s" % det)
    g = gpu_forward(inp, deterministic=det)
    st = check(inp, g)
    check_full_properties(inp, g)
    _say(str(st))


def test_relu_experts_fp32_full():
    inp = workloads.generate("relu")
    _say("relu T=4096 D=512 F=2048")
    g = gpu_forward(inp)
    st = check(inp, g)
    check_full_properties(inp, g)
    _say(str(st))


def test_worked_example_on_gpu():
    """The exercise's two-token example through the whole GPU layer: a ReLU
    layer whose router rows hold ln p and whose experts reproduce the printed
    expert outputs (crackedaicode "Mixture-of-Experts FFN", "Work through two
    tokens")."""
    from test_oracle_pins import worked_example_layer
    lay, g = worked_example_layer()
    d = {k: to_device(v) for k, v in lay.items()}
    out, sel, w = moe.forward(d["x"], d["router"], d["gate_up"], d["down"], top_k=2, act="relu")
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), np.array(g["expected_indices"]))
    np.testing.assert_allclose(out.cpu().numpy(), np.array(g["expected_out"]), rtol=0, atol=g["atol"])


EDGE = [
    # (T, D, F, E, K, act, dtype, biases, norm)
    (1, 64, 128, 8, 2, "swiglu", "f32", False, True),
    (300, 72, 200, 6, 2, "swiglu", "f32", False, True),
    (300, 72, 200, 6, 2, "swiglu", "bf16", False, True),
    (257, 13, 9, 5, 3, "swiglu", "f32", True, True),
    (257, 13, 9, 5, 3, "relu", "bf16", True, False),
    (1000, 128, 256, 4, 2, "swiglu", "bf16", False, True),
    (513, 96, 160, 3, 3, "relu", "f32", True, True),
    (200, 64, 64, 1, 1, "swiglu", "bf16", False, True),
    (333, 40, 48, 7, 1, "swiglu", "f32", False, False),
    (129, 256, 96, 256, 4, "swiglu", "bf16", False, True),
    (2048, 256, 512, 16, 4, "relu", "bf16", True, True),
    (77, 8, 8, 37, 37, "swiglu", "f32", False, True),
    # bf16 shapes on the direct-to-LDS kernels (K a multiple of 64), with
    # ragged row tiles and column tails: 128-row, 256-row and 32-row tiles
    (1000, 128, 320, 4, 2, "swiglu", "bf16", False, True),
    (600, 192, 448, 3, 1, "relu", "bf16", True, True),
    # fp32 between 64 and 512 rows per expert (256-row tiles, mostly partial)
    (1000, 128, 320, 4, 2, "swiglu", "f32", False, True),
    (600, 192, 448, 3, 1, "relu", "f32", True, True),
    (4096, 128, 192, 4, 2, "swiglu", "bf16", False, True),
    # 256-row tiles whose columns all lie inside N, without biases: the
    # interior-tile epilogue of the ReLU and down tiles
    (4096, 128, 256, 4, 2, "relu", "bf16", False, True),
    (40, 256, 384, 8, 2, "swiglu", "bf16", False, True),
    (64, 4096, 1024, 8, 2, "swiglu", "bf16", False, True),
    (3000, 64, 128, 40, 6, "swiglu", "bf16", False, True),

    # bf16 routers over more than 64 experts with D a multiple of 256 take the
    # LDS-staged logits kernel (64 tokens per block): ragged token blocks,
    # expert counts off the 16-row MFMA tile, a router bias, 8 and 16 tiles
    (1000, 512, 128, 128, 8, "swiglu", "bf16", True, True),
    (70, 256, 64, 100, 6, "swiglu", "bf16", False, True),
    (300, 768, 64, 200, 4, "relu", "bf16", True, False),
    # fp32 and non-multiple-of-256 widths over more than 64 experts keep the
    # logits inside the 16-token router blocks
    (200, 96, 64, 80, 4, "swiglu", "f32", True, True),
    # more 1024-assignment chunks than the scan has lanes per expert (137 > 128)
    (70000, 64, 64, 8, 2, "swiglu", "f32", False, True),
    (150, 320, 64, 130, 3, "swiglu", "bf16", False, True),
]
# The highest-index expert carries most rows (its segment ends at offsets[E]),
# over 64 or more experts, on the one-block and the multi-block sort.
EDGE_LAST = [
    (100, 128, 192, 128, 8, "swiglu", "bf16", False, True),
    (3000, 128, 256, 128, 8, "swiglu", "bf16", False, True),
    (2500, 64, 96, 256, 4, "relu", "f32", True, True),
    (700, 256, 320, 65, 2, "swiglu", "bf16", False, True),
]


# Decode-sized bf16 segments with K a multiple of 512 take the weight-streaming
# kernel: 1 to 16 K chunks of 512 (odd and even counts, so both ways through
# its two-chunk loop), the narrow (128 weight rows) and wide (256, with its
# last round split along K: parts of one and two chunks) tiles, the ReLU and
# SwiGLU epilogues, a column tail off the tile width, experts with more than
# 32 rows, and the 64-row narrow tile (28 or more rows per expert on
# average: one or two 32-row halves, experts with more than 64 rows over
# several tiles under the Zipf bias), and both sides of the switch to the
# 256-row tile at 58 rows per expert on average (228 and 232 tokens).  The
# last field names the kernels the plan must pick (gate_up, down) in the
# atomic and in the deterministic mode.
S, SN, S64, M32, G64 = "stream_m32", "stream_m32_narrow", "stream_m64_narrow", "direct_m32", "generic_m64"
M256 = "direct_m256_tail"
STREAM = [
    (40, 1024, 1536, 8, 2, "swiglu", "bf16", False, True, {False: (SN, SN), True: (SN, SN)}),
    (24, 1536, 2048, 4, 2, "relu", "bf16", True, True, {False: (SN, SN), True: (SN, SN)}),
    (16, 8192, 512, 4, 2, "swiglu", "bf16", False, True, {False: (S, SN), True: (S, SN)}),
    (30, 512, 1056, 8, 2, "swiglu", "bf16", True, False, {False: (SN, G64), True: (SN, G64)}),
    (50, 2560, 512, 8, 3, "relu", "bf16", False, True, {False: (SN, SN), True: (SN, SN)}),
    (128, 1024, 1536, 8, 2, "swiglu", "bf16", False, True, {False: (S64, S64), True: (S64, S64)}),
    (200, 1024, 1536, 8, 2, "swiglu", "bf16", False, False, {False: (S64, S64), True: (S64, S64)}),
    (100, 1536, 2048, 4, 2, "relu", "bf16", True, True, {False: (S64, S64), True: (S64, S64)}),
    (120, 512, 1056, 8, 2, "swiglu", "bf16", True, True, {False: (S64, G64), True: (S64, G64)}),
    (228, 1024, 1536, 8, 2, "swiglu", "bf16", False, True, {False: (S64, S64), True: (S64, S64)}),
    (232, 1024, 1536, 8, 2, "swiglu", "bf16", True, True, {False: (M256, M256), True: (M256, M256)}),
    (3, 512, 4096, 4, 2, "relu", "bf16", True, True, {False: (SN, SN), True: (SN, S)}),
]


@pytest.mark.parametrize("case", STREAM, ids=lambda c: "T%d_D%d_F%d_E%d_K%d_%s_%s_b%d_n%d" % tuple(c[:9]))
@pytest.mark.parametrize("det", [False, True])
def test_weight_streaming_shapes(case, det):
    T, D, F, E, K, act, dt, biases, norm, kernels = case
    desc = moe.make_desc(T, D, F, E, K, norm_topk_prob=norm, act="silu" if act == "swiglu" else "relu",
                         dtype=torch.bfloat16, deterministic=det)
    plan = moe.moe_gemm_plan(desc)
    assert (plan["gate_up"]["variant"], plan["down"]["variant"]) == kernels[det], plan
    cfg = workloads.small_config(T, D, F, E, K, act=act, dtype=dt, norm=norm, biases=biases,
                                 router_bias="zipf" if E >= 8 else None, cfg_id=500 + E + K)
    inp = workloads.generate(cfg)
    _say("stream %s det=%s" % (case[:9], det))
    g = gpu_forward(inp, deterministic=det)
    check(inp, g)
    check_full_properties(inp, g)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "T%d_D%d_F%d_E%d_K%d_%s_%s_b%d_n%d" % tuple(c))
@pytest.mark.parametrize("det", [False, True])
def test_edge_shapes(case, det):
    T, D, F, E, K, act, dt, biases, norm = case
    cfg = workloads.small_config(T, D, F, E, K, act=act, dtype=dt, norm=norm, biases=biases,
                                 router_bias="zipf" if E >= 8 else None, cfg_id=200 + E + K)
    inp = workloads.generate(cfg)
    _say("edge %s det=%s" % (case, det))
    g = gpu_forward(inp, deterministic=det)
    check(inp, g)
    check_full_properties(inp, g)


@pytest.mark.parametrize("case", EDGE_LAST, ids=lambda c: "T%d_D%d_F%d_E%d_K%d_%s_%s_b%d_n%d" % tuple(c))
@pytest.mark.parametrize("det", [False, True])
def test_edge_last_expert_heavy(case, det):
    T, D, F, E, K, act, dt, biases, norm = case
    cfg = workloads.small_config(T, D, F, E, K, act=act, dtype=dt, norm=norm, biases=biases,
                                 router_bias="last_heavy", cfg_id=260 + E + K)
    inp = workloads.generate(cfg)
    _say("edge-last %s det=%s" % (case, det))
    g = gpu_forward(inp, deterministic=det)
    assert g["counts"][E - 1] > T // 2
    check(inp, g)
    check_full_properties(inp, g)


# 256-row tiles whose expert's last tile holds 1-64, 65-128, 129-192 and
# 193-255 rows (so one to four of the wave row strips have rows; the waves
# past the end skip their MFMAs): each case has last tiles in all four
# classes (checked below) and is compared in full, in both combine modes.
SHORT_TILES = [
    # (T, D, F, E, K, act, biases, router bias, cfg id)
    (4096, 128, 256, 8, 2, "swiglu", False, "zipf", 610),
    (5000, 128, 256, 8, 2, "relu", True, None, 612),
]


@pytest.mark.parametrize("case", SHORT_TILES, ids=lambda c: "T%d_%s_b%d" % (c[0], c[5], c[6]))
@pytest.mark.parametrize("det", [False, True])
def test_short_row_tiles(case, det):
    T, D, F, E, K, act, biases, rb, cid = case
    desc = moe.make_desc(T, D, F, E, K, act="silu" if act == "swiglu" else "relu", dtype=torch.bfloat16,
                         deterministic=det)
    plan = moe.moe_gemm_plan(desc)
    assert plan["gate_up"]["variant"] == plan["down"]["variant"] == "direct_m256_tail", plan
    cfg = workloads.small_config(T, D, F, E, K, act=act, dtype="bf16", biases=biases, router_bias=rb, cfg_id=cid)
    inp = workloads.generate(cfg)
    _say("short tiles %s det=%s" % (case, det))
    g = gpu_forward(inp, deterministic=det)
    # last-tile rows c mod 256 above the 32 tail rows a full tile may absorb
    classes = {(int(c) % 256 - 1) // 64 for c in g["counts"] if int(c) % 256 > 32}
    assert classes == {0, 1, 2, 3}, g["counts"]
    check(inp, g)
    check_full_properties(inp, g)


def test_caller_workspace():
    """A caller's workspace is used when it is large enough (any dtype: its
    size counts in bytes); one on another device is refused before a launch."""
    inp = workloads.generate(workloads.small_config(200, 64, 128, 8, 2, dtype="bf16", cfg_id=620))
    d = device_inputs(inp)
    c = inp["cfg"]
    kw = dict(top_k=c["K"], norm_topk_prob=c["norm"])
    ref = moe.forward(d["x"], d["router"], d["gate_up"], d["down"], **kw)
    desc = moe.make_desc(c["T"], c["D"], c["F"], c["E"], c["K"], dtype=torch.bfloat16, deterministic=True)
    n = moe.moe_workspace_bytes(desc)
    ws = torch.empty(((n + 3) // 4,), dtype=torch.float32, device="cuda")
    got = moe.forward(d["x"], d["router"], d["gate_up"], d["down"], workspace=ws, **kw)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    with pytest.raises(ValueError, match="workspace"):
        moe.forward(d["x"], d["router"], d["gate_up"], d["down"], workspace=torch.empty(n, dtype=torch.uint8), **kw)


@pytest.mark.parametrize("seed", range(12))
def test_random_small_sweep(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 12))
    K = int(rng.integers(1, E + 1))
    cfg = workloads.small_config(int(rng.integers(1, 200)), int(rng.integers(1, 80)), int(rng.integers(1, 80)),
                                 E, K, act=["swiglu", "relu"][seed % 2], dtype=["f32", "bf16"][(seed // 2) % 2],
                                 norm=bool(seed % 3), biases=bool(seed % 4 == 1), cfg_id=300 + seed)
    inp = workloads.generate(cfg)
    _say("sweep seed=%d cfg=%s" % (seed, {k: cfg[k] for k in ("T", "D", "F", "E", "K", "act", "dtype")}))
    g = gpu_forward(inp, deterministic=bool(seed % 2))
    check(inp, g)
    check_full_properties(inp, g)


@pytest.mark.parametrize("T,D,F,E", [(400, 128, 192, 8), (4000, 256, 512, 4)])
def test_bf16_output(T, D, F, E):
    # 128-row tiles; 256-row tiles with tail rows and K-split parts
    cfg = workloads.small_config(T, D, F, E, 2, dtype="bf16", cfg_id=400 + E)
    inp = workloads.generate(cfg)
    for det in (False, True):
        g = gpu_forward(inp, deterministic=det, out_dtype=torch.bfloat16)
        check(inp, g, out_bf16=True)


def test_zero_tokens():
    d = device_inputs(workloads.generate(workloads.small_config(4, 16, 16, 4, 2, cfg_id=401)))
    out, sel, w = moe.forward(d["x"][:0], d["router"], d["gate_up"], d["down"], top_k=2)
    assert out.shape == (0, 16) and sel.shape == (0, 2)


def test_errors_map_to_python_exceptions():
    d = device_inputs(workloads.generate(workloads.small_config(4, 16, 16, 4, 2, cfg_id=402)))
    with pytest.raises(ValueError):
        moe.forward(d["x"], d["router"], d["gate_up"], d["down"], top_k=0)
    with pytest.raises(ValueError):
        moe.forward(d["x"], d["router"], d["gate_up"], d["down"], top_k=5)
    with pytest.raises(NotImplementedError):
        moe.forward(d["x"], d["router"], d["gate_up"], d["down"], top_k=2, act="gelu")
    with pytest.raises(TypeError):
        moe.forward(d["x"].double(), d["router"], d["gate_up"], d["down"], top_k=2)
    with pytest.raises(ValueError):
        moe.forward(d["x"], d["router"], d["gate_up"][:, :8], d["down"], top_k=2)


def test_deterministic_runs_are_bitwise_identical():
    cfg = workloads.small_config(1500, 128, 256, 16, 4, dtype="bf16", router_bias="zipf", cfg_id=403)
    inp = workloads.generate(cfg)
    d = device_inputs(inp)
    a = gpu_forward(inp, d, deterministic=True)
    b = gpu_forward(inp, d, deterministic=True)
    assert np.array_equal(a["out"], b["out"])
    # K = 2 atomics onto a zeroed buffer are also reproducible (0 + a + b = 0 + b + a).
    cfg2 = dict(cfg, K=2)
    inp2 = workloads.generate(cfg2)
    d2 = device_inputs(inp2)
    a2 = gpu_forward(inp2, d2)
    b2 = gpu_forward(inp2, d2)
    assert np.array_equal(a2["out"], b2["out"])


@pytest.mark.parametrize("T", [3000, 341, 1])  # multi-block sort; one-block sort (T*K <= 1024); one token
def test_dispatch_is_a_stable_counting_sort(T):
    cfg = workloads.small_config(T, 64, 64, 24, 3, dtype="bf16", router_bias="zipf", cfg_id=404)
    inp = workloads.generate(cfg)
    d = device_inputs(inp)
    r = moe.dispatch(d["x"], d["router"], top_k=3, router_bias=d["router_bias"])
    torch.cuda.synchronize()
    sel = r["selected_experts"].cpu().numpy()
    counts = r["expert_counts"].cpu().numpy()
    offs = r["expert_offsets"].cpu().numpy()
    tok = r["sorted_token"].cpu().numpy()
    slot = r["sorted_slot"].cpu().numpy()
    flat = sel.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=24))
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)]))
    # stable: exactly a stable argsort of the flattened expert ids
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(slot, order)
    assert np.array_equal(tok, order // 3)
    # the same router kernel as the full forward
    assert np.array_equal(sel, gpu_forward(inp, d)["sel"])


@pytest.mark.parametrize("E,T,K", [(64, 100, 4), (65, 100, 4), (128, 100, 8), (256, 250, 4),   # one-block sort
                                   (64, 3000, 4), (128, 3000, 8), (256, 5000, 4)])            # multi-block sort
def test_dispatch_many_experts_last_expert_loaded(E, T, K):
    """Routers with 64 or more experts, the highest-index expert favoured by a
    router bias so that it holds many rows: the end offset (written by thread
    E of the scan block, in another wave than thread 0) must be T*K exactly,
    and the order a stable argsort, on both the one-block (T*K <= 1024) and
    the multi-block sort."""
    cfg = workloads.small_config(T, 64, 64, E, K, dtype="bf16", router_bias="last_heavy", cfg_id=405)
    inp = workloads.generate(cfg)
    d = device_inputs(inp)
    _say("dispatch E=%d T=%d K=%d" % (E, T, K))
    r = moe.dispatch(d["x"], d["router"], top_k=K, router_bias=d["router_bias"])
    torch.cuda.synchronize()
    sel = r["selected_experts"].cpu().numpy()
    counts = r["expert_counts"].cpu().numpy()
    offs = r["expert_offsets"].cpu().numpy()
    flat = sel.ravel()
    assert counts[E - 1] == T, "the favoured expert should take every token"
    assert offs[E] == T * K
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(r["sorted_slot"].cpu().numpy(), order)
    assert np.array_equal(r["sorted_token"].cpu().numpy(), order // K)


# ----------------------------------------------------- full-size workloads
_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        _say("generating %s" % name)
        _CACHE[name] = workloads.generate(name)
    return _CACHE[name]


def _prefill_family():
    if "prefill" not in _CACHE:
        _CACHE.clear()
        _say("generating prefill")
        _CACHE["prefill"] = workloads.generate("prefill")
    return _CACHE["prefill"]


@pytest.mark.slow
def test_prefill_mixtral_shape_stratified():
    inp = _prefill_family()
    d = device_inputs(inp)
    _say("prefill T=8192 D=4096 F=14336 E=8 K=2 bf16")
    g = gpu_forward(inp, d)
    check_full_properties(inp, g)
    tok = _strata(inp, g, d)
    st = check(inp, g, tokens=tok)
    _say(str(st))
    # the same layer with the atomic combine (K = 2: reproducible) and with a
    # bf16 output, on the same compared tokens
    ga = gpu_forward(inp, d, deterministic=False)
    np.testing.assert_array_equal(ga["sel"], g["sel"])
    _say("atomic combine " + str(check(inp, ga, tokens=tok)))
    gb = gpu_forward(inp, d, out_dtype=torch.bfloat16)
    _say("bf16 output " + str(check(inp, gb, tokens=tok, out_bf16=True)))
    _CACHE["prefill_dev"] = d
    _CACHE["prefill_gpu"] = g


@pytest.mark.slow
def test_decode_mixtral_shape_full():
    base = _prefill_family()
    inp = dict(base, cfg=dict(base["cfg"], T=64), x=base["x"][:64])
    d = _CACHE.get("prefill_dev") or device_inputs(base)
    dd = dict(d, x=d["x"][:64].contiguous())
    _say("decode T=64 D=4096 F=14336 E=8 K=2 bf16")
    g = gpu_forward(inp, dd)
    check_full_properties(inp, g)
    st = check(inp, g)
    _say(str(st))
    # the entry point for callers that cannot allocate holds this shape in
    # its fixed scratch array and gives bitwise the same results
    c = inp["cfg"]
    desc = moe.make_desc(64, c["D"], c["F"], c["E"], c["K"], dtype=torch.bfloat16, deterministic=True)
    assert moe.moe_workspace_bytes(desc) <= moe.MOE_NOALLOC_MAX_BYTES
    out = torch.empty((64, c["D"]), dtype=torch.float32, device="cuda")
    sel = torch.empty((64, c["K"]), dtype=torch.int64, device="cuda")
    w = torch.empty((64, c["K"]), dtype=torch.float32, device="cuda")
    st = moe.moe_forward_noalloc(desc, dd["x"].data_ptr(), dd["router"].data_ptr(), dd["gate_up"].data_ptr(),
                                 dd["down"].data_ptr(), None, None, None, out.data_ptr(), sel.data_ptr(),
                                 w.data_ptr(), None, None, torch.cuda.current_stream().cuda_stream)
    assert st == moe.MOE_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), g["out"])
    np.testing.assert_array_equal(sel.cpu().numpy(), g["sel"])
    np.testing.assert_array_equal(w.cpu().numpy(), g["weights"])
    # the decode batch is the first 64 prefill tokens: same routing and output
    if "prefill_gpu" in _CACHE:
        pg = _CACHE["prefill_gpu"]
        assert np.array_equal(g["sel"], pg["sel"][:64])
        rms = np.sqrt(np.mean(pg["out"][:64] ** 2))
        assert np.abs(g["out"] - pg["out"][:64]).max() <= 1e-3 * rms
    _CACHE.pop("prefill_dev", None)


@pytest.mark.slow
def test_decode_128_tokens_full_size_64_row_tiles():
    """The first 128 prefill tokens at the real Mixtral shape: 32 rows per
    expert on average, so both GEMMs run the 64-row weight-streaming tiles
    (each expert's weights read once); every token compared."""
    base = _prefill_family()
    c = base["cfg"]
    T = 128
    inp = dict(base, cfg=dict(c, T=T), x=base["x"][:T])
    d = _CACHE.get("prefill_dev") or device_inputs(base)
    dd = dict(d, x=d["x"][:T].contiguous())
    desc = moe.make_desc(T, c["D"], c["F"], c["E"], c["K"], dtype=torch.bfloat16, deterministic=True)
    plan = moe.moe_gemm_plan(desc)
    assert plan["gate_up"]["variant"] == plan["down"]["variant"] == "stream_m64_narrow", plan
    _say("decode T=128 D=4096 F=14336 E=8 K=2 bf16 (64-row streaming tiles)")
    g = gpu_forward(inp, dd)
    assert int(g["counts"].max()) > 32  # some expert holds both halves of a tile
    check_full_properties(inp, g)
    _say(str(check(inp, g)))


@pytest.mark.slow
def test_one_expert_share_full_size():
    """One GPU's share under expert sharding: E = K = 1 at the Mixtral D and F
    (every token goes to the one expert, whose weight p/(p+1e-9) is 1 in
    fp32), 2080 rows = 8 full 256-row tiles and a 32-row tail, which both
    projections take into their last row tile (112 and 16 column tiles: one
    round fewer)."""
    inp = workloads.generate(workloads.small_config(2080, 4096, 14336, 1, 1, dtype="bf16", cfg_id=960))
    _say("one expert T=2080 D=4096 F=14336 E=1 K=1 bf16")
    g = gpu_forward(inp, deterministic=True)
    check_full_properties(inp, g)
    assert np.all(g["weights"] == 1.0) and np.all(g["sel"] == 0)
    st = check(inp, g, tokens=_strata(inp, g))
    _say(str(st))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["fine", "fine_zero"])
def test_fine_grained_128_experts_stratified(name):
    inp = _inputs(name)
    d = device_inputs(inp)
    _say("%s T=16384 D=2048 F=768 E=128 K=8 bf16" % name)
    g = gpu_forward(inp, d, deterministic=name == "fine_zero")
    check_full_properties(inp, g)
    st = check(inp, g, tokens=_strata(inp, g, d))
    _say(str(st))
    if name == "fine_zero":
        z = workloads.zero_load_experts(128)
        assert np.all(g["counts"][z] == 0)
        # Poison the experts no token reaches: the output must not change.
        gu, dn = d["gate_up"].clone(), d["down"].clone()
        zt = torch.from_numpy(z).to(gu.device)
        gu[zt] = float("nan")
        dn[zt] = float("nan")
        g2 = gpu_forward(inp, dict(d, gate_up=gu, down=dn), deterministic=True)
        assert np.array_equal(g2["out"], g["out"])
    _CACHE.pop(name, None)


def test_token_permutation_equivariance():
    """Permuting the tokens permutes the outputs (the exercise's layer mixes no
    tokens): same selections and weights bitwise, outputs within the fp32 bar
    (a permutation moves rows between tiles and K-split parts, which may change
    the fp32 summation order of the down projection)."""
    inp = workloads.generate(workloads.small_config(2048, 256, 512, 4, 2, dtype="bf16", cfg_id=950))
    perm = np.random.default_rng(9).permutation(2048)
    a = gpu_forward(inp)
    pinp = dict(inp, x=inp["x"][perm])
    b = gpu_forward(pinp)
    np.testing.assert_array_equal(b["sel"], a["sel"][perm])
    np.testing.assert_array_equal(b["weights"], a["weights"][perm])
    np.testing.assert_array_equal(b["logits"], a["logits"][perm])
    ref = a["out"][perm].astype(np.float64)
    err = np.abs(b["out"] - ref)
    assert err.max() <= 1e-5 * max(np.abs(ref).max(), 1e-30), err.max()


@pytest.mark.parametrize("E,K", [(8, 2), (128, 8)])
def test_router_is_batch_invariant(E, K):
    """Both router paths (16-token blocks for up to 64 experts; the logits
    kernel of 64-token blocks above) sum each (t, e) in one order whatever the
    batch: a permuted batch and a prefix of it give the same logits,
    selections and weights bitwise."""
    inp = workloads.generate(workloads.small_config(1000, 512, 128, E, K, dtype="bf16", router_bias="zipf",
                                                    cfg_id=952 + E))
    perm = np.random.default_rng(11).permutation(1000)
    a = gpu_forward(inp)
    b = gpu_forward(dict(inp, x=inp["x"][perm]))
    for k in ("sel", "weights", "logits"):
        np.testing.assert_array_equal(b[k], a[k][perm])
    T1 = 300
    c = gpu_forward(dict(inp, x=inp["x"][:T1], cfg=dict(inp["cfg"], T=T1)))
    for k in ("sel", "weights", "logits"):
        np.testing.assert_array_equal(c[k], a[k][:T1])


def test_misaligned_views_are_realigned():
    """Views that start off a 16-byte boundary go through the binding (which
    copies them) and give the aligned tensors' results bitwise."""
    inp = workloads.generate(workloads.small_config(300, 128, 256, 4, 2, dtype="bf16", cfg_id=953))
    d = device_inputs(inp)
    c = inp["cfg"]

    def off_by_one(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 != 0
        return v

    def run(x, gu, dn):
        out, sel, w = moe.forward(x, d["router"], gu, dn, top_k=c["K"], router_bias=d["router_bias"])
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy()

    a = run(d["x"], d["gate_up"], d["down"])
    b = run(off_by_one(d["x"]), off_by_one(d["gate_up"]), off_by_one(d["down"]))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_timed_entry_point_matches_forward():
    """moe_forward_timed is moe_forward plus event records: bitwise equal outputs."""
    import ctypes
    inp = workloads.generate(workloads.small_config(1000, 128, 256, 8, 2, dtype="bf16", cfg_id=951))
    d = device_inputs(inp)
    c = inp["cfg"]
    T, D, F, E, K = c["T"], c["D"], c["F"], c["E"], c["K"]
    desc = moe.make_desc(T, D, F, E, K, dtype=torch.bfloat16, deterministic=True)
    nbytes = moe.moe_workspace_bytes(desc)
    outs = []
    for timed in (False, True):
        ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        out = torch.empty((T, D), dtype=torch.float32, device="cuda")
        sel = torch.empty((T, K), dtype=torch.int64, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        args = [d["x"].data_ptr(), d["router"].data_ptr(), d["gate_up"].data_ptr(), d["down"].data_ptr(), None, None,
                None, out.data_ptr(), sel.data_ptr(), w.data_ptr(), None, None, ws.data_ptr(), nbytes, stream]
        if timed:
            import bench
            hip = bench.Hip()
            evs = [hip.event() for _ in range(moe.MOE_STAGE_EVENTS)]
            handles = (ctypes.c_void_p * moe.MOE_STAGE_EVENTS)(*evs)
            assert moe.moe_forward_timed(desc, *args, handles, moe.MOE_STAGE_EVENTS) == moe.MOE_OK
            torch.cuda.synchronize()
            assert hip.elapsed_ms(evs[0], evs[-1]) > 0.0
            for ev in evs:
                hip.destroy(ev)
        else:
            assert moe.moe_forward(desc, *args) == moe.MOE_OK
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), sel.cpu().numpy(), w.cpu().numpy()))
    for x, y in zip(*outs):
        np.testing.assert_array_equal(x, y)
