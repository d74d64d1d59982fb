"""GPU parity of the routing options against the oracle (needs an MI355X).

Routing replay (Dew "Mixture of experts", "Router behavior"), the dynamic
threshold (ES-MoE "API", settings of "ESMoE"), capacity-factor drops (Dew,
"Expert computation and placement") and the balancing statistics (ES-MoE
"API", "Balancing objectives"), all through the C ABI.

Bars: selected experts, kept flags, expert counts and the sorted order are
bit-exact (a token whose own selection is a near tie, |p_k - p_(k+1)| <=
1e-5, may differ; the oracle then replays the GPU's selection for it, so the
capacity decisions that follow use the same selection); weights |delta| <=
1e-5; out as in the plain layer; statistics |delta| <= 1e-5 relative (means,
objectives) and exact [gate > 0] fractions.  Thresholds are placed at least
2e-6 away from every weight they are compared with (the fp32 weights differ
from the oracle's by ~1e-7), so the fp32 decision cannot differ.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import (BF16_TOL, F32_TOL, NEAR_TIE, W_TOL, assert_strata_covered, device_inputs, stratified_tokens,
                    to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no ROCm device", allow_module_level=True)

import sparse_mixture_experts_02_amd as moe  # noqa: E402

STATS_TOL = 1e-5


def _say(msg):
    print("[gpu-routing] " + msg, flush=True)


def run_gpu(inp, dev=None, *, deterministic=True, **opts):
    c = inp["cfg"]
    d = dev if dev is not None else device_inputs(inp)
    for k in ("replay", "replay_mask"):
        if opts.get(k) is not None:
            opts[k] = torch.from_numpy(np.ascontiguousarray(opts[k])).cuda()
    out, sel, w, logits, counts, kept, stats = moe.forward(
        d["x"], d["router"], d["gate_up"], d["down"], top_k=c["K"], norm_topk_prob=c["norm"],
        act="silu" if c["act"] == "swiglu" else "relu", router_bias=d["router_bias"], up_bias=d["up_bias"],
        down_bias=d["down_bias"], deterministic=deterministic, return_logits=True, return_counts=True,
        return_kept=True, return_stats=True, **opts)
    torch.cuda.synchronize()
    return dict(out=out.float().cpu().numpy().reshape(-1, out.shape[-1]), sel=sel.cpu().numpy(),
                weights=w.cpu().numpy(), logits=logits.cpu().numpy(), counts=counts.cpu().numpy(),
                kept=kept.cpu().numpy(), stats=stats.cpu().numpy())


def safe_threshold(inp, q, margin=2e-6):
    """A threshold near the q-quantile of the non-leading renormalised weights
    of the oracle's own routing, at least `margin` away from every one."""
    c = inp["cfg"]
    r = oracle.route(inp["x"], inp["router"], top_k=c["K"], norm=c["norm"], router_bias=inp.get("router_bias"))
    w = np.sort(r["weights"][:, 1:].ravel())
    target = float(np.quantile(w, q))
    thr = target
    for _ in range(10000):
        if w.size == 0 or np.min(np.abs(w - thr)) > margin:
            return thr
        thr += 2 * margin
    raise AssertionError("no threshold with margin near %g" % target)


def reference(inp, gpu, tokens=None, replay=None, replay_mask=None, **opts):
    """The oracle with the same options; tokens whose own selection differs
    from the GPU's only through a near tie get the GPU's selection replayed."""
    c = inp["cfg"]
    T, K = c["T"], c["K"]
    ref = oracle.forward_routed(inp, tokens=tokens, replay=replay, replay_mask=replay_mask, **opts)
    covered = np.zeros(T, bool)
    if replay is not None:
        covered = np.ones(T, bool) if replay_mask is None else np.asarray(replay_mask, bool)
        bad = (np.asarray(replay) < 0) | (np.asarray(replay) >= c["E"])
        covered &= ~bad.any(1)
    diff = np.nonzero(~np.all(gpu["sel"] == ref["sel"], axis=1))[0]
    if diff.size == 0:
        return ref, 0
    assert not covered[diff].any(), "a replayed token's selection differs at %s" % diff[covered[diff]][:5]
    ps = -np.sort(-ref["probs"][diff], axis=1)[:, :K]
    pg = np.take_along_axis(ref["probs"][diff], gpu["sel"][diff], axis=1)
    near = np.all(np.abs(pg - ps) <= NEAR_TIE, axis=1)
    assert near.all(), "selection differs beyond a near tie at tokens %s" % diff[~near][:5]
    assert diff.size <= max(2, 0.02 * T), "too many near ties: %d" % diff.size
    rec = ref["sel"].copy() if replay is None else np.asarray(replay).copy()
    rec[diff] = gpu["sel"][diff]
    mask = covered.copy()
    mask[diff] = True
    ref = oracle.forward_routed(inp, tokens=tokens, replay=rec, replay_mask=mask, **opts)
    return ref, int(diff.size)


def compare(inp, gpu, ref, tokens=None):
    c = inp["cfg"]
    T = c["T"]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    np.testing.assert_array_equal(gpu["sel"], ref["sel"])
    np.testing.assert_array_equal(gpu["kept"], ref["kept"])
    dw = np.abs(gpu["weights"] - ref["weights"]).max()
    assert dw <= W_TOL, "weights differ by %g" % dw
    kept_sel = np.where(ref["kept"], ref["sel"], c["E"])
    np.testing.assert_array_equal(gpu["counts"], np.bincount(kept_sel.ravel(), minlength=c["E"] + 1)[:c["E"]])
    go = gpu["out"][tok].astype(np.float64)
    ro = ref["out"]
    rms = float(np.sqrt(np.mean(ro ** 2))) if ro.size else 0.0
    err = np.abs(go - ro)
    if rms == 0.0:
        assert np.all(go == 0.0)
        stat = 0.0
    elif c["dtype"] == "bf16":
        stat = float(err.max() / rms)
        assert stat <= BF16_TOL, "max|delta|/RMS = %g" % stat
    else:
        den = np.maximum(np.abs(ro), rms)
        stat = float((err / den).max())
        assert np.all(err <= F32_TOL * den), "fp32 out differs: worst rel %g" % stat
    # dropped slots add nothing: a token with no kept slot has out exactly 0
    none_kept = ~ref["kept"][tok].any(1)
    assert np.all(gpu["out"][tok][none_kept] == 0.0)
    return stat


def compare_stats(inp, gpu, ref):
    E = inp["cfg"]["E"]
    s, r = gpu["stats"], ref["stats"]
    np.testing.assert_allclose(s[:E], r["mean_probs"], rtol=STATS_TOL, atol=1e-7)
    np.testing.assert_allclose(s[E:2 * E], r["mean_gate"], rtol=STATS_TOL, atol=1e-7)
    np.testing.assert_allclose(s[2 * E:3 * E], r["frac_routed"], rtol=1e-6, atol=1e-7)
    for i, k in enumerate(("switch", "gshard", "master", "gshard_probs")):
        assert abs(s[3 * E + i] - r[k]) <= STATS_TOL * max(abs(r[k]), 1e-3), (k, s[3 * E + i], r[k])


def strata(sel, kept, E, strip=64):
    """Tokens of the first and last row of every `strip`-row strip of every
    expert segment of the kept assignments' sorted order (every row tile of
    both GEMMs has compared rows), plus tokens 0 and T-1."""
    T = sel.shape[0]
    tok = np.unique(np.concatenate([stratified_tokens(sel, E, strip, kept)[0], [0, T - 1]]))
    assert_strata_covered(tok, sel, E, strip, kept)
    _say("compared tokens %d" % tok.size)
    return tok


def _cfg(T, D, F, E, K, dtype="f32", **kw):
    return workloads.generate(workloads.small_config(T, D, F, E, K, dtype=dtype, **kw))


# ------------------------------------------------------------------ replay
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_with_mask(dtype):
    inp = _cfg(300, 72, 200, 6, 2, dtype=dtype, cfg_id=201)
    T, E, K = 300, 6, 2
    rng = np.random.default_rng(11)
    record = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    record[5] = [7, 0]     # not an expert: token 5 keeps its own choice
    mask = rng.random(T) < 0.7
    _say("replay %s T=%d covered=%d" % (dtype, T, mask.sum()))
    g = run_gpu(inp, replay=record, replay_mask=mask)
    ref, ex = reference(inp, g, replay=record, replay_mask=mask)
    st = compare(inp, g, ref)
    compare_stats(inp, g, ref)
    cov = mask.copy()
    cov[5] = False
    np.testing.assert_array_equal(g["sel"][cov], record[cov])
    _say("err %g exempt %d" % (st, ex))


def test_replay_of_own_selection_is_bitwise_identity():
    inp = _cfg(257, 64, 96, 8, 3, cfg_id=202)
    d = device_inputs(inp)
    a = run_gpu(inp, d)
    b = run_gpu(inp, d, replay=a["sel"])
    for k in ("out", "sel", "weights", "counts"):
        np.testing.assert_array_equal(a[k], b[k])


def test_replay_duplicate_experts():
    inp = _cfg(64, 64, 96, 4, 2, cfg_id=203)
    record = np.tile(np.array([[2, 2]]), (64, 1))
    record[::3] = [[1, 3]]
    g = run_gpu(inp, replay=record)
    ref, _ = reference(inp, g, replay=record)
    compare(inp, g, ref)


# -------------------------------------------------------- dynamic threshold
@pytest.mark.parametrize("T,D,F,E,K,dtype,q", [
    (300, 72, 200, 6, 2, "f32", 0.5),
    (257, 64, 96, 16, 4, "f32", 0.3),
    (1000, 128, 256, 8, 2, "bf16", 0.5),
    (129, 64, 64, 128, 8, "bf16", 0.7),
])
def test_dynamic_threshold(T, D, F, E, K, dtype, q):
    inp = _cfg(T, D, F, E, K, dtype=dtype, cfg_id=210 + K)
    thr = safe_threshold(inp, q)
    _say("threshold T=%d E=%d K=%d thr=%g" % (T, E, K, thr))
    g = run_gpu(inp, dynamic_threshold=thr)
    ref, ex = reference(inp, g, threshold=thr)
    dropped = int((~ref["kept"]).sum())
    assert dropped > 0 and ref["kept"][:, 0].all()
    st = compare(inp, g, ref)
    compare_stats(inp, g, ref)
    _say("dropped %d err %g exempt %d" % (dropped, st, ex))


def test_threshold_worked_example_on_gpu():
    """Hand-derived threshold cases of the exercise's two tokens through the
    whole GPU layer (0.4 drops both second slots, 0.3 only token 1's)."""
    import json
    import os
    from test_oracle_routing_pins import _worked_layer
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "routing_options_worked.json")))
    lay, _ = _worked_layer(g["probs"], g["expert_outs"])
    d = {k: to_device(v) for k, v in lay.items() if k != "cfg"}
    for c in g["threshold_cases"][:2]:
        out, sel, w, kept = moe.forward(d["x"], d["router"], d["gate_up"], d["down"], top_k=2, act="relu",
                                        dynamic_threshold=c["threshold"], return_kept=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kept.cpu().numpy().astype(int), c["kept"])
        np.testing.assert_allclose(w.cpu().numpy(), c["weights"], rtol=0, atol=g["atol_layer"])
        np.testing.assert_allclose(out.cpu().numpy(), c["out"], rtol=0, atol=g["atol_layer"])


# ---------------------------------------------------------- capacity factor
@pytest.mark.parametrize("T,D,F,E,K,dtype,L,cf,det", [
    (512, 64, 128, 8, 2, "f32", 64, 0.5, True),
    (512, 64, 128, 8, 2, "f32", 64, 0.5, False),
    (600, 96, 160, 6, 3, "bf16", 200, 0.8, True),
    (1024, 128, 256, 16, 4, "bf16", 1024, 1.0, True),
    (96, 32, 64, 4, 2, "f32", 1, 1.0, True),      # one-token sequences: one slot per expert
])
def test_capacity(T, D, F, E, K, dtype, L, cf, det):
    inp = _cfg(T, D, F, E, K, dtype=dtype, cfg_id=220 + K)
    _say("capacity T=%d E=%d K=%d L=%d cf=%g det=%s" % (T, E, K, L, cf, det))
    g = run_gpu(inp, capacity_factor=cf, seq_len=L, deterministic=det)
    ref, ex = reference(inp, g, capacity_factor=cf, seq_len=L)
    dropped = int((~ref["kept"]).sum())
    st = compare(inp, g, ref)
    compare_stats(inp, g, ref)
    _say("slots %s dropped %d err %g exempt %d" % (ref["slots"], dropped, st, ex))


def test_capacity_with_threshold_and_replay():
    T, E, K = 400, 8, 3
    inp = _cfg(T, 64, 96, E, K, cfg_id=230)
    rng = np.random.default_rng(12)
    record = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    mask = rng.random(T) < 0.5
    thr = safe_threshold(inp, 0.3)
    g = run_gpu(inp, replay=record, replay_mask=mask, dynamic_threshold=thr, capacity_factor=0.7, seq_len=100)
    ref, _ = reference(inp, g, replay=record, replay_mask=mask, threshold=thr, capacity_factor=0.7, seq_len=100)
    assert (~ref["kept"]).sum() > 0
    compare(inp, g, ref)
    compare_stats(inp, g, ref)


def test_capacity_zero_slots_and_no_drop_limits():
    inp = _cfg(64, 32, 64, 8, 2, cfg_id=231)
    d = device_inputs(inp)
    g = run_gpu(inp, d, capacity_factor=0.25, seq_len=1)   # floor(max(0.25, 0.25)) = 0 slots
    assert not g["kept"].any() and np.all(g["out"] == 0.0) and np.all(g["counts"] == 0)
    base = run_gpu(inp, d)
    big = run_gpu(inp, d, capacity_factor=100.0)
    for k in ("out", "sel", "weights", "counts"):
        np.testing.assert_array_equal(big[k], base[k])
    assert big["kept"].all()


def test_capacity_dispatch_order_is_exact():
    """The sorted order of the kept slots: inside each expert's segment, the
    kept assignments in increasing (t, k)."""
    T, E, K, L = 700, 8, 2, 100
    inp = _cfg(T, 64, 32, E, K, cfg_id=232)
    d = device_inputs(inp)
    r = moe.dispatch(d["x"], d["router"], top_k=K, capacity_factor=0.6, seq_len=L)
    torch.cuda.synchronize()
    sel = r["selected_experts"].cpu().numpy()
    kept = r["kept"].cpu().numpy()
    ref = oracle.route(inp["x"], inp["router"], top_k=K)
    ref_sel = ref["sel"]
    # no decision here is close: the K+1 largest probabilities of every token
    # are > 1e-6 apart (about 6.6e-6 at the closest), far above fp32 rounding
    top = -np.sort(-ref["probs"], axis=1)[:, :K + 1]
    assert np.min(-np.diff(top, axis=1)) > 1e-6
    np.testing.assert_array_equal(sel, ref_sel)
    slots = oracle.capacity_slots(L, K, E, 0.6)
    ref_kept = oracle.capacity(ref_sel, ref["kept"], num_experts=E, seq_len=L, slots=slots)
    np.testing.assert_array_equal(kept, ref_kept)
    flat = np.nonzero(ref_kept.ravel())[0]
    es = ref_sel.ravel()[flat]
    order = flat[np.argsort(es, kind="stable")]
    counts = np.bincount(es, minlength=E)
    np.testing.assert_array_equal(r["expert_counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(r["expert_offsets"].cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
    n = int(counts.sum())
    np.testing.assert_array_equal(r["sorted_slot"].cpu().numpy()[:n], order)
    np.testing.assert_array_equal(r["sorted_token"].cpu().numpy()[:n], order // K)


# ------------------------------------------------ small and ragged batches
@pytest.mark.parametrize("T,E,K,dtype", [(1, 8, 2, "f32"), (17, 16, 4, "bf16"), (40, 8, 2, "bf16"),
                                         (63, 16, 3, "f32"), (64, 16, 16, "bf16")])
def test_small_batches_with_routing_options(T, E, K, dtype):
    """Decode-sized batches (one token; router blocks of 16 tokens with a
    ragged last block; K = E) through the one-block sort, with replay of a
    masked record, the dynamic threshold and the per-block statistics."""
    inp = _cfg(T, 64, 96, E, K, dtype=dtype, cfg_id=290 + T)
    rng = np.random.default_rng(T)
    record = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    mask = rng.random(T) < 0.5
    _say("fused route+sort T=%d E=%d K=%d %s" % (T, E, K, dtype))
    g = run_gpu(inp, replay=record, replay_mask=mask)
    ref, _ = reference(inp, g, replay=record, replay_mask=mask)
    compare(inp, g, ref)
    compare_stats(inp, g, ref)
    np.testing.assert_array_equal(g["sel"][mask], record[mask])
    np.testing.assert_array_equal(g["counts"], np.bincount(g["sel"].ravel(), minlength=E))
    thr = safe_threshold(inp, 0.5)
    g2 = run_gpu(inp, dynamic_threshold=thr)
    ref2, _ = reference(inp, g2, threshold=thr)
    compare(inp, g2, ref2)
    compare_stats(inp, g2, ref2)


# ------------------------------------------------------------- statistics
@pytest.mark.parametrize("name_or_cfg", ["tiny", "relu"])
def test_stats_plain_routing(name_or_cfg):
    inp = workloads.generate(name_or_cfg)
    g = run_gpu(inp)
    ref, _ = reference(inp, g)
    compare(inp, g, ref)
    compare_stats(inp, g, ref)
    E = inp["cfg"]["E"]
    s = g["stats"]
    assert abs(s[3 * E + 2] - (s[3 * E + 1] - 1.0) / E ** 2) <= 1e-6  # master = (gshard - 1)/E^2


def test_stats_are_reproducible():
    inp = _cfg(4096, 64, 32, 128, 8, dtype="bf16", cfg_id=240)
    d = device_inputs(inp)
    a = run_gpu(inp, d)
    b = run_gpu(inp, d)
    np.testing.assert_array_equal(a["stats"], b["stats"])
    ref, _ = reference(inp, a, tokens=np.arange(8))
    compare_stats(inp, a, ref)


# ------------------------------------------------------ full-size workloads
@pytest.mark.slow
def test_prefill_capacity_full_size_stratified():
    """The Mixtral-shaped prefill (T=8192) as two 4096-token sequences at
    capacity factor 1.0, compared on the tokens of every 64-row strip's first
    and last row of every expert segment; kept flags and counts for every
    token."""
    inp = workloads.generate("prefill")
    T = inp["cfg"]["T"]
    _say("prefill capacity T=%d" % T)
    g = run_gpu(inp, capacity_factor=1.0, seq_len=4096)
    tok = strata(g["sel"], g["kept"], inp["cfg"]["E"])
    ref, ex = reference(inp, g, tokens=tok, capacity_factor=1.0, seq_len=4096)
    st = compare(inp, g, ref, tokens=tok)
    compare_stats(inp, g, ref)
    _say("slots %d dropped %d err %g exempt %d" % (ref["slots"], int((~ref["kept"]).sum()), st, ex))


@pytest.mark.slow
def test_fine_experts_threshold_and_capacity_full_size_stratified():
    """The 128-expert workload (T=16384, K=8, Zipf-skewed loads) with a
    dynamic threshold and capacity factor 1.25 over four 4096-token
    sequences: kept flags, counts and statistics for every token, outputs on
    the tokens of every 64-row strip's first and last row of every expert
    segment."""
    inp = workloads.generate("fine")
    T = inp["cfg"]["T"]
    thr = safe_threshold(inp, 0.3)
    _say("fine threshold %.6f + capacity 1.25 x 4096, T=%d" % (thr, T))
    g = run_gpu(inp, dynamic_threshold=thr, capacity_factor=1.25, seq_len=4096)
    tok = strata(g["sel"], g["kept"], inp["cfg"]["E"])
    ref, ex = reference(inp, g, tokens=tok, threshold=thr, capacity_factor=1.25, seq_len=4096)
    st = compare(inp, g, ref, tokens=tok)
    compare_stats(inp, g, ref)
    _say("slots %d dropped %d err %g exempt %d" % (ref["slots"], int((~ref["kept"]).sum()), st, ex))


@pytest.mark.slow
def test_prefill_replay_full_size_stratified():
    """The Mixtral-shaped prefill replaying a record that differs from the own
    selection (each covered token's experts shifted by one) on 60% of the
    tokens."""
    inp = workloads.generate("prefill")
    c = inp["cfg"]
    T, E, K = c["T"], c["E"], c["K"]
    own = oracle.route(inp["x"], inp["router"], top_k=K)["sel"]
    record = (own + 1) % E
    mask = np.random.default_rng(6).random(T) < 0.6
    _say("prefill replay T=%d covered=%d" % (T, mask.sum()))
    g = run_gpu(inp, replay=record, replay_mask=mask)
    tok = strata(g["sel"], g["kept"], E)
    ref, ex = reference(inp, g, tokens=tok, replay=record, replay_mask=mask)
    st = compare(inp, g, ref, tokens=tok)
    np.testing.assert_array_equal(g["sel"][mask], record[mask])
    _say("err %g exempt %d" % (st, ex))


# ------------------------------------------------- tail rows of the last tile
@pytest.mark.parametrize("act,D,F,deterministic", [
    ("swiglu", 256, 2816, True),    # gate_up: 264 plain items vs 220 with tails; down unchanged
    ("swiglu", 5632, 2816, False),  # both projections take tails; atomic combine
    ("relu", 5632, 2816, True),     # ReLU (one weight block per output block), split down
])
def test_tail_rows_join_last_tile(act, D, F, deterministic):
    """Replay fixes the expert counts at 800 = 3*256 + 32 and 288 = 256 + 32
    (the tail joins the expert's last 256-row tile), 545 = 2*256 + 33 (one
    row too many: a tile of its own) and 767.  The work lists take the tails
    when that saves a round on the device's compute units: with 256 CUs the
    shapes are chosen so that it does (e.g. 22 column tiles: 264 items = one
    round and a split remainder, against 220 with tails).  The layer must
    match the oracle as with any other routing."""
    T, E, K = 1200, 4, 2
    counts = [800, 545, 288, 767]
    labels = np.repeat(np.arange(E), counts)
    record = np.stack([labels[:T], labels[T:]], axis=1)
    assert np.all(record[:, 0] != record[:, 1])
    inp = _cfg(T, D, F, E, K, dtype="bf16", act=act, cfg_id=270 + D % 7)
    _say("tail rows act=%s D=%d F=%d deterministic=%s counts=%s" % (act, D, F, deterministic, counts))
    g = run_gpu(inp, replay=record, deterministic=deterministic)
    tokens = None if D <= 256 else strata(g["sel"], g["kept"], E, strip=32)
    np.testing.assert_array_equal(g["counts"], counts)
    ref, _ = reference(inp, g, tokens=tokens, replay=record)
    st = compare(inp, g, ref, tokens=tokens)
    _say("err %g" % st)
