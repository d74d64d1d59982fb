"""Pins of the oracle's routing options to things other than the oracle.

  * routing replay (Dew "Mixture of experts", section "Router behavior"):
    against a dense numpy evaluation of every expert, gathered at the recorded
    experts; uncovered tokens and invalid records keep the router's choice;
  * dynamic threshold (ES-MoE "API", settings table of "ESMoE"): values
    derived by hand from the crackedaicode exercise's printed two-token
    example, and the limits 0 (no effect) and > 1 (leader only);
  * capacity factor (Dew, section "Expert computation and placement"): the
    slot formula on hand-computed cases, a three-token case derived by hand, a
    constructed layer whose drops are known in advance, and the no-drop limit;
  * balancing objectives (ES-MoE "API", section "Balancing objectives"): the
    two-token example by hand, the closed form master = (gshard - 1)/E^2, and
    the uniform and one-hot limits.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_layer(seed, T, D, F, E, scale=0.3, router_bias=None):
    rng = np.random.default_rng(seed)
    f = lambda *s: (rng.standard_normal(s) * scale).astype(np.float32)  # noqa: E731
    return dict(x=f(T, D) / scale, router=f(E, D), gate_up=f(E, 2 * F, D), down=f(E, D, F),
                router_bias=router_bias, up_bias=None, down_bias=None)


def _inp(lay, K, norm=True, act="swiglu"):
    T, D = lay["x"].shape
    E, _, F = lay["down"].shape
    return dict(lay, cfg=dict(T=T, D=D, F=F, E=E, K=K, norm=norm, act=act))


def _dense(lay):
    """Probabilities (T,E) and every expert's SwiGLU output (T,E,D), numpy fp64."""
    x = lay["x"].astype(np.float64)
    rb = 0.0 if lay["router_bias"] is None else np.asarray(lay["router_bias"], np.float64)
    p = scipy.special.softmax(x @ lay["router"].astype(np.float64).T + rb, axis=-1)
    F = lay["down"].shape[2]
    outs = []
    for e in range(lay["router"].shape[0]):
        a = x @ lay["gate_up"][e].astype(np.float64).T
        h = scipy.special.expit(a[:, :F]) * a[:, :F] * a[:, F:]
        outs.append(h @ lay["down"][e].astype(np.float64).T)
    return p, np.stack(outs, axis=1)


def _gather(p, eo, sel, w):
    return (np.take_along_axis(eo, sel[:, :, None], axis=1) * w[:, :, None]).sum(1)


def _worked_layer(probs, expert_outs):
    """ReLU layer whose forward on x = I reproduces given probabilities and
    expert outputs (router rows ln p, W1 = I, W2[e][:, t] = expert_outs[t, e])."""
    p = np.asarray(probs, np.float64)
    eo = np.asarray(expert_outs, np.float64)
    T, E = p.shape
    D = eo.shape[2] if eo is not None else T
    x = np.eye(T, dtype=np.float32)
    router = np.log(p).T.astype(np.float32)
    W1 = np.tile(np.eye(T, T, dtype=np.float32), (E, 1, 1))
    W2 = np.transpose(eo, (1, 2, 0)).astype(np.float32)
    return dict(x=x, router=router, gate_up=W1, down=W2, router_bias=None, up_bias=None, down_bias=None,
                cfg=dict(T=T, D=T, F=T, E=E, K=2, norm=True, act="relu")), D


# ------------------------------------------------------------------ replay
def test_replay_matches_dense_gather_with_mask():
    T, E, K = 24, 6, 2
    lay = _rand_layer(31, T, 12, 8, E)
    p, eo = _dense(lay)
    rng = np.random.default_rng(5)
    record = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    mask = rng.random(T) < 0.6
    r = oracle.forward_routed(_inp(lay, K), replay=record, replay_mask=mask)
    own = np.argsort(-p.astype(np.float32), axis=1, kind="stable")[:, :K]
    sel = np.where(mask[:, None], record, own)
    ps = np.take_along_axis(p, sel, 1)
    w = ps / (ps.sum(1, keepdims=True) + 1e-9)
    np.testing.assert_array_equal(r["sel"], sel)
    np.testing.assert_allclose(r["weights"], w, rtol=1e-12)
    np.testing.assert_allclose(r["out"], _gather(p, eo, sel, w), rtol=1e-10, atol=1e-12)
    assert r["kept"].all()


def test_replay_of_own_selection_is_identity():
    lay = _rand_layer(32, 16, 8, 6, 5)
    base = oracle.forward_routed(_inp(lay, 2))
    rep = oracle.forward_routed(_inp(lay, 2), replay=base["sel"])
    np.testing.assert_array_equal(rep["out"], base["out"])
    np.testing.assert_array_equal(rep["weights"], base["weights"])


def test_replay_invalid_record_keeps_own_choice():
    lay = _rand_layer(33, 6, 8, 6, 5)
    base = oracle.forward_routed(_inp(lay, 2))
    record = np.tile(np.array([[4, 3]]), (6, 1))
    record[1] = [4, 5]      # 5 is not an expert
    record[3] = [-1, 0]
    r = oracle.forward_routed(_inp(lay, 2), replay=record)
    for t in range(6):
        want = base["sel"][t] if t in (1, 3) else record[t]
        np.testing.assert_array_equal(r["sel"][t], want)


def test_replay_duplicate_experts_weigh_twice():
    """A record naming one expert twice: both slots carry p_e / (2 p_e + guard)."""
    lay = _rand_layer(34, 4, 8, 6, 4)
    p, eo = _dense(lay)
    record = np.array([[2, 2]] * 4)
    r = oracle.forward_routed(_inp(lay, 2), replay=record)
    w = p[:, 2] / (2 * p[:, 2] + 1e-9)
    np.testing.assert_allclose(r["weights"], np.stack([w, w], 1), rtol=1e-12)
    np.testing.assert_allclose(r["out"], eo[:, 2] * (2 * w)[:, None], rtol=1e-10, atol=1e-12)


# -------------------------------------------------------- dynamic threshold
@pytest.mark.parametrize("case", range(3))
def test_threshold_worked_example(case):
    g = _load("routing_options_worked.json")
    c = g["threshold_cases"][case]
    inp, _ = _worked_layer(g["probs"], g["expert_outs"])
    r = oracle.forward_routed(inp, threshold=c["threshold"])
    np.testing.assert_array_equal(r["sel"], [[0, 1], [2, 0]])
    np.testing.assert_array_equal(r["kept"].astype(int), c["kept"])
    np.testing.assert_allclose(r["weights"], c["weights"], rtol=0, atol=g["atol_layer"])
    np.testing.assert_allclose(r["out"], c["out"], rtol=0, atol=g["atol_layer"])


def test_threshold_zero_is_no_op_and_above_one_keeps_leader():
    lay = _rand_layer(35, 20, 10, 6, 6)
    inp = _inp(lay, 3)
    base = oracle.forward_inputs(inp)
    r0 = oracle.forward_routed(inp, threshold=0.0)
    np.testing.assert_array_equal(r0["out"], base["out"])
    np.testing.assert_array_equal(r0["weights"], base["weights"])
    p, eo = _dense(lay)
    r1 = oracle.forward_routed(inp, threshold=1.5)
    np.testing.assert_array_equal(r1["kept"], np.array([[True, False, False]] * 20))
    np.testing.assert_array_equal(r1["weights"], np.array([[1.0, 0.0, 0.0]] * 20))
    lead = r1["sel"][:, 0]
    np.testing.assert_allclose(r1["out"], eo[np.arange(20), lead], rtol=1e-10, atol=1e-12)


def test_threshold_needs_renormalised_weights():
    lay = _rand_layer(36, 4, 8, 6, 4)
    with pytest.raises(ValueError):
        oracle.forward_routed(_inp(lay, 2, norm=False), threshold=0.2)


# ---------------------------------------------------------- capacity factor
@pytest.mark.parametrize("L,K,E,cf,want", [
    (4096, 2, 8, 1.0, 1024),   # ceil(8192/8) = 1024
    (4096, 2, 8, 1.25, 1280),  # 1024 * 1.25
    (1, 2, 8, 2.0, 2),         # ceil(2/8) = 1 -> max(2, 2)
    (10, 2, 8, 0.5, 1),        # ceil(20/8) = 3 -> 1.5 -> one whole slot
    (7, 1, 4, 1.1, 2),         # ceil(7/4) = 2 -> 2.2 -> 2
    (1, 1, 8, 0.25, 0),        # max(0.25, 0.25) -> no whole slot
    (16, 8, 128, 3.0, 3),      # ceil(128/128) = 1 -> 3
])
def test_capacity_slot_formula(L, K, E, cf, want):
    assert oracle.capacity_slots(L, K, E, cf) == want


def test_capacity_three_token_hand_case():
    g = _load("capacity_three_tokens.json")
    p = np.asarray(g["probs"])
    inp, _ = _worked_layer(p, np.zeros((3, 3, 3)))
    r = oracle.route(inp["x"], inp["router"], top_k=2, threshold=g["threshold"])
    np.testing.assert_array_equal(r["sel"], g["expected_sel"])
    kept = oracle.capacity(r["sel"], r["kept"], num_experts=3, seq_len=3, slots=g["slots"])
    np.testing.assert_array_equal(kept.astype(int), g["expected_kept"])
    np.testing.assert_allclose(r["weights"], g["expected_weights"], rtol=0, atol=1e-6)


def test_capacity_constructed_layer_drops_late_tokens():
    """Every token picks experts 0 and 1 (router bias +30 / +29): with 2 slots
    per sequence of 4 tokens, tokens 0-1 of each sequence keep both slots and
    tokens 2-3 lose both, so their output is exactly 0."""
    T, E, K, L = 12, 5, 2, 4
    rb = np.zeros(E, np.float32)
    rb[0], rb[1] = 30.0, 29.0
    lay = _rand_layer(37, T, 8, 6, E, scale=0.05, router_bias=rb)
    p, eo = _dense(lay)
    # ceil(L*K/E) = ceil(8/5) = 2 slots at capacity factor 1
    r = oracle.forward_routed(_inp(lay, K), capacity_factor=1.0, seq_len=L)
    assert r["slots"] == 2
    assert np.all(r["sel"] == [0, 1])
    pos = np.arange(T) % L
    np.testing.assert_array_equal(r["kept"], np.repeat((pos < 2)[:, None], K, 1))
    assert np.all(r["out"][pos >= 2] == 0.0)
    w = r["weights"]
    np.testing.assert_allclose(r["out"][pos < 2], _gather(p, eo, r["sel"], w)[pos < 2], rtol=1e-10, atol=1e-12)


def test_capacity_large_factor_drops_nothing():
    lay = _rand_layer(38, 32, 8, 6, 4)
    inp = _inp(lay, 2)
    base = oracle.forward_inputs(inp)
    r = oracle.forward_routed(inp, capacity_factor=100.0, seq_len=8)
    assert r["kept"].all()
    np.testing.assert_array_equal(r["out"], base["out"])


def test_capacity_counts_per_sequence():
    """Kept assignments per (sequence, expert) = min(routed, slots); the kept
    ones are the earliest in (token, k) order."""
    T, E, K, L = 64, 4, 2, 16
    lay = _rand_layer(39, T, 8, 6, E)
    r = oracle.forward_routed(_inp(lay, K), capacity_factor=0.75, seq_len=L)
    slots = r["slots"]
    assert slots == oracle.capacity_slots(L, K, E, 0.75) == 6
    sel, kept = r["sel"], r["kept"]
    for s in range(T // L):
        blk_sel, blk_kept = sel[s * L:(s + 1) * L].ravel(), kept[s * L:(s + 1) * L].ravel()
        for e in range(E):
            idx = np.nonzero(blk_sel == e)[0]
            assert blk_kept[idx].sum() == min(idx.size, slots)
            assert np.all(blk_kept[idx[:slots]]) and not np.any(blk_kept[idx[slots:]])


# ----------------------------------------------------- balancing objectives
def test_balance_worked_example():
    g = _load("routing_options_worked.json")
    b = g["balance"]
    c = oracle.combine(np.array(g["probs"]), np.array(g["expert_outs"]), top_k=2)
    st = oracle.balance_stats(np.array(g["probs"]), c["sel"], c["weights"])
    for k in ("mean_gate", "mean_probs", "frac_routed"):
        np.testing.assert_allclose(st[k], b[k], rtol=0, atol=g["atol"])
    for k in ("switch", "gshard", "master", "gshard_probs"):
        assert abs(st[k] - b[k]) <= g["atol"], k


def test_balance_closed_form_master():
    lay = _rand_layer(40, 50, 8, 6, 7)
    r = oracle.forward_routed(_inp(lay, 3))
    st = r["stats"]
    E = 7
    assert abs(st["master"] - (st["gshard"] - 1.0) / E ** 2) < 1e-14


def test_balance_uniform_and_one_hot_limits():
    E = 6
    # uniform: zero router -> p = 1/E; K = E -> equal gates
    lay = _rand_layer(41, 10, 8, 6, E)
    lay["router"] = np.zeros_like(lay["router"])
    st = oracle.forward_routed(_inp(lay, E))["stats"]
    assert abs(st["gshard"] - 1.0) < 1e-12 and abs(st["master"]) < 1e-14
    assert abs(st["gshard_probs"] - 1.0) < 1e-12 and abs(st["switch"] - E) < 1e-12
    # one-hot: bias +50 on expert 2, K = 1 -> every gate at expert 2
    rb = np.zeros(E, np.float32)
    rb[2] = 50.0
    lay = _rand_layer(42, 10, 8, 6, E, scale=0.05, router_bias=rb)
    st = oracle.forward_routed(_inp(lay, 1))["stats"]
    assert abs(st["gshard"] - E) < 1e-9
    assert abs(st["master"] - (E - 1) / E ** 2) < 1e-9
    np.testing.assert_array_equal(st["frac_routed"], np.eye(E)[2])
    assert abs(st["switch"] - E * st["mean_probs"][2]) < 1e-12
