"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test names what fixes the expected value: a worked example printed on
the pages, a closed form, an independent implementation run from an installed
library, a reduction to plain matrix products, brute force, or an invariant
the pages state.  Each is chosen so that a plausible slip in the oracle (a
dropped bias, gate and up swapped, a transposed operand, a wrong tie-break or
ordering, a missing guard term) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(seed, T, D, F, E, act="swiglu", biases=False, router_bias=False, scale=0.3):
    rng = np.random.default_rng(seed)
    G = 2 if act == "swiglu" else 1
    f = lambda *s: (rng.standard_normal(s) * scale).astype(np.float32)  # noqa: E731
    lay = dict(x=f(T, D) / scale, router=f(E, D), gate_up=f(E, G * F, D), down=f(E, D, F),
               router_bias=f(E) if router_bias else None,
               up_bias=f(E, G * F) if biases else None, down_bias=f(E, D) if biases else None)
    return lay


def _run(lay, K, norm=True, act="swiglu", **kw):
    return oracle.forward(lay["x"], lay["router"], lay["gate_up"], lay["down"], top_k=K, norm=norm, act=act,
                          router_bias=lay["router_bias"], up_bias=lay["up_bias"], down_bias=lay["down_bias"],
                          nthreads=2, **kw)


# --------------------------------------------------------------------------
# The exercise's two-token worked example (crackedaicode "Mixture-of-Experts
# FFN", section "Work through two tokens").
# --------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLDEN, "worked_example_two_tokens.json")) as f:
        return json.load(f)


def test_worked_example_combine():
    g = _golden()
    r = oracle.combine(np.array(g["probs"]), np.array(g["expert_outs"]), top_k=g["top_k"], norm=g["norm"])
    assert np.array_equal(r["sel"], np.array(g["expected_indices"]))
    np.testing.assert_allclose(r["out"], np.array(g["expected_out"]), rtol=0, atol=g["atol"])


def worked_example_layer():
    """A ReLU layer (D=2, F=2, E=3) whose forward on x = I reproduces the example.

    Router rows hold ln(p): for x = e_t the logits are ln p[t], so the softmax
    returns p[t] and the 0.2/0.2 tie stays exact.  W1[e] = I and b1 = 0 make
    h = relu(e_t) = e_t, and column t of W2[e] holds expert_outs[t, e], so the
    expert output for token t is exactly the printed one.
    """
    g = _golden()
    p = np.array(g["probs"])          # (T=2, E=3)
    eo = np.array(g["expert_outs"])   # (T, E, D=2)
    T, E = p.shape
    D = F = 2
    x = np.eye(2, dtype=np.float32)
    router = np.log(p).T.astype(np.float32)                  # (E, D): router[e, t] = ln p[t, e]
    W1 = np.tile(np.eye(F, D, dtype=np.float32), (E, 1, 1))  # (E, F, D)
    W2 = np.transpose(eo, (1, 2, 0)).astype(np.float32)      # (E, D, F): W2[e, :, t] = eo[t, e, :]
    return dict(x=x, router=router, gate_up=W1, down=W2, router_bias=None, up_bias=None, down_bias=None), g


def test_worked_example_full_layer():
    lay, g = worked_example_layer()
    r = _run(lay, K=2, act="relu")
    assert np.array_equal(r["sel"], np.array(g["expected_indices"]))
    np.testing.assert_allclose(r["out"], np.array(g["expected_out"]), rtol=0, atol=g["atol"])


# --------------------------------------------------------------------------
# Closed-form parameter count (same page, section "Selection does not imply
# sparse computation"): E*(2DF+F+D) + DE + E for the ReLU layer with biases.
# --------------------------------------------------------------------------
def test_param_count_closed_form():
    inp = workloads.generate("relu", T=1)
    c = inp["cfg"]
    D, F, E = c["D"], c["F"], c["E"]
    closed = E * (2 * D * F + F + D) + D * E + E
    assert closed == 16_801_800
    buffers = sum(inp[k].size for k in ("router", "router_bias", "gate_up", "up_bias", "down", "down_bias"))
    assert buffers == closed
    assert oracle.param_count(D, F, E, act="relu", expert_biases=True, router_bias=True) == closed
    # The SwiGLU block in the Hugging Face layout: router (E,D) + E*(2F*D + D*F).
    p = workloads.CONFIGS["prefill"]
    assert oracle.param_count(p["D"], p["F"], p["E"]) == 1_409_318_912


# --------------------------------------------------------------------------
# Independent implementations: the installed transformers Mixtral block
# (softmax, top-k, always renormalised) and Qwen3-MoE block (norm_topk_prob
# switch), both using the same Hugging Face weight layouts as the MoEBlock
# page.  They are run, not copied; parameters are found by shape at run time.
# --------------------------------------------------------------------------
def _hf_block(kind, D, F, E, K, norm):
    torch = pytest.importorskip("torch")
    tf = pytest.importorskip("transformers")
    if kind == "mixtral":
        from transformers.models.mixtral.modeling_mixtral import MixtralSparseMoeBlock
        cfg = tf.MixtralConfig(hidden_size=D, intermediate_size=F, num_local_experts=E, num_experts_per_tok=K)
        blk = MixtralSparseMoeBlock(cfg)
    else:
        from transformers.models.qwen3_moe.modeling_qwen3_moe import Qwen3MoeSparseMoeBlock
        cfg = tf.Qwen3MoeConfig(hidden_size=D, moe_intermediate_size=F, num_experts=E, num_experts_per_tok=K,
                                norm_topk_prob=norm)
        blk = Qwen3MoeSparseMoeBlock(cfg)
    return torch, blk.double().eval()


def _load_hf(torch, blk, lay):
    E, D = lay["router"].shape
    by_shape = {(E, D): lay["router"], lay["gate_up"].shape: lay["gate_up"], lay["down"].shape: lay["down"]}
    with torch.no_grad():
        n = 0
        for _, prm in blk.named_parameters():
            src = by_shape[tuple(prm.shape)]
            prm.copy_(torch.from_numpy(src.astype(np.float64)))
            n += 1
    assert n == 3


@pytest.mark.parametrize("kind,norm", [("mixtral", True), ("qwen3", True), ("qwen3", False)])
def test_against_transformers_block(kind, norm):
    D, F, E, K, T = 12, 10, 6, 2, 40
    lay = _rand_layer(11, T, D, F, E)
    torch, blk = _hf_block(kind, D, F, E, K, norm)
    _load_hf(torch, blk, lay)
    with torch.no_grad():
        xt = torch.from_numpy(lay["x"].astype(np.float64))[None]
        ref = blk(xt)
        ref = (ref[0] if isinstance(ref, tuple) else ref)[0].numpy()
        _, hf_w, hf_sel = blk.gate(xt[0])
    r = _run(lay, K=K, norm=norm)
    assert np.array_equal(r["sel"], hf_sel.numpy())
    # transformers keeps its routing weights in float32, hence the 1e-6 band.
    np.testing.assert_allclose(r["weights"], hf_w.double().numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


# --------------------------------------------------------------------------
# E=1, K=1: the layer reduces to plain matrix products times 1/(1+1e-9).
# --------------------------------------------------------------------------
def test_single_expert_swiglu_is_matmul():
    T, D, F = 17, 9, 13
    lay = _rand_layer(3, T, D, F, 1)
    r = _run(lay, K=1)
    x = lay["x"].astype(np.float64)
    W = lay["gate_up"][0].astype(np.float64)
    g, u = x @ W[:F].T, x @ W[F:].T
    h = g * scipy.special.expit(g) * u
    want = (h @ lay["down"][0].astype(np.float64).T) / (1.0 + 1e-9)
    np.testing.assert_allclose(r["out"], want, rtol=1e-13, atol=1e-15)
    assert np.all(r["sel"] == 0)


def test_single_expert_relu_biases_is_matmul():
    T, D, F = 15, 7, 11
    lay = _rand_layer(4, T, D, F, 1, act="relu", biases=True, router_bias=True)
    r = _run(lay, K=1, act="relu")
    x = lay["x"].astype(np.float64)
    h = np.maximum(x @ lay["gate_up"][0].astype(np.float64).T + lay["up_bias"][0], 0.0)
    y = h @ lay["down"][0].astype(np.float64).T + lay["down_bias"][0]
    np.testing.assert_allclose(r["out"], y / (1.0 + 1e-9), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Brute force: the exercise's own dense algorithm (every expert on every
# token, softmax from scipy, a stable sort for the ranking, then gather).
# --------------------------------------------------------------------------
def dense_eval(lay, K, norm, act):
    x = lay["x"].astype(np.float64)
    E = lay["router"].shape[0]
    F = lay["down"].shape[2]
    rb = 0.0 if lay["router_bias"] is None else lay["router_bias"].astype(np.float64)
    p = scipy.special.softmax(x @ lay["router"].astype(np.float64).T + rb, axis=-1)
    outs = []
    for e in range(E):
        W = lay["gate_up"][e].astype(np.float64)
        ub = 0.0 if lay["up_bias"] is None else lay["up_bias"][e].astype(np.float64)
        a = x @ W.T + ub
        h = scipy.special.expit(a[:, :F]) * a[:, :F] * a[:, F:] if act == "swiglu" else np.maximum(a, 0.0)
        db = 0.0 if lay["down_bias"] is None else lay["down_bias"][e].astype(np.float64)
        outs.append(h @ lay["down"][e].astype(np.float64).T + db)
    eo = np.stack(outs, axis=1)                                            # (T, E, D)
    idx = np.argsort(-p.astype(np.float32), axis=1, kind="stable")[:, :K]  # descending, ties -> lower index
    ps = np.take_along_axis(p, idx, axis=1)
    w = ps / (ps.sum(-1, keepdims=True) + 1e-9) if norm else ps
    out = (np.take_along_axis(eo, idx[:, :, None], axis=1) * w[:, :, None]).sum(1)
    return idx, w, out


try:
    from hypothesis import given, settings, strategies as st
    HAVE_HYP = True
except ImportError:  # pragma: no cover
    HAVE_HYP = False


if HAVE_HYP:
    @settings(max_examples=40, deadline=None)
    @given(T=st.integers(1, 8), D=st.integers(1, 16), F=st.integers(1, 16), E=st.integers(1, 6),
           kfrac=st.floats(0, 1), norm=st.booleans(), act=st.sampled_from(["swiglu", "relu"]),
           biases=st.booleans(), seed=st.integers(0, 10_000))
    def test_bruteforce_dense(T, D, F, E, kfrac, norm, act, biases, seed):
        K = 1 + int(kfrac * (E - 1))
        lay = _rand_layer(seed, T, D, F, E, act=act, biases=biases, router_bias=biases)
        idx, w, out = dense_eval(lay, K, norm, act)
        r = _run(lay, K=K, norm=norm, act=act)
        assert np.array_equal(r["sel"], idx)
        np.testing.assert_allclose(r["weights"], w, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12 * max(1.0, np.abs(out).max()))


def test_bruteforce_dense_fixed():
    for seed, (T, D, F, E, K, act) in enumerate([(5, 8, 6, 5, 3, "swiglu"), (6, 3, 4, 4, 4, "relu"),
                                                 (3, 16, 16, 6, 1, "swiglu")]):
        lay = _rand_layer(seed, T, D, F, E, act=act, biases=act == "relu", router_bias=True)
        idx, w, out = dense_eval(lay, K, True, act)
        r = _run(lay, K=K, act=act)
        assert np.array_equal(r["sel"], idx)
        np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Invariants the pages state.
# --------------------------------------------------------------------------
def test_weights_nonnegative_and_sum_to_one():
    lay = _rand_layer(5, 64, 16, 8, 8)
    r = _run(lay, K=3)
    assert np.all(r["weights"] >= 0)
    s = r["weights"].sum(1)
    np.testing.assert_allclose(s, 1.0, rtol=0, atol=1e-8)
    assert np.all(s < 1.0)  # the 1e-9 guard keeps the sum strictly below one
    # descending order of the selected probabilities
    ps = np.take_along_axis(r["probs"], r["sel"], 1)
    assert np.all(np.diff(ps, axis=1) <= 0)


def test_k1_weight_guard_closed_form():
    lay = _rand_layer(6, 32, 8, 8, 5)
    r = _run(lay, K=1)
    p = np.take_along_axis(r["probs"], r["sel"], 1)[:, 0]
    assert np.all(p == r["probs"].max(1))
    # w = p / (p + 1e-9): 1 - w equals 1e-9 / (p + 1e-9) (the guard is present).
    np.testing.assert_allclose(1.0 - r["weights"][:, 0], 1e-9 / (p + 1e-9), rtol=1e-6)


def test_no_norm_returns_raw_probabilities():
    lay = _rand_layer(7, 32, 8, 8, 6)
    r = _run(lay, K=2, norm=False)
    np.testing.assert_array_equal(r["weights"], np.take_along_axis(r["probs"], r["sel"], 1))
    np.testing.assert_allclose(r["probs"].sum(1), 1.0, rtol=0, atol=1e-14)


def test_k_equals_e_is_dense_mixture():
    T, D, F, E = 12, 10, 7, 5
    lay = _rand_layer(8, T, D, F, E, router_bias=True)
    r = _run(lay, K=E)
    ys = []
    for e in range(E):
        one = dict(lay, router=lay["router"][e:e + 1], gate_up=lay["gate_up"][e:e + 1],
                   down=lay["down"][e:e + 1], router_bias=None)
        ys.append(_run(one, K=1)["out"] * (1.0 + 1e-9))       # expert e alone, guard undone
    mix = sum(r["probs"][:, e:e + 1] * ys[e] for e in range(E)) / (1.0 + 1e-9)
    np.testing.assert_allclose(r["out"], mix, rtol=1e-9, atol=1e-12)


def test_token_permutation_equivariance():
    lay = _rand_layer(9, 20, 8, 6, 6)
    r = _run(lay, K=2)
    perm = np.random.default_rng(0).permutation(20)
    r2 = _run(dict(lay, x=lay["x"][perm]), K=2)
    np.testing.assert_array_equal(r2["sel"], r["sel"][perm])
    np.testing.assert_array_equal(r2["out"], r["out"][perm])


def test_unselected_expert_never_enters():
    lay = _rand_layer(10, 24, 8, 6, 6)
    r = _run(lay, K=2)
    unused = sorted(set(range(6)) - set(r["sel"].ravel().tolist()))
    if not unused:  # force one: a router bias that keeps expert 5 out of every top-2
        lay["router_bias"] = np.array([0, 0, 0, 0, 0, -100], np.float32)
        r = _run(lay, K=2)
        unused = [5]
    assert 5 not in r["sel"] or unused != [5]
    bad = dict(lay, gate_up=lay["gate_up"].copy(), down=lay["down"].copy())
    for e in unused:
        bad["gate_up"][e] = np.nan
        bad["down"][e] = np.nan
    r2 = _run(bad, K=2)
    np.testing.assert_array_equal(r2["out"], r["out"])


def test_gate_up_halves():
    """Gate is rows [0,F) of gate_up_proj, up is rows [F,2F): the output is
    linear in up (doubling up doubles it exactly) but not in the gate."""
    T, D, F, E = 16, 8, 6, 4
    lay = _rand_layer(12, T, D, F, E)
    r = _run(lay, K=2)
    up2 = dict(lay, gate_up=lay["gate_up"].copy())
    up2["gate_up"][:, F:] *= 2
    np.testing.assert_array_equal(_run(up2, K=2)["out"], 2 * r["out"])
    g2 = dict(lay, gate_up=lay["gate_up"].copy())
    g2["gate_up"][:, :F] *= 2
    assert not np.allclose(_run(g2, K=2)["out"], 2 * r["out"], rtol=1e-3)


def test_decision_is_taken_in_float32():
    """Two probabilities that differ in fp64 but round to the same float32 tie,
    and the tie goes to the lower index."""
    lay = dict(x=np.ones((1, 1), np.float32), router=np.array([[0.0], [1e-12], [-5.0]], np.float32),
               gate_up=np.ones((3, 2, 1), np.float32), down=np.ones((3, 1, 1), np.float32),
               router_bias=None, up_bias=None, down_bias=None)
    r = _run(lay, K=1)
    assert r["probs"][0, 1] > r["probs"][0, 0]
    assert np.float32(r["probs"][0, 1]) == np.float32(r["probs"][0, 0])
    assert r["sel"][0, 0] == 0


def test_bf16_inputs_widen_exactly():
    lay = _rand_layer(13, 9, 8, 6, 4, router_bias=True)
    b = {k: (workloads.f32_to_bf16_bits(v) if k in ("x", "router", "gate_up", "down") else v)
         for k, v in lay.items()}
    f = {k: (workloads.bf16_bits_to_f32(v) if k in ("x", "router", "gate_up", "down") else v)
         for k, v in b.items()}
    rb, rf = _run(b, K=2), _run(f, K=2)
    np.testing.assert_array_equal(rb["out"], rf["out"])
    np.testing.assert_array_equal(rb["sel"], rf["sel"])


def test_replay_forced_selection():
    """Dew's routing replay: recorded experts replace the top-k, the weights
    still come from this forward's probabilities."""
    lay = _rand_layer(14, 10, 8, 6, 5)
    r = _run(lay, K=2)
    same = _run(lay, K=2, forced_sel=r["sel"])
    np.testing.assert_array_equal(same["out"], r["out"])
    forced = np.tile(np.array([[4, 3]]), (10, 1))
    f = _run(lay, K=2, forced_sel=forced)
    p = np.take_along_axis(f["probs"], forced, 1)
    np.testing.assert_allclose(f["weights"], p / (p.sum(1, keepdims=True) + 1e-9), rtol=1e-15)
    np.testing.assert_array_equal(f["sel"], forced)


def test_token_subset_matches_full():
    lay = _rand_layer(15, 30, 8, 6, 5)
    r = _run(lay, K=2)
    sub = np.array([29, 0, 7, 7, 13])
    s = _run(lay, K=2, tokens=sub)
    np.testing.assert_array_equal(s["out"], r["out"][sub])
    np.testing.assert_array_equal(s["sel"], r["sel"][sub])


def test_invalid_arguments_rejected():
    lay = _rand_layer(16, 4, 4, 4, 3)
    with pytest.raises(ValueError):
        _run(lay, K=0)
    with pytest.raises(ValueError):
        _run(lay, K=4)
    with pytest.raises(ValueError):
        _run(lay, K=1, tokens=np.array([4]))


def test_workload_recipe_is_reproducible():
    a = workloads.generate("tiny")
    b = workloads.generate("tiny")
    assert workloads.input_sha256(a) == workloads.input_sha256(b)
    # The MoEBlock page's example input for the tiny block.
    x = np.random.default_rng(0).random((4, 16, 64), dtype=np.float32)
    np.testing.assert_array_equal(a["x"], x.reshape(64, 64))
    # decode x is the first 64 tokens of the prefill x.
    d = workloads.generate("decode", with_weights=False)["x"]
    p = workloads.generate("prefill", T=128, with_weights=False)["x"]
    np.testing.assert_array_equal(d, p[:64])


def test_fine_zero_experts_get_no_tokens():
    """The skewed 128-expert workload with 8 experts pushed away: a sample of
    its tokens never selects them (router only: E=128, K=8)."""
    inp = workloads.generate("fine", T=256, with_weights=False)
    zb = workloads.zipf_rank_bias(128)
    assert np.all(np.diff(zb) < 0)
    z = workloads.zero_load_experts(128)
    assert len(set(z.tolist())) == 8
    assert inp["x"].dtype == np.uint16


def test_oracle_cache_returns_the_same_reference(tmp_path, monkeypatch):
    """The parity helpers' oracle cache (keyed by the inputs' sha256 manifest
    and the tokens) returns what a fresh oracle call returns, from memory and
    from its disk copy, and a different input gets a different entry."""
    import parity
    monkeypatch.setenv("MOE_ORACLE_CACHE_DIR", str(tmp_path))
    inp = workloads.generate(workloads.small_config(40, 16, 24, 4, 2, cfg_id=990))
    tok = np.arange(0, 40, 3)
    fresh = oracle.forward_inputs(inp, tokens=tok)
    a = parity.oracle_reference(inp, tok)
    assert len(list(tmp_path.glob("oracle_*.npz"))) == 1
    parity._ORACLE_CACHE.clear()
    b = parity.oracle_reference(dict(inp), tok)  # from disk
    for k in ("out", "sel", "weights", "logits", "probs"):
        np.testing.assert_array_equal(a[k], fresh[k])
        np.testing.assert_array_equal(b[k], fresh[k])
    other = dict(inp, x=inp["x"] + np.float32(1.0))
    c = parity.oracle_reference(other, tok)
    assert not np.array_equal(c["out"], a["out"])
    assert len(list(tmp_path.glob("oracle_*.npz"))) == 2
