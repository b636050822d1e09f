"""Pins for the oracle: checks against facts fixed outside the oracle itself.

Each pin checks the oracle against something it cannot agree with by
construction: values derived by hand (tests/golden/), exact rational
arithmetic with a rounding-error bound, closed forms, special cases that
reduce to a textbook routine (scipy's softmax and expit), brute force over
all k-subsets, and invariants of the definition (relabelling, batch
independence, power-of-two scaling, identical experts, k = 1).

The layer follows "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and
Responsibly" (Part 1, sections 1-3); the post prints no worked example, so no
pin comes from printed values.

test_planted_mistakes_are_caught builds mutated copies of the oracle's C
source (a dropped term, a wrong sign or index, swapped operands) and checks
that every mutant fails at least one pin.
"""
import itertools
import json
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(a):
    return torch.tensor(np.asarray(a, dtype=np.float32), dtype=torch.bfloat16)


def rand_bf(rng, shape, std=1.0):
    return bf(rng.standard_normal(shape) * std)


def tiny_layer(rng, d=16, E=6, I=4, Is=4, dlat=16, bias=False):
    w = {
        "w_router": rand_bf(rng, (E, d), 1 / math.sqrt(d)),
        "bias": torch.tensor(rng.standard_normal(E), dtype=torch.float32) if bias else None,
        "w_lat": rand_bf(rng, (dlat, d), 1 / math.sqrt(d)),
        "w13": rand_bf(rng, (E, 2 * I, dlat), 1 / math.sqrt(dlat)),
        "w2": rand_bf(rng, (E, d, I), 1 / math.sqrt(I)),
        "w13_s": rand_bf(rng, (2 * Is, d), 1 / math.sqrt(d)),
        "w2_s": rand_bf(rng, (d, Is), 1 / math.sqrt(Is)),
    }
    return w


def _eval(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "sqrt": math.sqrt})


# ------------------------------------------------------------------ pins
def pin_golden_moe():
    """Hand-derived tiny MoE block (tests/golden/hand_moe_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_moe_example.json")))
    w = {key: bf(g[key]) for key in ("w_router", "w_lat", "w13", "w2", "w13_s", "w2_s")}
    w["bias"] = None
    out = oracle.moe_block(bf(g["x"]), w, g["config"]["k"])
    ex = g["expect"]
    assert out["ids"].tolist() == ex["ids"]
    for key in ("logits", "w", "z", "y_s", "y_r", "y"):
        want = np.array([[_eval(v) for v in row] for row in ex[key]])
        np.testing.assert_allclose(out[key], want, rtol=1e-12, atol=1e-12, err_msg=key)


def pin_golden_chain():
    """Hand-derived projection chain (tests/golden/hand_chain_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_chain_example.json")))
    out = oracle.chain(bf(g["x"]), bf(g["r"]), bf(g["w_in"]), bf(g["w_o"]), bf(g["gamma"]),
                       g["eps"])
    for key in ("q", "h", "y"):
        want = np.array([[_eval(v) for v in row] for row in g["expect"][key]])
        np.testing.assert_allclose(out[key], want, rtol=1e-14, atol=0, err_msg=key)


def pin_linear_exact_rational():
    """|oracle - exact| <= gamma_K * sum|x_i w_i| (Higham's bound, u = 2^-53),
    exact sums in rationals; non-square W so a transposed operand fails."""
    rng = np.random.default_rng(1)
    b, K, N = 3, 37, 5
    x = rng.standard_normal((b, K))
    W = rand_bf(rng, (N, K))
    y = oracle.linear(x, W)
    Wf = W.float().numpy().astype(np.float64)
    u = 2.0 ** -53
    gam = K * u / (1 - K * u)
    for t in range(b):
        for n in range(N):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(Wf[n, i])) for i in range(K))
            bound = gam * sum(abs(x[t, i] * Wf[n, i]) for i in range(K))
            assert abs(Fraction(float(y[t, n])) - exact) <= Fraction(bound) + Fraction(1, 10**300)


def pin_power_of_two_scaling():
    """Scaling the input by 2^m scales linear maps and router logits exactly."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 24))
    W = rand_bf(rng, (7, 24))
    np.testing.assert_array_equal(oracle.linear(8.0 * x, W), 8.0 * oracle.linear(x, W))
    np.testing.assert_array_equal(oracle.router_logits(0.25 * x, W),
                                  np.float32(0.25) * oracle.router_logits(x, W))


def pin_topk_bruteforce_subsets():
    """The selected set maximises the logit sum over all k-subsets (distinct
    logits), in descending order; w_j = 1 / sum_{i in S} exp(l_i - l_j)."""
    rng = np.random.default_rng(3)
    E, k = 7, 3
    logits = rng.standard_normal((5, E)).astype(np.float32)
    ids, w = oracle.topk_softmax(logits, k)
    for t in range(logits.shape[0]):
        l = logits[t].astype(np.float64)
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(l[list(S)]))
        assert sorted(ids[t].tolist()) == sorted(best)
        assert all(l[ids[t][j]] > l[ids[t][j + 1]] for j in range(k - 1))
        for j in range(k):
            want = 1.0 / sum(math.exp(l[i] - l[ids[t][j]]) for i in ids[t])
            assert abs(w[t, j] - want) < 1e-14


def pin_topk_full_is_softmax():
    """With k = E the weights are the textbook softmax and sum to 1."""
    rng = np.random.default_rng(4)
    logits = (3 * rng.standard_normal((4, 9))).astype(np.float32)
    ids, w = oracle.topk_softmax(logits, 9)
    for t in range(4):
        ref = scipy.special.softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(w[t], ref[ids[t]], rtol=1e-13)
        assert abs(w[t].sum() - 1.0) < 1e-14
    ids2, w2 = oracle.topk_softmax(logits, 4)
    np.testing.assert_allclose(w2.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def pin_topk_ties_lower_index():
    """Equal logits: the lower expert index wins; all-equal gives ids 0..k-1, w = 1/k."""
    ids, w = oracle.topk_softmax(np.zeros((1, 8), np.float32), 3)
    assert ids.tolist() == [[0, 1, 2]]
    np.testing.assert_allclose(w, 1 / 3, rtol=1e-15)
    ids, w = oracle.topk_softmax(np.array([[1, 3, 3, 0, 3]], np.float32), 2)
    assert ids.tolist() == [[1, 2]]
    np.testing.assert_allclose(w, 0.5, rtol=1e-15)


def pin_router_bias():
    """The bias is added to the fp32 logits and moves the selection."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 16))
    W = rand_bf(rng, (6, 16), 0.25)
    bias = np.array([0, 0, 0, 50, 0, -50], np.float32)
    l0 = oracle.router_logits(x, W)
    l1 = oracle.router_logits(x, W, bias)
    np.testing.assert_array_equal(l1, l0 + bias)
    ids, _ = oracle.topk_softmax(l1, 1)
    assert (ids[:, 0] == 3).all()


def pin_swiglu_closed_forms():
    """One-hot input and one-hot down rows expose h_j = silu(g_j) * u_j, with
    silu from scipy's expit: silu(g) = g * expit(g); silu(0) = 0; silu(g) ~ g
    for large g."""
    I, din = 4, 3
    gate = [0.0, 1.0, -2.0, 30.0]
    up = [5.0, 0.5, 3.0, 1.0]
    W13 = np.zeros((2 * I, din), np.float32)
    W13[:I, 0] = gate
    W13[I:, 0] = up
    W2 = np.eye(I, dtype=np.float32)  # dout = I, out = h
    y = oracle.shared_expert(np.array([[1.0, 0.0, 0.0]]), bf(W13), bf(W2))
    want = [g * scipy.special.expit(g) * u for g, u in zip(gate, up)]
    np.testing.assert_allclose(y[0], want, rtol=1e-14, atol=0)
    assert y[0, 0] == 0.0
    assert abs(y[0, 3] - 30.0) < 1e-11


def pin_identical_experts():
    """All routed experts equal: y_r = Expert(z) for any routing (sum w = 1);
    the shared expert equal to them too gives y = Expert(z) + Expert(x)."""
    rng = np.random.default_rng(6)
    w = tiny_layer(rng)
    E = w["w13"].shape[0]
    w["w13"] = w["w13"][:1].repeat(E, 1, 1)
    w["w2"] = w["w2"][:1].repeat(E, 1, 1)
    w["w13_s"] = w["w13"][0].clone()
    w["w2_s"] = w["w2"][0].clone()
    x = rand_bf(rng, (4, 16))
    out = oracle.moe_block(x, w, 3)
    one = oracle.shared_expert(out["z"], w["w13"][0], w["w2"][0])
    np.testing.assert_allclose(out["y_r"], one, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["y"], one + oracle.shared_expert(x, w["w13"][0], w["w2"][0]),
                               rtol=1e-12, atol=1e-14)


def pin_k1_argmax():
    """k = 1: w = 1 and y_r = Expert_argmax(z)."""
    rng = np.random.default_rng(7)
    w = tiny_layer(rng)
    x = rand_bf(rng, (3, 16))
    out = oracle.moe_block(x, w, 1)
    assert (out["w"] == 1.0).all()
    assert (out["ids"][:, 0] == np.argmax(out["logits"], axis=1)).all()
    for t in range(3):
        e = int(out["ids"][t, 0])
        one = oracle.shared_expert(out["z"][t:t + 1], w["w13"][e], w["w2"][e])
        np.testing.assert_allclose(out["y_r"][t], one[0], rtol=1e-13, atol=1e-15)


def pin_relabel_experts():
    """Permuting the experts (router rows, bias, w13, w2 together) permutes the
    ids and leaves the logits bit for bit and the outputs up to the rounding
    of the softmax normaliser (its sum runs in expert order)."""
    rng = np.random.default_rng(8)
    w = tiny_layer(rng, bias=True)
    x = rand_bf(rng, (5, 16))
    out = oracle.moe_block(x, w, 3)
    perm = rng.permutation(6)
    inv = np.argsort(perm)
    wp = dict(w)
    for key in ("w_router", "w13", "w2"):
        wp[key] = w[key][torch.as_tensor(perm)]
    wp["bias"] = w["bias"][torch.as_tensor(perm)]
    outp = oracle.moe_block(x, wp, 3)
    np.testing.assert_array_equal(perm[outp["ids"]], out["ids"])
    assert (inv[out["ids"]] == outp["ids"]).all()
    np.testing.assert_array_equal(outp["logits"][:, inv], out["logits"])
    np.testing.assert_allclose(outp["y"], out["y"], rtol=1e-13, atol=1e-15)


def pin_batch_independence():
    """Token t's outputs at batch b equal its batch-1 outputs bit for bit."""
    rng = np.random.default_rng(9)
    w = tiny_layer(rng, bias=True)
    x = rand_bf(rng, (4, 16))
    out = oracle.moe_block(x, w, 2)
    for t in range(4):
        one = oracle.moe_block(x[t:t + 1], w, 2)
        for key in ("logits", "ids", "w", "z", "y_s", "y"):
            np.testing.assert_array_equal(one[key][0], out[key][t], err_msg=key)


def pin_latent_identity():
    """W_lat = I gives z = x exactly; the shared expert reads x, not z."""
    rng = np.random.default_rng(10)
    w = tiny_layer(rng)
    w["w_lat"] = bf(np.eye(16))
    x = rand_bf(rng, (2, 16))
    out = oracle.moe_block(x, w, 2)
    np.testing.assert_array_equal(out["z"], x.double().numpy())
    w["w_lat"] = bf(2 * np.eye(16))
    out2 = oracle.moe_block(x, w, 2)
    np.testing.assert_array_equal(out2["y_s"], oracle.shared_expert(x, w["w13_s"], w["w2_s"]))


def pin_moe_bruteforce_dense():
    """Brute force: every expert on every token (numpy fp64 matmuls), the
    selection from all k-subsets, combined by a dense masked sum."""
    rng = np.random.default_rng(11)
    w = tiny_layer(rng, bias=True)
    x = rand_bf(rng, (3, 16))
    k = 3
    out = oracle.moe_block(x, w, k)
    X = x.double().numpy()
    f = {key: (v.double().numpy() if v is not None and v.dtype == torch.bfloat16 else v)
         for key, v in w.items()}
    logits = np.float32(X @ f["w_router"].T) + w["bias"].numpy()
    np.testing.assert_allclose(out["logits"], logits, rtol=2e-7, atol=1e-7)
    Z = X @ f["w_lat"].T
    np.testing.assert_allclose(out["z"], Z, rtol=1e-12, atol=1e-13)
    E, I = 6, 4

    def expert(v, w13, w2):
        g, u = w13[:I] @ v, w13[I:] @ v
        return w2 @ (g * scipy.special.expit(g) * u)

    for t in range(3):
        l = logits[t].astype(np.float64)
        S = max(itertools.combinations(range(E), k), key=lambda s: sum(l[list(s)]))
        c = np.zeros(E)
        for e in S:
            c[e] = 1.0 / sum(math.exp(l[i] - l[e]) for i in S)
        y_r = sum(c[e] * expert(Z[t], f["w13"][e], f["w2"][e]) for e in range(E))
        y_s = expert(X[t], f["w13_s"], f["w2_s"])
        np.testing.assert_allclose(out["y"][t], y_s + y_r, rtol=1e-11, atol=1e-13)


def pin_moe_experts_y_add():
    """The routed call adds y_add before the weighted expert outputs."""
    rng = np.random.default_rng(12)
    w = tiny_layer(rng)
    z = rng.standard_normal((2, 16))
    ids = np.array([[1, 4], [0, 5]], np.int32)
    wt = np.array([[0.75, 0.25], [0.5, 0.5]])
    fn = lambda e: (w["w13"][e], w["w2"][e])  # noqa: E731
    base = oracle.moe_experts(z, ids, wt, fn, 6)
    ya = rng.standard_normal(base.shape)
    np.testing.assert_allclose(oracle.moe_experts(z, ids, wt, fn, 6, y_add=ya), base + ya,
                               rtol=1e-13, atol=1e-13)
    one = [oracle.shared_expert(z[t:t + 1], w["w13"][e], w["w2"][e])[0]
           for t, e in ((0, 1), (0, 4))]
    np.testing.assert_allclose(base[0], 0.75 * one[0] + 0.25 * one[1], rtol=1e-13, atol=1e-14)


def pin_oproj_zero_weights():
    """W_o = 0 gives h = r exactly; with gamma = 1, mean(y^2) = ms/(ms + eps)."""
    rng = np.random.default_rng(13)
    r = rand_bf(rng, (3, 10))
    a = rng.standard_normal((3, 6))
    h, y = oracle.oproj_residual_rmsnorm(a, bf(np.zeros((10, 6))), r, bf(np.ones(10)), 1e-6)
    np.testing.assert_array_equal(h, r.double().numpy())
    ms = (h ** 2).mean(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), ms / (ms + 1e-6), rtol=1e-13)


def pin_rmsnorm_eps_inside():
    """With mean(h^2) near eps the eps position shows: mean(y^2) = ms/(ms + eps)
    holds only with eps inside the square root; the mean runs over the width."""
    h0 = np.array([[1e-3, -2e-3, 0.5e-3, 1e-3]])
    r = bf(h0)
    _, y = oracle.oproj_residual_rmsnorm(np.zeros((1, 2)), bf(np.zeros((4, 2))), r,
                                         bf(np.ones(4)), 1e-6)
    hf = r.double().numpy()
    ms = (hf ** 2).sum() / 4
    np.testing.assert_allclose((y ** 2).mean(), ms / (ms + 1e-6), rtol=1e-12)
    _, y2 = oracle.oproj_residual_rmsnorm(np.zeros((1, 2)), bf(np.zeros((4, 2))), r,
                                          bf([1.0, 2.0, 0.5, -1.0]), 1e-6)
    np.testing.assert_allclose(y2[0], y[0] * np.array([1.0, 2.0, 0.5, -1.0]), rtol=1e-15)


def pin_oproj_residual_linear():
    """h - r is linear in a (doubling a doubles it exactly); h reads a's first
    K columns only when a is a slice of a wider q (chain)."""
    rng = np.random.default_rng(14)
    a = rng.standard_normal((2, 6))
    Wo = rand_bf(rng, (5, 6))
    r = rand_bf(rng, (2, 5))
    g = bf(np.ones(5))
    h1, _ = oracle.oproj_residual_rmsnorm(a, Wo, r, g, 1e-6)
    h0, _ = oracle.oproj_residual_rmsnorm(np.zeros_like(a), Wo, r, g, 1e-6)
    np.testing.assert_array_equal(h0, r.double().numpy())
    np.testing.assert_allclose(h1 - h0, a @ Wo.double().numpy().T, rtol=1e-12, atol=1e-14)


PINS = [pin_golden_moe, pin_golden_chain, pin_linear_exact_rational, pin_power_of_two_scaling,
        pin_topk_bruteforce_subsets, pin_topk_full_is_softmax, pin_topk_ties_lower_index,
        pin_router_bias, pin_swiglu_closed_forms, pin_identical_experts, pin_k1_argmax,
        pin_relabel_experts, pin_batch_independence, pin_latent_identity,
        pin_moe_bruteforce_dense, pin_moe_experts_y_add, pin_oproj_zero_weights,
        pin_rmsnorm_eps_inside, pin_oproj_residual_linear]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(oracle_lib, pin):
    pin()


# Plausible mistakes, planted in a copy of the oracle's C source. Each must
# make at least one pin fail. Every mutant stays memory-safe.
MUTATIONS = {
    "swap_gate_up": ("h[j] = silu(g) * u;", "h[j] = silu(u) * g;"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "drop_bias": ("l = l + bias[e];", "l = l + 0.0f * bias[e];"),
    "tie_upper_index": ("return a < b;", "return a > b;"),
    "sort_ascending": ("ranks_before(l, e, order[j - 1])", "ranks_before(l, order[j - 1], e)"),
    "no_renormalise": ("w[(int64_t)t * k + j] = p[order[j]] / sel;",
                       "w[(int64_t)t * k + j] = p[order[j]];"),
    "softmax_sign": ("p[e] = exp((double)l[e] - m);", "p[e] = exp(m - (double)l[e]);"),
    "linear_reversed_index": ("s += xt[i] * bf16_value(wn[i]);",
                              "s += xt[i] * bf16_value(wn[K - 1 - i]);"),
    "down_wrong_index": ("s += bf16_value(wr[j]) * h[j];", "s += bf16_value(wr[j]) * h[I - 1 - j];"),
    "up_rows_offset": ("W13 + (int64_t)(I + j) * din;", "W13 + (int64_t)j * din;"),
    "drop_combine_weight": ("yt[r] += wj * o[r];", "yt[r] += o[r];"),
    "drop_y_add": ("yt[r] = y_add ? y_add[(int64_t)t * dout + r] : 0.0;", "yt[r] = 0.0;"),
    "drop_residual": ("ht[n] += rt[n];", "ht[n] += 0.0 * rt[n];"),
    "eps_outside_sqrt": ("double inv = 1.0 / sqrt(ss / d + eps);",
                         "double inv = 1.0 / (sqrt(ss / d) + eps);"),
    "mean_wrong_width": ("double inv = 1.0 / sqrt(ss / d + eps);",
                         "double inv = 1.0 / sqrt(ss / (d + 1) + eps);"),
    "norm_no_gamma": ("y[(int64_t)t * d + n] = ht[n] * inv * gamma[n];",
                      "y[(int64_t)t * d + n] = ht[n] * inv;"),
    "logit_rounding_dropped_sum_term": ("for (int i = 0; i < d; ++i)\n            s += xt[i] * bf16_value(we[i]);",
                                        "for (int i = 1; i < d; ++i)\n            s += xt[i] * bf16_value(we[i]);"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="k3orc_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_lib, mutant_dir, name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "k3_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path_c = os.path.join(mutant_dir, f"{name}.c")
    path_so = os.path.join(mutant_dir, f"{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o",
                           path_so, path_c, "-lm"])
    failed = []
    with oracle.use_library(path_so):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
