"""Pins of the CPU oracle against values and facts fixed outside it.

Each test ties one oracle function to something other than the oracle: a value
a page prints (fixtures under tests/golden/, each naming its source), a case
worked by hand here, a closed form, an invariant of the rule, or a library
routine (torch, float64) that computes the same step by another route.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAPS = {"grouped": oracle.MAP_GROUPED, "tiled": oracle.MAP_TILED}


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_unit_rows(rng, shape):
    x = rng.normal(size=shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- printed values

def test_scalar_recurrence_printed_case():
    gd = golden("scalar_recurrence.json")
    i = gd["inputs"]
    o, S = oracle.recurrence(np.array(i["q"]).reshape(1, 1, 1), np.array(i["k"]).reshape(1, 1, 1),
                             np.array(i["v"]).reshape(1, 1, 1), np.array(i["g"]).reshape(1, 1),
                             np.array(i["beta"]).reshape(1, 1), np.array(i["S0"]).reshape(1, 1, 1),
                             MAPS[i["head_map"]])
    tol = gd["tolerance_abs"]
    assert abs(S.ravel()[0] - gd["expected"]["S"][0]) <= tol
    assert abs(o.ravel()[0] - gd["expected"]["o"][0]) <= tol


def test_head_maps_printed_case():
    gd = golden("head_maps.json")
    for c in gd["k_head"]:
        assert oracle.k_head(MAPS[c["map"]], c["h"], c["Hk"], c["Hv"]) == c["expected"]
    i = gd["step"]["inputs"]
    for name, expected in gd["step"]["expected_o"].items():
        o, _ = oracle.recurrence(np.array(i["q"]).reshape(1, 2, 1), np.array(i["k"]).reshape(1, 2, 1),
                                 np.array(i["v"]).reshape(1, 4, 1), np.array(i["g"]).reshape(1, 4),
                                 np.array(i["beta"]).reshape(1, 4), np.array(i["S0"]).reshape(4, 1, 1),
                                 MAPS[name])
        assert o.ravel().tolist() == expected


def test_l2_normalize_printed_cases():
    gd = golden("l2_normalize.json")
    for c in gd["cases"]:
        y = oracle.l2norm(np.array(c["x"]), c["eps"])
        assert np.max(np.abs(y - np.array(c["expected"]))) <= c["tolerance_abs"]


def test_l2_normalize_eps_inside_root():
    # Reading: eps is added to the sum of squares under the root, so a tiny
    # vector is not blown up to unit length (closed form of that reading).
    y = oracle.l2norm(np.array([1e-4, 0.0]), 1e-6)
    assert y[0] == pytest.approx(1e-4 / math.sqrt(1e-8 + 1e-6), rel=1e-14)
    assert y[1] == 0.0


# ---------------------------------------------------------------- hand-worked cases

def test_d4_two_token_worked_example():
    """Hk = Hv = 1, d = 4, scale = 1/sqrt(4) = 1/2, every number dyadic.

    Token 1: S0 = I, k = (1/2,1/2,1/2,1/2), q = e0, v = (1,2,3,4), alpha = 1/2, beta = 1/2.
      decay: S = I/2;  prediction p_j = S_j . k = 1/4 for every row
      d = beta (v - p) = (3/8, 7/8, 11/8, 15/8)
      S1 = I/2 + d k^T  -> row j is d_j/2 everywhere plus 1/2 on the diagonal
      o1 = scale * S1 q = (column 0 of S1)/2 = (11/32, 7/32, 11/32, 15/32)
    Token 2: k = e0, q = e3, v = 0, alpha = 1, beta = 1.
      p_j = S1[j][0];  d_j = -S1[j][0];  S2 = S1 with column 0 zeroed
      o2 = (column 3 of S2)/2 = (3/32, 7/32, 11/32, 23/32)
    S1 is not symmetric and token 2 reads one column and writes another, so a
    transposed state, a swapped q/k, a missing decay or a flipped sign all fail.
    """
    q = np.array([[1, 0, 0, 0], [0, 0, 0, 1]], dtype=float).reshape(2, 1, 4)
    k = np.array([[.5, .5, .5, .5], [1, 0, 0, 0]], dtype=float).reshape(2, 1, 4)
    v = np.array([[1, 2, 3, 4], [0, 0, 0, 0]], dtype=float).reshape(2, 1, 4)
    g = np.array([[math.log(0.5)], [0.0]])
    beta = np.array([[0.5], [1.0]])
    S0 = np.eye(4).reshape(1, 4, 4)
    o, S = oracle.recurrence(q, k, v, g, beta, S0, oracle.MAP_GROUPED)
    S1_rows = [[0.6875, 0.1875, 0.1875, 0.1875], [0.4375, 0.9375, 0.4375, 0.4375],
               [0.6875, 0.6875, 1.1875, 0.6875], [0.9375, 0.9375, 0.9375, 1.4375]]
    S2 = np.array(S1_rows)
    S2[:, 0] = 0.0
    np.testing.assert_allclose(o[0, 0], [11 / 32, 7 / 32, 11 / 32, 15 / 32], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[1, 0], [3 / 32, 7 / 32, 11 / 32, 23 / 32], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0], S2, rtol=0, atol=1e-15)
    # one token at a time gives the same (the carried state is the only link)
    o1, Sa = oracle.recurrence(q[:1], k[:1], v[:1], g[:1], beta[:1], S0, oracle.MAP_GROUPED)
    np.testing.assert_allclose(Sa[0], np.array(S1_rows), rtol=0, atol=1e-15)
    o2, Sb = oracle.recurrence(q[1:], k[1:], v[1:], g[1:], beta[1:], Sa, oracle.MAP_GROUPED)
    assert np.array_equal(o2[0], o[1]) and np.array_equal(Sb, S)


def test_conv_hand_case():
    # w = (1/4, 1/2, -1/2, 1), carried window (1, 2, 3), new input 4:
    # pre = 1/4 + 1 - 3/2 + 4 = 15/4, y = pre * sigmoid(pre), new window (2, 3, 4).
    y, st = oracle.conv(np.array([[4.0]]), np.array([[0.25, 0.5, -0.5, 1.0]]),
                        np.array([[1.0, 2.0, 3.0]]))
    pre = 3.75
    assert y[0, 0] == pytest.approx(pre / (1.0 + math.exp(-pre)), rel=1e-15)
    assert y[0, 0] == pytest.approx(3.663834862837404, rel=1e-14)
    assert st.ravel().tolist() == [2.0, 3.0, 4.0]


# ---------------------------------------------------------------- exact rational brute force

def _exact_recurrence(q, k, v, alpha, beta, S0, scale):
    """Exact rational arithmetic, tiny d: the rule with Fractions."""
    T, d = len(q), len(S0)
    S = [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        o = []
        for j in range(d):
            S[j] = [alpha[t] * x for x in S[j]]
            p = sum(S[j][i] * k[t][i] for i in range(d))
            dd = beta[t] * (v[t][j] - p)
            S[j] = [S[j][i] + dd * k[t][i] for i in range(d)]
            o.append(scale * sum(S[j][i] * q[t][i] for i in range(d)))
        outs.append(o)
    return outs, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_dyadic(seed):
    rng = np.random.default_rng(seed)
    d, T = 4, 3

    def dy(n):  # dyadic values k/8 in [-2, 2]
        return [Fraction(int(x), 8) for x in rng.integers(-16, 17, n)]

    q = [dy(d) for _ in range(T)]
    k = [dy(d) for _ in range(T)]
    v = [dy(d) for _ in range(T)]
    S0 = [dy(d) for _ in range(d)]
    alpha = [Fraction(1, 2 ** int(e)) for e in rng.integers(0, 3, T)]
    beta = [Fraction(int(x), 4) for x in rng.integers(0, 5, T)]
    o_ex, S_ex = _exact_recurrence(q, k, v, alpha, beta, S0, Fraction(1, 2))
    f = lambda a: np.array([[float(x) for x in r] for r in a])  # noqa: E731
    g = np.array([[math.log(float(a))] for a in alpha])
    o, S = oracle.recurrence(f(q).reshape(T, 1, d), f(k).reshape(T, 1, d), f(v).reshape(T, 1, d),
                             g, np.array([[float(b)] for b in beta]), f(S0).reshape(1, d, d),
                             oracle.MAP_TILED)
    # exp(log(2^-e)) may be off by one ulp; everything else is exact in binary
    np.testing.assert_allclose(o[:, 0, :], f(o_ex), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S[0], f(S_ex), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- invariants of the rule

@pytest.mark.parametrize("head_map", [oracle.MAP_GROUPED, oracle.MAP_TILED])
def test_unit_k_no_decay_full_beta_stores_v(head_map):
    # g = 0, beta = 1, |k| = 1  =>  S_new k = v exactly (up to rounding)
    rng = np.random.default_rng(3)
    Hk, Hv, d = 2, 4, 16
    k = rand_unit_rows(rng, (1, Hk, d))
    q = rng.normal(size=(1, Hk, d))
    v = rng.normal(size=(1, Hv, d))
    S0 = rng.normal(size=(Hv, d, d))
    _, S = oracle.recurrence(q, k, v, np.zeros((1, Hv)), np.ones((1, Hv)), S0, head_map)
    for h in range(Hv):
        kh = oracle.k_head(head_map, h, Hk, Hv)
        np.testing.assert_allclose(S[h] @ k[0, kh], v[0, h], atol=1e-12)


def test_zero_beta_no_decay_keeps_state_and_reads_out_with_dk_scale():
    rng = np.random.default_rng(4)
    Hk, Hv, dk, dv = 1, 2, 8, 4  # dk != dv: the scale is 1/sqrt(dk)
    q = rng.normal(size=(1, Hk, dk))
    k = rng.normal(size=(1, Hk, dk))
    v = rng.normal(size=(1, Hv, dv))
    S0 = rng.normal(size=(Hv, dv, dk))
    o, S = oracle.recurrence(q, k, v, np.zeros((1, Hv)), np.zeros((1, Hv)), S0, oracle.MAP_GROUPED)
    assert np.array_equal(S, S0)
    for h in range(Hv):
        np.testing.assert_allclose(o[0, h], S0[h] @ q[0, 0] / math.sqrt(dk), rtol=1e-14, atol=1e-14)


def test_full_decay_leaves_rank_one_write():
    # alpha = exp(-800) = 0 in double: S_new = beta v k^T, o = beta v (k.q)/sqrt(dk)
    rng = np.random.default_rng(5)
    Hk, Hv, d = 1, 1, 8
    q, k = rng.normal(size=(1, Hk, d)), rng.normal(size=(1, Hk, d))
    v = rng.normal(size=(1, Hv, d))
    S0 = rng.normal(size=(Hv, d, d))
    o, S = oracle.recurrence(q, k, v, np.full((1, Hv), -800.0), np.full((1, Hv), 0.3), S0,
                             oracle.MAP_TILED)
    np.testing.assert_allclose(S[0], 0.3 * np.outer(v[0, 0], k[0, 0]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], 0.3 * v[0, 0] * (k[0, 0] @ q[0, 0]) / math.sqrt(d),
                               rtol=1e-13, atol=1e-15)


def test_zero_beta_closed_form_over_tokens():
    # beta = 0: S_t = (prod_{s<=t} alpha_s) S0, o_t = gamma_t S0 q_t / sqrt(dk)
    rng = np.random.default_rng(6)
    T, Hk, Hv, d = 7, 1, 2, 8
    q, k = rng.normal(size=(T, Hk, d)), rng.normal(size=(T, Hk, d))
    v = rng.normal(size=(T, Hv, d))
    g = -rng.uniform(0, 0.5, size=(T, Hv))
    S0 = rng.normal(size=(Hv, d, d))
    o, S = oracle.recurrence(q, k, v, g, np.zeros((T, Hv)), S0, oracle.MAP_GROUPED)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        for h in range(Hv):
            np.testing.assert_allclose(o[t, h], math.exp(G[t, h]) * S0[h] @ q[t, 0] / math.sqrt(d),
                                       rtol=1e-12, atol=1e-14)
    for h in range(Hv):
        np.testing.assert_allclose(S[h], math.exp(G[-1, h]) * S0[h], rtol=1e-12)


def test_orthonormal_keys_reduce_to_causal_linear_attention():
    # g = 0, beta = 1, S0 = 0, k_t = e_t: each token writes v_t into column t, so
    # o = scale * tril(Q K^T) V with K = I, the textbook causal linear attention.
    rng = np.random.default_rng(7)
    T, d = 6, 8
    q = rng.normal(size=(T, 1, d))
    k = np.eye(d)[:T].reshape(T, 1, d)
    v = rng.normal(size=(T, 1, d))
    o, S = oracle.recurrence(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), np.zeros((1, d, d)),
                             oracle.MAP_TILED)
    Q, K, V = (torch.from_numpy(x[:, 0]) for x in (q, k, v))
    ref = torch.tril(Q @ K.T) @ V / math.sqrt(d)
    np.testing.assert_allclose(o[:, 0], ref.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S[0], (V.T @ K).numpy(), atol=1e-15)


def test_value_rows_are_independent():
    rng = np.random.default_rng(8)
    T, Hk, Hv, d = 5, 2, 4, 8
    q, k = rng.normal(size=(T, Hk, d)), rng.normal(size=(T, Hk, d))
    v = rng.normal(size=(T, Hv, d))
    g, beta = -rng.uniform(0, 1, (T, Hv)), rng.uniform(0, 1, (T, Hv))
    S0 = rng.normal(size=(Hv, d, d))
    perm = rng.permutation(d)
    o, S = oracle.recurrence(q, k, v, g, beta, S0, oracle.MAP_TILED)
    op, Sp = oracle.recurrence(q, k, v[:, :, perm], g, beta, S0[:, perm, :], oracle.MAP_TILED)
    np.testing.assert_array_equal(op, o[:, :, perm])
    np.testing.assert_array_equal(Sp, S[:, perm, :])


def test_equal_head_counts_make_maps_identical():
    rng = np.random.default_rng(9)
    T, H, d = 4, 3, 8
    args = (rng.normal(size=(T, H, d)), rng.normal(size=(T, H, d)), rng.normal(size=(T, H, d)),
            -rng.uniform(0, 1, (T, H)), rng.uniform(0, 1, (T, H)), rng.normal(size=(H, d, d)))
    og, Sg = oracle.recurrence(*args, oracle.MAP_GROUPED)
    ot, St = oracle.recurrence(*args, oracle.MAP_TILED)
    assert np.array_equal(og, ot) and np.array_equal(Sg, St)


def test_head_subset_matches_full_run():
    rng = np.random.default_rng(10)
    T, Hk, Hv, d = 3, 2, 6, 8
    args = (rng.normal(size=(T, Hk, d)), rng.normal(size=(T, Hk, d)), rng.normal(size=(T, Hv, d)),
            -rng.uniform(0, 1, (T, Hv)), rng.uniform(0, 1, (T, Hv)), rng.normal(size=(Hv, d, d)))
    o, S = oracle.recurrence(*args, oracle.MAP_GROUPED)
    os_, Ss = oracle.recurrence(*args, oracle.MAP_GROUPED, heads=(2, 4))
    assert np.array_equal(os_[:, 2:4], o[:, 2:4]) and np.array_equal(Ss[2:4], S[2:4])
    assert np.all(os_[:, :2] == 0) and np.array_equal(Ss[:2], args[5][:2])


# ---------------------------------------------------------------- conv

def test_conv_matches_torch_conv1d():
    rng = np.random.default_rng(11)
    T, C, K = 5, 6, 4
    x, w, st = rng.normal(size=(T, C)), rng.normal(size=(C, K)), rng.normal(size=(C, K - 1))
    y, st2 = oracle.conv(x, w, st)
    seq = torch.cat([torch.from_numpy(st), torch.from_numpy(x).T], dim=1)  # [C][K-1+T]
    ref = F.silu(F.conv1d(seq.unsqueeze(0), torch.from_numpy(w).unsqueeze(1), groups=C))[0].T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st2, seq[:, -(K - 1):].numpy())


def test_conv_tap_special_cases():
    rng = np.random.default_rng(12)
    T, C = 5, 3
    x, st = rng.normal(size=(T, C)), rng.normal(size=(C, 3))
    y, _ = oracle.conv(x, np.tile([0.0, 0.0, 0.0, 1.0], (C, 1)), st)
    np.testing.assert_allclose(y, x / (1 + np.exp(-x)), rtol=1e-14)
    y, _ = oracle.conv(x, np.tile([1.0, 0.0, 0.0, 0.0], (C, 1)), st)
    xhat = np.concatenate([st.T, x], axis=0)  # [3 + T][C]
    np.testing.assert_allclose(y, xhat[:T] / (1 + np.exp(-xhat[:T])), rtol=1e-14)


def test_conv_one_call_equals_token_by_token():
    rng = np.random.default_rng(13)
    T, C = 6, 4
    x, w, st = rng.normal(size=(T, C)), rng.normal(size=(C, 4)), rng.normal(size=(C, 3))
    y, s_all = oracle.conv(x, w, st)
    s = st
    for t in range(T):
        yt, s = oracle.conv(x[t:t + 1], w, s)
        assert np.array_equal(yt[0], y[t])
    assert np.array_equal(s, s_all)
    # short segments keep part of the old window
    y1, s1 = oracle.conv(x[:1], w, st)
    assert s1.tolist() == np.concatenate([st[:, 1:], x[:1].T], axis=1).tolist()


# ---------------------------------------------------------------- gates and norms

def test_gates_against_torch_and_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert oracle.sigmoid(0.0) == 0.5
    xs = torch.linspace(-40, 40, 801, dtype=torch.float64)
    sp = torch.tensor([oracle.softplus(float(x)) for x in xs], dtype=torch.float64)
    hi = xs >= -20  # torch has no lower cut-over; below -20 the page's form is exp(x)
    np.testing.assert_allclose(sp[hi].numpy(), F.softplus(xs[hi], beta=1, threshold=20).numpy(),
                               rtol=1e-14)
    np.testing.assert_allclose(sp[~hi].numpy(), torch.exp(xs[~hi]).numpy(), rtol=1e-15)
    np.testing.assert_allclose(sp[~hi].numpy(), F.softplus(xs[~hi]).numpy(), rtol=1e-8)
    sg = torch.tensor([oracle.sigmoid(float(x)) for x in xs], dtype=torch.float64)
    np.testing.assert_allclose(sg.numpy(), torch.sigmoid(xs).numpy(), rtol=1e-14)
    # A_log = 0 and a + dt_bias = 0: g = -ln 2, so the decay exp(g) is one half
    g, beta = oracle.gates(np.array([[0.25, 0.0]]), np.array([[0.0, 3.0]]), np.array([0.0, 0.0]),
                           np.array([-0.25, 0.0]))
    assert g[0, 0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert math.exp(g[0, 0]) == pytest.approx(0.5, rel=1e-15)
    assert beta[0, 0] == 0.5 and beta[0, 1] == pytest.approx(1 / (1 + math.exp(-3.0)), rel=1e-15)


def test_negative_rate_decay_equals_log_rate():
    rng = np.random.default_rng(14)
    a, b = rng.normal(size=(3, 5)), rng.normal(size=(3, 5))
    A_log, dtb = rng.uniform(-2, 0, 5), rng.normal(size=5)
    g1, b1 = oracle.gates(a, b, A_log, dtb, oracle.DECAY_LOG_RATE)
    g2, b2 = oracle.gates(a, b, -np.exp(A_log), dtb, oracle.DECAY_NEGATIVE_RATE)
    np.testing.assert_array_equal(g1, g2)
    np.testing.assert_array_equal(b1, b2)
    assert np.all(g1 < 0)


def test_gated_rmsnorm_against_torch():
    rng = np.random.default_rng(15)
    o, z, w = rng.normal(size=(6, 16)), rng.normal(size=(6, 16)), rng.uniform(0.5, 1.5, 16)
    y = oracle.gated_rmsnorm(o, z, w, 1e-6)
    ref = F.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps=1e-6) * \
        F.silu(torch.from_numpy(z))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)
    # scale invariance (eps aside)
    y2 = oracle.gated_rmsnorm(1000.0 * o, z, w, 1e-6)
    np.testing.assert_allclose(y2, y, rtol=1e-6)


# ---------------------------------------------------------------- composition

def _layer_inputs(rng, T, Hk, Hv, d):
    QKV = 2 * Hk * d + Hv * d
    return dict(x=rng.normal(size=(T, QKV)), conv_w=rng.normal(0, 0.5, size=(QKV, 4)),
                conv_state=rng.normal(size=(QKV, 3)), S0=rng.normal(0, 0.1, size=(Hv, d, d)),
                a=rng.normal(size=(T, Hv)), b=rng.normal(size=(T, Hv)),
                decay_param=rng.uniform(-2, 0, Hv), dt_bias=rng.normal(size=Hv),
                z=rng.normal(size=(T, Hv, d)), norm_w=rng.uniform(0.5, 1.5, d))


@pytest.mark.parametrize("head_map", [oracle.MAP_GROUPED, oracle.MAP_TILED])
def test_segment_equals_library_composition(head_map):
    """Whole layer vs a composition of torch float64 library steps (conv1d,
    normalize, softplus, sigmoid, rms_norm) around the oracle's recurrence:
    pins the split offsets (q, then k, then v) and the order of the steps."""
    rng = np.random.default_rng(16)
    T, Hk, Hv, d = 4, 2, 4, 8
    L = _layer_inputs(rng, T, Hk, Hv, d)
    y, cs, S = oracle.segment(L["x"], L["conv_w"], L["conv_state"], L["S0"], Hk=Hk, Hv=Hv, dk=d,
                              dv=d, head_map=head_map, a=L["a"], b=L["b"],
                              decay_param=L["decay_param"], dt_bias=L["dt_bias"], z=L["z"],
                              norm_w=L["norm_w"])
    tt = torch.from_numpy
    QKV = L["x"].shape[1]
    seq = torch.cat([tt(L["conv_state"]), tt(L["x"]).T], dim=1)
    mixed = F.silu(F.conv1d(seq.unsqueeze(0), tt(L["conv_w"]).unsqueeze(1), groups=QKV))[0].T
    q = mixed[:, :Hk * d].reshape(T, Hk, d)
    k = mixed[:, Hk * d:2 * Hk * d].reshape(T, Hk, d)
    v = mixed[:, 2 * Hk * d:].reshape(T, Hv, d)
    q = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
    k = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    g = -torch.exp(tt(L["decay_param"])) * F.softplus(tt(L["a"]) + tt(L["dt_bias"]), threshold=20)
    beta = torch.sigmoid(tt(L["b"]))
    o, S_ref = oracle.recurrence(q.numpy(), k.numpy(), v.numpy(), g.numpy(), beta.numpy(), L["S0"],
                                 head_map)
    ref = F.rms_norm(tt(o), (d,), tt(L["norm_w"]), eps=1e-6) * F.silu(tt(L["z"]))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(cs, seq[:, -3:].numpy())


def test_segment_split_3_plus_1_is_bitwise():
    rng = np.random.default_rng(17)
    T, Hk, Hv, d = 4, 2, 4, 8
    L = _layer_inputs(rng, T, Hk, Hv, d)
    common = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=oracle.MAP_GROUPED,
                  decay_param=L["decay_param"], dt_bias=L["dt_bias"], norm_w=L["norm_w"])
    y, cs, S = oracle.segment(L["x"], L["conv_w"], L["conv_state"], L["S0"], a=L["a"], b=L["b"],
                              z=L["z"], **common)
    y1, cs1, S1 = oracle.segment(L["x"][:3], L["conv_w"], L["conv_state"], L["S0"], a=L["a"][:3],
                                 b=L["b"][:3], z=L["z"][:3], **common)
    y2, cs2, S2 = oracle.segment(L["x"][3:], L["conv_w"], cs1, S1, a=L["a"][3:], b=L["b"][3:],
                                 z=L["z"][3:], **common)
    assert np.array_equal(np.concatenate([y1, y2]), y)
    assert np.array_equal(cs2, cs) and np.array_equal(S2, S)


def test_batch_driver_equals_per_sequence_calls():
    rng = np.random.default_rng(18)
    B, T, Hk, Hv, d = 5, 2, 2, 4, 8
    Ls = [_layer_inputs(rng, T, Hk, Hv, d) for _ in range(B)]
    cw, dp, dtb, nw = Ls[0]["conv_w"], Ls[0]["decay_param"], Ls[0]["dt_bias"], Ls[0]["norm_w"]
    st = lambda key: np.stack([L[key] for L in Ls])  # noqa: E731
    for nthreads in (1, 3):
        y, cs, S = oracle.batch(B=B, T=T, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=oracle.MAP_TILED,
                                S0=st("S0"), a=st("a"), b=st("b"), decay_param=dp, dt_bias=dtb,
                                z=st("z"), norm_w=nw, x=st("x"), conv_w=cw,
                                conv_state=st("conv_state"), nthreads=nthreads)
        for i, L in enumerate(Ls):
            yi, csi, Si = oracle.segment(L["x"], cw, L["conv_state"], L["S0"], Hk=Hk, Hv=Hv, dk=d,
                                         dv=d, head_map=oracle.MAP_TILED, a=L["a"], b=L["b"],
                                         decay_param=dp, dt_bias=dtb, z=L["z"], norm_w=nw)
            assert np.array_equal(y[i], yi) and np.array_equal(cs[i], csi)
            assert np.array_equal(S[i], Si)


def test_core_given_gates_equals_recurrence():
    rng = np.random.default_rng(19)
    T, Hk, Hv, d = 3, 2, 4, 8
    q, k = rng.normal(size=(T, Hk, d)), rng.normal(size=(T, Hk, d))
    v = rng.normal(size=(T, Hv, d))
    g, beta = -rng.uniform(0, 1, (T, Hv)), rng.uniform(0, 1, (T, Hv))
    S0 = rng.normal(size=(Hv, d, d))
    y, S = oracle.core(q, k, v, S0, oracle.MAP_TILED, g=g, beta=beta, l2norm_qk=False)
    o, S2 = oracle.recurrence(q, k, v, g, beta, S0, oracle.MAP_TILED)
    assert np.array_equal(y, o) and np.array_equal(S, S2)


@pytest.mark.parametrize("head_map", ["grouped", "tiled"])
@pytest.mark.parametrize("raw", [True, False])
def test_packed_driver_equals_per_sequence_core(head_map, raw):
    """oracle.packed (one (sequence, v-head) pair per call, spread over threads) adds
    no arithmetic: it equals core over each whole sequence bit for bit, empty
    sequences leave their states alone, and a v-head subset leaves the rest."""
    rng = np.random.default_rng(31)
    Hk, Hv, dk, dv = 2, 6, 8, 4
    lengths = [5, 0, 3, 7]
    T, N = sum(lengths), len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k = rng.normal(size=(T, Hk, dk)), rng.normal(size=(T, Hk, dk))
    v, z = rng.normal(size=(T, Hv, dv)), rng.normal(size=(T, Hv, dv))
    S0 = rng.normal(0, 0.1, size=(N, Hv, dv, dk))
    kw = dict(z=z, norm_w=rng.normal(size=dv))
    if raw:
        kw.update(a=rng.normal(size=(T, Hv)), b=rng.normal(size=(T, Hv)),
                  decay_param=rng.uniform(-2, 0, Hv), dt_bias=rng.normal(size=Hv))
    else:
        kw.update(g=-rng.uniform(0, 0.5, (T, Hv)), beta=rng.uniform(0, 1, (T, Hv)))
    y, S = oracle.packed(q, k, v, S0, MAPS[head_map], cu, nthreads=3, **kw)
    for i in range(N):
        lo, hi = cu[i], cu[i + 1]
        if lo == hi:
            assert np.array_equal(S[i], S0[i])
            continue
        seq = {key: (val[lo:hi] if key in ("a", "b", "g", "beta", "z") else val)
               for key, val in kw.items()}
        yi, Si = oracle.core(q[lo:hi], k[lo:hi], v[lo:hi], S0[i], MAPS[head_map], **seq)
        assert np.array_equal(y[lo:hi], yi) and np.array_equal(S[i], Si)
    ys, Ss = oracle.packed(q, k, v, S0, MAPS[head_map], cu, heads=[1, 4], **kw)
    assert np.array_equal(ys[:, [1, 4]], y[:, [1, 4]]) and np.all(ys[:, [0, 2, 3, 5]] == 0)
    assert np.array_equal(Ss[:, [1, 4]], S[:, [1, 4]])
    assert np.array_equal(Ss[:, [0, 2, 3, 5]], S0[:, [0, 2, 3, 5]])
