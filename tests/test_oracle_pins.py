"""Pins of the fp64 oracle to facts it does not compute itself.

Each test fixes one part of the oracle against a hand-written fixture, a
closed form, an invariant, brute force on tiny inputs, a special case that
reduces to a textbook or library routine, or finite differences.  Passages:
the skill card "Reversible Sparse MoE Single Node" (Principle 3 "TQP
Optimizer Strategy", Architecture Details, Implementation Considerations) and
the abstract of "Reversible Foundations: Training a 120B Sparse MoE through
State-Preserving Scaling".
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_moe_expert_fp32_amd import configs, inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    base = dict(name="pin", cfg_id=101, T=24, d=64, E=6, k=2, f=64, r=4, group=32,
                act="f32", router_bias_var=0.0)
    base.update(kw)
    return configs.LayerConfig(**base)


# ------------------------------------------------------------- int4 base --

def test_int4_layout_golden():
    g = json.load(open(os.path.join(GOLD, "int4_layout.json")))
    for case in g["cases"]:
        vals = np.array(case["values"], dtype=np.int8)[None, :]
        packed = inputs.pack_int4(vals)
        assert packed[0].tolist() == case["bytes"]
        back = oracle.unpack_int4(np.array(case["bytes"], np.uint8)[None, :])
        assert back[0].tolist() == case["values"]
    sc = g["scaled"]
    w = oracle.dequantize(inputs.pack_int4(np.array(sc["values"], np.int8)[None, :]),
                          np.array([[sc["scale_bits"]]], np.uint16), 8)
    assert w[0].tolist() == sc["dequant"]


@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantize_error_bound_and_exact_dequant(group):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, 256)) * rng.uniform(0.01, 3, (48, 1))).astype(np.float32)
    w[3, :group] = 0.0                      # an all-zero group
    q, s = inputs.quantize_int4(w, group)
    wh = oracle.dequantize(q, s, group)
    sf = oracle.to_f64(s)
    bound = np.repeat(sf, group, axis=1) / 2
    assert np.all(np.abs(w.astype(np.float64) - wh) <= bound * (1 + 1e-12))
    assert np.all(wh[3, :group] == 0.0) and np.all(sf[3, 0] == 0.0)
    # q * s is exact: every value is an integer multiple of its scale
    qi = oracle.unpack_int4(q)
    assert np.abs(qi).max() <= 8 and qi.min() >= -8
    assert np.all(qi.max(axis=1) <= 7)
    # the largest magnitude of every non-zero group quantises to +-7
    qa = np.abs(qi).reshape(48, -1, group).max(axis=2)
    assert np.all(qa[sf > 0] == 7)


# ------------------------------------------------------------- int8 base --

def test_int8_layout_and_quantizer_golden():
    """The int8 storage ("Int8 or Int4", TQP Quantization): bytes, decoding,
    dequantisation and one hand-worked quantisation."""
    g = json.load(open(os.path.join(GOLD, "int8_layout.json")))
    for case in g["cases"]:
        back = oracle.unpack_int8(np.array(case["bytes"], np.uint8)[None, :])
        assert back[0].tolist() == case["values"]
    sc = g["scaled"]
    q = np.array(sc["values"], np.int8).view(np.uint8)[None, :]
    w = oracle.dequantize(q, np.array([[sc["scale_bits"]]], np.uint16), 8)
    assert w[0].tolist() == sc["dequant"]
    qz = g["quantize"]
    q8, s8 = inputs.quantize_int8(np.array([qz["w"]], np.float32), qz["group"])
    assert s8.tolist() == [[qz["scale_bits"]]]
    assert q8.view(np.int8)[0].tolist() == qz["q"]


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_int8_error_bound_and_exact_dequant(group):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((32, 256)) * rng.uniform(0.01, 3, (32, 1))).astype(np.float32)
    w[5, group:2 * group] = 0.0             # an all-zero group
    q, s = inputs.quantize_int8(w, group)
    assert q.shape == (32, 256)
    wh = oracle.dequantize(q, s, group)
    sf = oracle.to_f64(s)
    bound = np.repeat(sf, group, axis=1) / 2
    assert np.all(np.abs(w.astype(np.float64) - wh) <= bound * (1 + 1e-12))
    assert np.all(wh[5, group:2 * group] == 0.0) and sf[5, 1] == 0.0
    qi = oracle.unpack_int8(q)
    assert qi.min() >= -128 and qi.max() <= 127
    # the largest magnitude of every non-zero group quantises to +-127, and
    # -128 is never produced
    qa = np.abs(qi).reshape(32, -1, group).max(axis=2)
    assert np.all(qa[sf > 0] == 127) and qi.min() >= -127


def test_int8_and_int4_layers_agree_on_shared_values():
    """Values in [-7, 7] stored as int8 and as int4 with the same scales give
    the same dequantised experts, so the oracle's layer must be identical for
    both storage widths (a wrong int8 decoding -- unsigned bytes, a wrong
    group repeat -- changes it)."""
    cfg = tiny(act="f32")
    inp4 = inputs.generate(cfg, 3)
    inp8 = dict(inp4)
    rng = np.random.default_rng(11)
    for m in ("gate", "up", "down"):
        E, N, _ = inp4[f"q_{m}"].shape
        K = inp4[f"s_{m}"].shape[-1] * cfg.group
        vals = rng.integers(-7, 8, size=(E, N, K)).astype(np.int8)
        inp4[f"q_{m}"] = inputs.pack_int4(vals)
        inp8[f"q_{m}"] = np.ascontiguousarray(vals.view(np.uint8))
    f4 = oracle.forward(inp4, cfg.k, cfg.group)
    f8 = oracle.forward(inp8, cfg.k, cfg.group)
    assert np.array_equal(f4["y"], f8["y"])
    b4 = oracle.backward(inp4, f4, cfg.k, cfg.group)
    b8 = oracle.backward(inp8, f8, cfg.k, cfg.group)
    for key in b4:
        assert np.array_equal(b4[key], b8[key]), key
    # and a value outside the int4 range changes the int8 layer
    inp8["q_down"] = inp8["q_down"].copy()
    inp8["q_down"][0, 0, 0] = np.uint8(100)
    assert not np.array_equal(oracle.forward(inp8, cfg.k, cfg.group)["y"], f8["y"])


# ---------------------------------------------------------------- router --

def test_router_logits_dyadic_exact():
    """x in {i/16}, W_r in {j/64}: the exact rational result, from integer
    arithmetic, must be reproduced bit for bit."""
    rng = np.random.default_rng(1)
    T, d, E = 7, 40, 9
    xi = rng.integers(-32, 33, (T, d))
    wi = rng.integers(-64, 65, (d, E))
    bi = rng.integers(-100, 101, E)
    x = (xi / 16).astype(np.float32)
    w = (wi / 64).astype(np.float32)
    b = (bi / 1024).astype(np.float32)
    l = oracle.router_logits(x, w, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(int(xi[t, c]), 16) * Fraction(int(wi[c, e]), 64)
                        for c in range(d)) + Fraction(int(bi[e]), 1024)
            assert Fraction(l[t, e]) == exact


def _brute_topk(row, k):
    """Unique k-subset S with: every i in S beats every j outside S
    (larger logit, or equal logit and lower index)."""
    E = len(row)
    beats = lambda i, j: row[i] > row[j] or (row[i] == row[j] and i < j)
    good = [S for S in itertools.combinations(range(E), k)
            if all(beats(i, j) for i in S for j in range(E) if j not in S)]
    assert len(good) == 1
    S = list(good[0])
    # descending logit, ties to lower index: sort by pairwise "beats"
    for a in range(len(S)):
        for b in range(len(S) - 1 - a):
            if beats(S[b + 1], S[b]):
                S[b], S[b + 1] = S[b + 1], S[b]
    return S


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (8, 3), (10, 4), (12, 6), (7, 7)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # coarse values force many exact ties
    l = rng.integers(-3, 4, (40, E)).astype(np.float64)
    idx = oracle.topk(l, k)
    for t in range(l.shape[0]):
        assert idx[t].tolist() == _brute_topk(l[t], k)


def test_exact_tie_lower_index():
    """Duplicated router columns give bitwise-equal logits; the lower expert
    index must win."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 32)).astype(np.float32)
    w = rng.standard_normal((32, 6)).astype(np.float32)
    w[:, 4] = w[:, 1]
    l = oracle.router_logits(x, w)
    assert np.array_equal(l[:, 4], l[:, 1])
    idx = oracle.topk(l, 6)
    for t in range(16):
        row = idx[t].tolist()
        assert row.index(1) < row.index(4)


# ----------------------------------------------------------------- gates --

def test_gates_invariants():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 9)) * 3
    for k in (1, 3, 9):
        idx = oracle.topk(l, k)
        g = oracle.gates(l, idx)
        assert np.allclose(g.sum(axis=1), 1.0, atol=4 * k * np.finfo(float).eps)
        assert np.all(np.diff(g, axis=1) <= 1e-15)           # descending like the logits
        g2 = oracle.gates(l + 123.25, idx)
        assert np.allclose(g, g2, rtol=1e-12, atol=0)
        if k == 1:
            assert np.all(g == 1.0)
    # k = E: the gates are the plain softmax over all experts (scipy)
    from scipy.special import softmax
    idx = oracle.topk(l, 9)
    g = oracle.gates(l, idx)
    ref = np.take_along_axis(softmax(l, axis=1), idx.astype(np.int64), axis=1)
    assert np.allclose(g, ref, rtol=1e-13, atol=0)


def test_near_tie_masks():
    l = np.array([[3.0, 2.0, 2.0 - 5e-6, 0.0],
                  [3.0, 3.0 - 1e-6, 1.0, 0.0],
                  [3.0, 2.0, 1.0, 0.0]])
    b, o = oracle.near_ties(l, 2)
    assert b.tolist() == [True, False, False]
    assert o.tolist() == [False, True, False]


# ----------------------------------------------------------- permutation --

def test_permutation_invariants_and_recount():
    rng = np.random.default_rng(4)
    T, E, k = 57, 11, 3
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
    idx[5] = [10, 0, 3]
    counts, offsets, perm_src, slot_pos = oracle.permutation(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert sorted(perm_src.tolist()) == list(range(T * k))
    assert np.all(slot_pos[perm_src] == np.arange(T * k))
    # brute force: slots sorted by (expert, token)
    order = sorted(range(T * k), key=lambda s: (int(idx.reshape(-1)[s]), s // k))
    assert perm_src.tolist() == order
    for e in range(E):
        assert counts[e] == int((idx == e).sum())


# ---------------------------------------------------------------- experts --

def _layer(cfg, seed=0, mutate=None):
    inp = inputs.generate(cfg, seed, threads=1)
    if mutate:
        mutate(inp)
    return inp


def _dense_mixture(inp, cfg, lam):
    """k = E: y = sum_e softmax(l)_e FFN_e(x), a dense loop over experts with
    no routing, permutation or gather."""
    from scipy.special import softmax
    x = oracle.to_f64(inp["x"])
    p = softmax(oracle.router_logits(inp["x"], inp["w_router"], inp.get("b_router")), axis=1)
    y = np.zeros_like(x)
    for e in range(cfg.E):
        ex = oracle.Expert(inp, e, cfg.group)
        y += p[:, e:e + 1] * oracle.expert_forward(ex, x, lam)["O"]
    return y


def test_k_equals_E_is_dense_softmax_mixing():
    cfg = tiny(k=6, router_bias_var=0.3)
    inp = _layer(cfg)
    out = oracle.forward(inp, cfg.k, cfg.group, 0.7)
    assert np.allclose(out["y"], _dense_mixture(inp, cfg, 0.7), rtol=1e-12, atol=1e-13)


def test_textbook_swiglu_single_expert():
    """E = 1, k = 1, lam = 0: y = W_d (silu(W_g x) * (W_u x)), written with
    torch.nn.functional in float64."""
    import torch
    import torch.nn.functional as F
    cfg = tiny(E=1, k=1)
    inp = _layer(cfg)
    out = oracle.forward(inp, 1, cfg.group, 0.0)
    W = {m: torch.from_numpy(oracle.dequantize(inp[f"q_{m}"][0], inp[f"s_{m}"][0], cfg.group))
         for m in ("gate", "up", "down")}
    x = torch.from_numpy(oracle.to_f64(inp["x"]))
    y = F.linear(F.silu(F.linear(x, W["gate"])) * F.linear(x, W["up"]), W["down"])
    assert np.allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-13)


def test_zero_B_reduces_to_dequantized_base():
    cfg = tiny()

    def zero_b(inp):
        for m in ("gate", "up", "down"):
            inp[f"B_{m}"][:] = 0
    inp = _layer(cfg, mutate=zero_b)
    out = oracle.forward(inp, cfg.k, cfg.group, 1.0)
    base = oracle.forward(inp, cfg.k, cfg.group, 0.0)
    assert np.array_equal(out["y"], base["y"])
    # and the base alone equals a per-token loop over the selected experts
    x = oracle.to_f64(inp["x"])
    for t in range(cfg.T):
        acc = np.zeros(cfg.d)
        for j in range(cfg.k):
            e = out["topk_idx"][t, j]
            Wg, Wu, Wd = (oracle.dequantize(inp[f"q_{m}"][e], inp[f"s_{m}"][e], cfg.group)
                          for m in ("gate", "up", "down"))
            h = oracle.silu(Wg @ x[t]) * (Wu @ x[t])
            acc += out["gates"][t, j] * (Wd @ h)
        assert np.allclose(out["y"][t], acc, rtol=1e-12, atol=1e-13)


def test_zero_base_isolates_low_rank_path():
    """q = 0: every matrix is lam * A @ B, computed here as explicit dense
    adapter matrices with torch."""
    import torch
    import torch.nn.functional as F
    cfg = tiny(E=1, k=1)

    def zero_q(inp):
        for m in ("gate", "up", "down"):
            inp[f"q_{m}"][:] = 0
    inp = _layer(cfg, mutate=zero_q)
    lam = 0.5
    out = oracle.forward(inp, 1, cfg.group, lam)
    M = {m: lam * torch.from_numpy(oracle.to_f64(inp[f"B_{m}"][0]) @ oracle.to_f64(inp[f"A_{m}"][0]))
         for m in ("gate", "up", "down")}
    x = torch.from_numpy(oracle.to_f64(inp["x"]))
    y = F.linear(F.silu(F.linear(x, M["gate"])) * F.linear(x, M["up"]), M["down"])
    assert np.abs(out["y"]).max() > 1e-3
    assert np.allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-14)


def test_down_adapter_enters_linearly():
    cfg = tiny()
    inp = _layer(cfg)
    Bd = inp["B_down"].copy()

    def run(scale):
        inp["B_down"][:] = Bd * scale
        return oracle.forward(inp, cfg.k, cfg.group, 1.0)["y"]
    y0, y1, y2 = run(0.0), run(1.0), run(2.0)
    assert np.allclose(y2 - y0, 2 * (y1 - y0), rtol=1e-11, atol=1e-12)
    assert np.abs(y1 - y0).max() > 1e-4


# --------------------------------------------------------------- backward --

def _loss(inp, cfg, lam, idx):
    out = oracle.forward(inp, cfg.k, cfg.group, lam, topk_idx=idx)
    return float((oracle.to_f64(inp["dy"]) * out["y"]).sum())


ADAPTERS = ("A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down")


def test_backward_directional_finite_difference():
    cfg = tiny(router_bias_var=0.2)
    inp = _layer(cfg)
    lam = 0.8
    fwd = oracle.forward(inp, cfg.k, cfg.group, lam, keep=True)
    g = oracle.backward(inp, fwd, cfg.k, cfg.group, lam)
    rng = np.random.default_rng(9)
    base = {n: inp[n].astype(np.float64).copy() for n in ADAPTERS + ("x",)}
    dirs = {n: rng.standard_normal(base[n].shape) for n in base}
    # fp64 inputs are accepted by the oracle as exact values
    pred = sum((g["d" + n] * dirs[n]).sum() for n in ADAPTERS) + (g["dx"] * dirs["x"]).sum()
    eps = 1e-6
    vals = []
    for sgn in (+1, -1):
        for n in base:
            inp[n] = base[n] + sgn * eps * dirs[n]
        assert np.array_equal(oracle.route(inp, cfg.k)["topk_idx"], fwd["topk_idx"])
        vals.append(_loss(inp, cfg, lam, None))
    fd = (vals[0] - vals[1]) / (2 * eps)
    assert abs(fd - pred) <= 1e-6 * max(1.0, abs(pred))


def test_backward_single_entries_finite_difference():
    cfg = tiny()
    inp = _layer(cfg)
    lam = 1.0
    fwd = oracle.forward(inp, cfg.k, cfg.group, lam, keep=True)
    g = oracle.backward(inp, fwd, cfg.k, cfg.group, lam)
    rng = np.random.default_rng(11)
    for n in ADAPTERS:
        inp[n] = inp[n].astype(np.float64)
    inp["x"] = inp["x"].astype(np.float64)
    for _ in range(60):
        n = ADAPTERS[rng.integers(len(ADAPTERS))] if rng.random() < 0.8 else "x"
        a = inp[n]
        i = tuple(int(rng.integers(s)) for s in a.shape)
        old = a[i]
        eps = 1e-6 * max(1.0, abs(old))
        a[i] = old + eps
        lp = _loss(inp, cfg, lam, fwd["topk_idx"] if n != "x" else None)
        a[i] = old - eps
        lm = _loss(inp, cfg, lam, fwd["topk_idx"] if n != "x" else None)
        a[i] = old
        fd = (lp - lm) / (2 * eps)
        an = g["dx"][i] if n == "x" else g["d" + n][i]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, i, fd, an)


def test_backward_matches_torch_autograd_dense():
    """An independent formulation: per-token, per-selected-expert loop in
    torch float64 with autograd through x, every A and B and the softmax over
    the selected logits."""
    import torch
    import torch.nn.functional as F
    for k in (2, 6):
        cfg = tiny(k=k, router_bias_var=0.4)
        inp = _layer(cfg)
        lam = 0.9
        fwd = oracle.forward(inp, cfg.k, cfg.group, lam, keep=True)
        g = oracle.backward(inp, fwd, cfg.k, cfg.group, lam)
        tt = lambda a: torch.from_numpy(oracle.to_f64(a)).requires_grad_(True)
        x = tt(inp["x"])
        P = {n: tt(inp[n]) for n in ADAPTERS}
        W = {m: torch.from_numpy(oracle.dequantize(inp[f"q_{m}"], inp[f"s_{m}"], cfg.group))
             for m in ("gate", "up", "down")}
        wr = torch.from_numpy(oracle.to_f64(inp["w_router"]))
        logits = x @ wr
        if inp.get("b_router") is not None:
            logits = logits + torch.from_numpy(oracle.to_f64(inp["b_router"]))
        idx = torch.from_numpy(fwd["topk_idx"].astype(np.int64))
        gam = torch.softmax(torch.gather(logits, 1, idx), dim=1)
        y = torch.zeros_like(x)
        for t in range(cfg.T):
            for j in range(cfg.k):
                e = int(idx[t, j])
                lin = lambda v, m: (F.linear(v, W[m][e])
                                    + lam * F.linear(F.linear(v, P[f"A_{m}"][e]), P[f"B_{m}"][e]))
                h = F.silu(lin(x[t], "gate")) * lin(x[t], "up")
                y[t] = y[t] + gam[t, j] * lin(h, "down")
        (y * torch.from_numpy(oracle.to_f64(inp["dy"]))).sum().backward()
        assert np.allclose(g["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
        for n in ADAPTERS:
            assert np.allclose(g["d" + n], P[n].grad.numpy(), rtol=1e-10, atol=1e-12), n


def test_backward_special_cases():
    cfg = tiny(E=8, k=1)

    def prep(inp):
        for m in ("gate", "up", "down"):
            inp[f"B_{m}"][:] = 0
        # no token picks expert 7: a very negative router bias
        b = np.zeros(cfg.E, np.float32)
        b[7] = -100.0
        inp["b_router"] = b
    inp = _layer(cfg, mutate=prep)
    fwd = oracle.forward(inp, cfg.k, cfg.group, 1.0, keep=True)
    assert fwd["counts"][7] == 0
    g = oracle.backward(inp, fwd, cfg.k, cfg.group, 1.0)
    for m in ("gate", "up", "down"):
        assert np.all(g[f"dA_{m}"] == 0.0)          # B = 0  =>  dA = 0 exactly
        assert np.all(g[f"dB_{m}"][7] == 0.0)       # empty expert
    assert np.abs(g["dB_gate"]).max() > 0


# --------------------------------------------------------- sampled forms --

def test_sampled_forms_agree_with_whole_layer():
    cfg = tiny(T=30, E=7, k=3, router_bias_var=0.5)
    inp = _layer(cfg)
    lam = 1.0
    fwd = oracle.forward(inp, cfg.k, cfg.group, lam, keep=True)
    bwd = oracle.backward(inp, fwd, cfg.k, cfg.group, lam)
    toks = [0, 7, 29]
    ft = oracle.forward_tokens(inp, toks, cfg.k, cfg.group, lam)
    assert np.array_equal(ft["topk_idx"], fwd["topk_idx"][toks])
    assert np.allclose(ft["y"], fwd["y"][toks], rtol=1e-12, atol=1e-13)
    dxt = oracle.backward_tokens(inp, toks, cfg.k, cfg.group, lam)
    assert np.allclose(dxt, bwd["dx"][toks], rtol=1e-11, atol=1e-12)
    R = oracle.route(inp, cfg.k)
    for e in range(cfg.E):
        ge = oracle.expert_grads(inp, R, e, cfg.k, cfg.group, lam)
        for n in ADAPTERS:
            assert np.allclose(ge["d" + n], bwd["d" + n][e], rtol=1e-11, atol=1e-13)


def test_generator_is_deterministic():
    a = inputs.generate(configs.C1, 0, threads=1)
    b = inputs.generate(configs.C1, 0, threads=4)
    assert inputs.checksums(a) == inputs.checksums(b)
    c = inputs.generate(configs.C1, 1, threads=1)
    assert inputs.checksums(a)["x"] != inputs.checksums(c)["x"]


# ----------------------------------------------- adapter optimizer (AdamW) --
# The pages put the optimizer state on the adapters only (skill card,
# Principle 3 "TQP Optimizer Strategy"); the optimizer itself is read as
# AdamW (decoupled weight decay, bias-corrected moments).

ADAMW_HP = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.05)


def test_adamw_first_step_is_sign_step():
    # from zero moments at t = 1 the bias corrections cancel exactly:
    # m_hat = g, v_hat = g^2, so the step is lr * g / (|g| + eps) + decay
    rng = np.random.default_rng(7)
    p, g = rng.standard_normal(1000), rng.standard_normal(1000)
    z = np.zeros(1000)
    p1, m1, v1 = oracle.adamw_step(p, g, z, z, step=1, **ADAMW_HP)
    hp = ADAMW_HP
    np.testing.assert_allclose(m1, (1 - hp["beta1"]) * g, rtol=1e-15)
    np.testing.assert_allclose(v1, (1 - hp["beta2"]) * g * g, rtol=1e-15)
    want = p - hp["lr"] * (np.sign(g) * np.abs(g) / (np.abs(g) + hp["eps"]) + hp["weight_decay"] * p)
    np.testing.assert_allclose(p1, want, rtol=1e-13, atol=1e-15)


def test_adamw_constant_gradient_closed_form():
    # with a constant gradient, m_t = (1 - beta1^t) g and v_t = (1 - beta2^t)
    # g^2, so every bias-corrected step is the same: p_t = p_0 - t lr g/(|g|+eps)
    # (no weight decay); a wrong power of beta or step index breaks this
    rng = np.random.default_rng(8)
    p0, g = rng.standard_normal(64), rng.standard_normal(64)
    p, m, v = p0.copy(), np.zeros(64), np.zeros(64)
    hp = dict(ADAMW_HP, weight_decay=0.0)
    for t in range(1, 41):
        p, m, v = oracle.adamw_step(p, g, m, v, step=t, **hp)
        np.testing.assert_allclose(m, (1 - hp["beta1"] ** t) * g, rtol=1e-12)
        np.testing.assert_allclose(v, (1 - hp["beta2"] ** t) * g * g, rtol=1e-12)
    np.testing.assert_allclose(p, p0 - 40 * hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-11,
                               atol=1e-13)


def test_adamw_zero_gradient_is_pure_decay():
    p = np.linspace(-2, 2, 17)
    z = np.zeros(17)
    p1, m1, v1 = oracle.adamw_step(p, z, z, z, step=3, **ADAMW_HP)
    assert np.all(m1 == 0) and np.all(v1 == 0)
    np.testing.assert_allclose(p1, p * (1 - ADAMW_HP["lr"] * ADAMW_HP["weight_decay"]), rtol=1e-15)


def test_adamw_matches_torch_adamw_float64():
    # the library routine torch.optim.AdamW (decoupled weight decay, on the
    # CPU in float64) over several steps of random gradients
    import torch
    rng = np.random.default_rng(9)
    p0 = rng.standard_normal((5, 7))
    grads = [rng.standard_normal((5, 7)) for _ in range(6)]
    hp = ADAMW_HP
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, step=t, **hp)
    st = opt.state[tp]
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-15)


# ---- reversible residual block around the layer

def test_reversible_block_inverts_and_reduces():
    """y2 = x2 + MoE(y1) is undone by x2 = y2 - MoE(y1) up to float64
    rounding; with x2 = 0 it is the layer itself; with a zero layer (zero base
    and zero B, so every expert output is 0) it is the identity, exactly."""
    cfg = tiny()
    inp = _layer(cfg)
    rng = np.random.default_rng(5)
    x2 = rng.standard_normal((cfg.T, cfg.d)).astype(np.float32)
    y2 = oracle.rev_forward(inp, x2, cfg.k, cfg.group)
    m = oracle.forward(inp, cfg.k, cfg.group)["y"]
    assert np.abs(m).max() > 1e-3
    back = oracle.rev_inverse(inp, y2, cfg.k, cfg.group)
    bound = 4 * np.finfo(np.float64).eps * (np.abs(x2) + np.abs(m))
    assert np.all(np.abs(back - x2) <= bound)
    assert np.array_equal(oracle.rev_forward(inp, np.zeros_like(x2), cfg.k, cfg.group), m)

    def zero_layer(inp):
        for mat in ("gate", "up", "down"):
            inp[f"q_{mat}"][:] = 0
            inp[f"B_{mat}"][:] = 0
    z = _layer(cfg, mutate=zero_layer)
    assert np.array_equal(oracle.rev_forward(z, x2, cfg.k, cfg.group), x2.astype(np.float64))
    assert np.array_equal(oracle.rev_inverse(z, x2, cfg.k, cfg.group), x2.astype(np.float64))


# ---- few -> many expert growth

@pytest.mark.parametrize("factor", [2, 3])
def test_growth_preserves_the_function(factor):
    """Unperturbed growth by F with F k experts per token: every original
    selection becomes its F copies, each with 1/F of the gate, and the layer
    output is unchanged up to float64 rounding."""
    cfg = tiny(router_bias_var=0.5)
    inp = _layer(cfg)
    g = oracle.grow(inp, factor)
    assert g["q_gate"].shape[0] == cfg.E * factor
    y0 = oracle.forward(inp, cfg.k, cfg.group)["y"]
    R0, R1 = oracle.route(inp, cfg.k), oracle.route(g, cfg.k * factor)
    for t in range(cfg.T):
        assert sorted(R1["topk_idx"][t] // factor) == sorted(np.repeat(R0["topk_idx"][t], factor))
        for e in R0["topk_idx"][t]:
            sel = R1["topk_idx"][t] // factor == e
            j = list(R0["topk_idx"][t]).index(e)
            assert np.allclose(R1["gates"][t][sel], R0["gates"][t][j] / factor, rtol=1e-12)
    y1 = oracle.forward(g, cfg.k * factor, cfg.group)["y"]
    assert np.allclose(y1, y0, rtol=1e-11, atol=1e-13)


def test_growth_router_noise_moves_only_copies():
    cfg = tiny()
    inp = _layer(cfg)
    z = np.random.default_rng(3).standard_normal((cfg.d, cfg.E * 2)).astype(np.float32)
    g = oracle.grow(inp, 2, z, 0.25)
    w0 = inp["w_router"]
    assert np.array_equal(g["w_router"][:, 0::2], w0)
    want = (w0.astype(np.float64) + 0.25 * z[:, 1::2].astype(np.float64)).astype(np.float32)
    assert np.array_equal(g["w_router"][:, 1::2], want)
    st = oracle.routing_load(oracle.route(g, cfg.k * 2)["topk_idx"], cfg.E * 2)
    assert st["max_over_mean"] >= 1.0 and 0 <= st["empty"] <= cfg.E * 2


def test_routing_load_hand_counted_fixture():
    """The routing-collapse statistic against hand-counted loads
    (tests/golden/routing_load.json): empty experts, including the
    highest-index one, and a maximum shared by two experts."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "routing_load.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        st = oracle.routing_load(np.array(c["topk_idx"], np.int32), c["E"])
        assert st["empty"] == c["empty"], c["note"]
        assert st["max_over_mean"] == c["max_over_mean"], c["note"]


def test_parallel_executor_matches_whole_layer():
    """tests/oracle_parallel.py (the oracle's per-expert function in worker
    processes, routing, combine and gate path in the caller) reproduces
    oracle.forward / oracle.backward to float64 rounding, empty experts
    included."""
    import oracle_parallel
    cfg = tiny(T=40, E=9, k=3, cfg_id=140, router_bias_var=0.5)
    inp = inputs.generate(cfg, 0)
    fwd = oracle.forward(inp, cfg.k, cfg.group, cfg.lora_scale, keep=True)
    bwd = oracle.backward(inp, fwd, cfg.k, cfg.group, cfg.lora_scale)
    par = oracle_parallel.layer(inp, cfg, backward=True, workers=3)
    assert np.array_equal(par["topk_idx"], fwd["topk_idx"])
    assert np.array_equal(par["perm_src"], fwd["perm_src"])
    for key, ref in (("e_out", fwd["e_out"]), ("y", fwd["y"]), ("dx", bwd["dx"]),
                     *((n, bwd[n]) for n in oracle.ADAPTER_GRADS)):
        np.testing.assert_allclose(par[key], ref, rtol=1e-12, atol=1e-14, err_msg=key)
