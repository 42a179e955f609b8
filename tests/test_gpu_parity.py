"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

Shapes the oracle finishes in seconds, spanning several tiles with ragged
tails, plus the edge cases of the layer.  The full-size shapes are in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import oracle
from parity import ADAPTERS, check_routing, full_parity, rel_l2, run_gpu
from sparse_moe_expert_fp32_amd import configs, inputs

pytestmark = pytest.mark.gpu


def cfg_of(**kw):
    base = dict(name="t", cfg_id=200, T=300, d=256, E=16, k=4, f=384, r=16, group=128,
                act="bf16", router_bias_var=0.3, train=True)
    base.update(kw)
    return configs.LayerConfig(**base)


def show(name, rep):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in rep.items()), flush=True)


def test_tiny_f32_forward_backward(cuda_ok):
    cfg = configs.C1
    inp = inputs.generate(cfg, 0)
    rep, _ = full_parity(cfg, inp)
    show("C1", rep)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_small_bf16_forward_backward(cuda_ok, group):
    cfg = cfg_of(group=group, cfg_id=210 + group)
    rep, _ = full_parity(cfg, inputs.generate(cfg, 0))
    show(f"bf16 g{group}", rep)


def test_small_f32_ragged(cuda_ok):
    cfg = cfg_of(act="f32", T=77, d=192, E=12, k=3, f=160, r=5, group=32, cfg_id=220)
    rep, _ = full_parity(cfg, inputs.generate(cfg, 1))
    show("f32 ragged", rep)


@pytest.mark.parametrize("kw", [
    dict(T=1, cfg_id=230),                               # one token
    dict(T=37, k=1, cfg_id=231),                         # k = 1, ragged T
    dict(E=8, k=8, T=50, cfg_id=232),                    # k = E
    dict(E=70, k=5, T=129, cfg_id=233),                  # E not a multiple of 64
    dict(E=130, k=12, T=64, cfg_id=234, router_bias_var=0.0),  # many empty experts
    dict(E=40, k=13, T=45, cfg_id=235),                  # k not a multiple of 4
    dict(E=48, k=20, T=40, cfg_id=236),                  # k > 16: block-per-token kernels
    dict(d=384, cfg_id=237),                             # d % 256 != 0: partial column tile
    dict(d=640, f=256, T=150, cfg_id=238),               # (down output and dX_perm)
    dict(T=127, cfg_id=239, router_bias_var=4.0),        # short batch, experts of 33+ rows
])
def test_edge_shapes(cuda_ok, kw):
    cfg = cfg_of(**kw)
    rep, gpu = full_parity(cfg, inputs.generate(cfg, 0))
    show(f"edge {kw}", rep)


def test_routing_collapse_to_one_expert(cuda_ok):
    cfg = cfg_of(T=200, E=10, k=1, cfg_id=240)
    inp = inputs.generate(cfg, 0)
    b = np.zeros(cfg.E, np.float32)
    b[3] = 1e4
    inp["b_router"] = b
    rep, gpu = full_parity(cfg, inp)
    assert gpu["counts"][3] == cfg.T and gpu["counts"].sum() == cfg.T
    for n in ADAPTERS:
        assert np.all(np.delete(gpu[n], 3, axis=0) == 0.0)
    show("collapse", rep)


def test_vanishing_gate_takes_the_direct_gate_gradient(cuda_ok):
    """One expert's router bias 200 above the rest: every token's second gate
    underflows to 0 in float32, so the per-token pass cannot divide the dH
    partials by it and takes the dots with e_out instead."""
    cfg = cfg_of(T=96, E=8, k=2, cfg_id=241, router_bias_var=0.0)
    inp = inputs.generate(cfg, 0)
    b = np.zeros(cfg.E, np.float32)
    b[5] = 200.0
    inp["b_router"] = b
    rep, gpu = full_parity(cfg, inp)
    assert gpu["counts"][5] == cfg.T
    show("vanishing gate", rep)


def test_router_dyadic_bit_exact(cuda_ok):
    """x in {i/16}, W_r in {j/64}: every fp32 partial sum is exact, so the GPU
    logits equal the oracle's bit for bit and routing needs no tie exemption."""
    for act in ("f32", "bf16"):
        cfg = cfg_of(act=act, T=256, d=512, E=100, k=12, cfg_id=250, router_bias_var=0.0)
        inp = inputs.generate(cfg, 0)
        rng = np.random.default_rng(7)
        xi = rng.integers(-64, 65, (cfg.T, cfg.d)).astype(np.float32) / 16
        inp["x"] = xi if act == "f32" else inputs.bf16_bits(xi)
        inp["w_router"] = rng.integers(-64, 65, (cfg.d, cfg.E)).astype(np.float32) / 64
        gpu, _ = run_gpu(cfg, inp, backward=False)
        l64 = oracle.router_logits(inp["x"], inp["w_router"])
        assert np.array_equal(gpu["logits"].astype(np.float64), l64)
        assert np.array_equal(gpu["topk_idx"], oracle.topk(l64, cfg.k))


def test_router_exact_ties_lower_index(cuda_ok):
    cfg = cfg_of(T=128, E=20, k=5, cfg_id=251, router_bias_var=0.0)
    inp = inputs.generate(cfg, 0)
    w = inp["w_router"]
    w[:, 9] = w[:, 2]
    w[:, 15] = w[:, 2]
    gpu, _ = run_gpu(cfg, inp, backward=False)
    assert np.array_equal(gpu["logits"][:, 2], gpu["logits"][:, 9])
    l64 = oracle.router_logits(inp["x"], w)
    ref = oracle.topk(l64, cfg.k)
    for t in range(cfg.T):
        row = gpu["topk_idx"][t].tolist()
        for a, b in ((2, 9), (2, 15), (9, 15)):
            if a in row and b in row:
                assert row.index(a) < row.index(b)
            if b in row:
                assert a in row
    check_routing(cfg, gpu, l64)
    assert (gpu["topk_idx"] == ref).all(axis=1).mean() > 0.99


def test_permute_on_oracle_indices(cuda_ok):
    """moe_permute alone, fed the oracle's selection: exact, no exemption."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(T=1000, E=460, k=12, d=128, f=128, cfg_id=252)
    inp = inputs.generate(cfg, 0)
    idx = oracle.route(inp, cfg.k)["topk_idx"]
    L = DeviceLayer(cfg, inp, want_x_perm=True, with_backward=False)
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.permute()
    torch.cuda.synchronize()
    ref = oracle.permutation(idx, cfg.E)
    for name, r in zip(("counts", "offsets", "perm_src", "slot_pos"), ref):
        assert np.array_equal(to_numpy(getattr(L, name)), r), name
    xp = to_numpy(L.x_perm)
    assert np.array_equal(xp, inp["x"][ref[2] // cfg.k])


def test_bitwise_deterministic(cuda_ok):
    import torch
    from sparse_moe_expert_fp32_amd.layer import to_numpy
    cfg = cfg_of(T=500, E=40, k=6, cfg_id=260)
    inp = inputs.generate(cfg, 0)
    a, L = run_gpu(cfg, inp)
    L.train_step()
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(L.y), a["y"])
    assert np.array_equal(to_numpy(L.dx), a["dx"])
    for n in ADAPTERS:
        assert np.array_equal(to_numpy(L.grads[n]), a[n]), n


@pytest.mark.parametrize("kw", [
    dict(T=60, E=64, k=2, cfg_id=270),                # 120 rows over 64 experts: some get none
    dict(T=70, E=48, k=2, d=384, f=256, cfg_id=271),  # down output columns 384: a partial tile
])
def test_packed_base_matches_plain_layout(cuda_ok, kw):
    """The layer with the base packed once (moe_pack_base_f for the forward,
    moe_pack_base_t for the backward) gives the same bits as the layer that
    reads the plain layout (and re-lays out the base in its workspace for the
    backward), also with experts that receive no rows (the packing covers
    every expert) and with a partial last column tile."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(**kw)
    inp = inputs.generate(cfg, 0)
    from sparse_moe_expert_fp32_amd import binding as B
    out = []
    for pack in (False, True, "mixed"):
        L = DeviceLayer(cfg, inp, device="cuda:0", pack_base=bool(pack))
        assert bool(L.packed) == bool(pack) and bool(L.packed_f) == bool(pack)
        if pack == "mixed":
            # a forward-packed down and gate but a plain up: gate/up falls back
            # to the plain layout (both or neither), down stays packed
            L.w["up"] = B.qlora(L.t["q_up"], L.t["s_up"], L.t["A_up"], L.t["B_up"],
                                L.packed["up"], None)
            # (the forward now re-derives the ratio tables: a workspace with room)
            L.ws[B.CALL_EXPERT_FWD] = torch.empty(
                B.moe_workspace_size(L.dm, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN),
                dtype=torch.uint8, device="cuda:0")
        L.train_step()
        torch.cuda.synchronize()
        out.append({"y": to_numpy(L.y), "e_out": to_numpy(L.e_out), "dx": to_numpy(L.dx),
                    **{n: to_numpy(L.grads[n]) for n in ADAPTERS}})
        counts = to_numpy(L.counts)
    assert (counts == 0).any()
    for o in out[1:]:
        for n in out[0]:
            assert np.array_equal(out[0][n], o[n]), n


def test_reversible_block_replay(cuda_ok):
    """Reversible residual block around the layer: y2 = x2 + MoE(y1) on the
    GPU agrees with the oracle to the layer tolerance; the backward's replay
    recomputes MoE(y1) bit for bit (stateless routing) and recovers x2 within
    the two roundings to bf16 (half an ulp of y2 plus half an ulp of x2)."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(T=200, E=16, k=4, cfg_id=280, train=False)
    inp = inputs.generate(cfg, 0)
    L = DeviceLayer(cfg, inp, device="cuda:0", with_backward=False)
    rng = np.random.default_rng(11)
    x2 = torch.from_numpy(rng.standard_normal((cfg.T, cfg.d)).astype(np.float32)).to(
        "cuda:0").to(torch.bfloat16)
    y2, back = torch.empty_like(x2), torch.empty_like(x2)
    L.rev_forward(x2, y2)
    m1 = to_numpy(L.y)
    idx = to_numpy(L.topk_idx)
    L.rev_inverse(y2, back)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(L.y), m1)          # replayed bit for bit
    x2n, y2n, bn = to_numpy(x2), to_numpy(y2), to_numpy(back)
    R = oracle.route(inp, cfg.k)
    b, o = oracle.near_ties(R["logits"], cfg.k)
    assert np.all((idx == R["topk_idx"]).all(axis=1) | b | o)
    ref = oracle.rev_forward(inp, x2n, cfg.k, cfg.group, cfg.lora_scale, topk_idx=idx)
    e_y2 = rel_l2(oracle.to_f64(y2n), ref)
    assert e_y2 <= 1e-2
    ulp = lambda v: np.spacing(np.abs(oracle.to_f64(v)).astype(np.float32)).astype(np.float64) * 65536
    err = np.abs(oracle.to_f64(bn) - oracle.to_f64(x2n))
    assert np.all(err <= 0.5 * (ulp(y2n) + ulp(bn)) * 1.001)
    show("reversible", {"y2": e_y2, "max_abs_x2_err": float(err.max()),
                        "exact_fraction": float((err == 0).mean())})


def test_expert_growth(cuda_ok):
    """Few -> many growth on the GPU (moe_grow_copy, moe_grow_router): the
    grown tensors equal the oracle's growth bit for bit (router columns moved
    by noise: within one float32 ulp); unperturbed, the grown layer with
    twice the experts and twice k routes every token to both copies of its
    original experts and computes the original function; perturbed, the
    routing-collapse statistic of the grown router is reported."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, grow_inputs, to_device, to_numpy
    F = 2
    cfg = cfg_of(T=128, E=12, k=3, cfg_id=290, router_bias_var=0.5, train=False)
    inp = inputs.generate(cfg, 0)
    z = np.random.default_rng(9).standard_normal((cfg.d, cfg.E * F)).astype(np.float32)
    t = {k: to_device(v, "cuda:0") for k, v in inp.items()}
    for s in (0.0, 0.05):
        cfg2, g = grow_inputs(t, cfg, F, z, s)
        torch.cuda.synchronize()
        ref = oracle.grow(inp, F, z, s)
        for key, v in ref.items():
            if v is None or key in ("x", "dy"):
                continue
            got = to_numpy(g[key])
            if key == "w_router":
                assert np.all(np.abs(got.astype(np.float64) - v) <= np.spacing(np.abs(v))), key
            else:
                assert np.array_equal(got, v), key
    L0 = DeviceLayer(cfg, inp, device="cuda:0", with_backward=False)
    L0.forward()
    cfg2, g = grow_inputs(t, cfg, F)
    L1 = DeviceLayer(cfg2, g, device="cuda:0", with_backward=False)
    L1.forward()
    torch.cuda.synchronize()
    i0, i1 = to_numpy(L0.topk_idx), to_numpy(L1.topk_idx)
    for t_ in range(cfg.T):
        assert sorted(i1[t_] // F) == sorted(np.repeat(i0[t_], F))
    yref = oracle.forward(inp, cfg.k, cfg.group, cfg.lora_scale, topk_idx=i0)["y"]
    e0 = rel_l2(oracle.to_f64(to_numpy(L0.y)), yref)
    e1 = rel_l2(oracle.to_f64(to_numpy(L1.y)), yref)
    assert e0 <= 1e-2 and e1 <= 1e-2
    cfg3, g3 = grow_inputs(t, cfg, F, z, 0.05)
    L3 = DeviceLayer(cfg3, g3, device="cuda:0", with_backward=False)
    L3.forward()
    torch.cuda.synchronize()
    st0 = oracle.routing_load(i0, cfg.E)
    st3 = oracle.routing_load(to_numpy(L3.topk_idx), cfg3.E)
    e3 = rel_l2(oracle.to_f64(to_numpy(L3.y)), yref)
    show("growth", {"y_grown": e1, "y_orig": e0, "y_perturbed_vs_orig": e3,
                    "max_over_mean_before": st0["max_over_mean"],
                    "max_over_mean_after": st3["max_over_mean"], "empty_after": st3["empty"]})


def test_grow_copy_and_couple_scalar_paths(cuda_ok):
    """The byte-wise path of moe_grow_copy (blocks not a multiple of 16
    bytes) and the element-wise path of moe_rev_couple (pointers not 16-byte
    aligned, float32 activations), against numpy."""
    import torch
    from sparse_moe_expert_fp32_amd import binding as B
    rng = np.random.default_rng(13)
    src_np = rng.integers(0, 256, size=(5, 7), dtype=np.uint8)
    src = torch.from_numpy(src_np).to("cuda:0")
    dst = torch.empty((15, 7), dtype=torch.uint8, device="cuda:0")
    B.moe_grow_copy(src, dst, 7, 5, 3)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), np.repeat(src_np, 3, axis=0))
    cfg = cfg_of(act="f32", T=3, d=64, E=4, k=1, f=128, r=4, group=32, cfg_id=291)
    dm = B.dims_of(cfg)
    x_np = rng.standard_normal(cfg.T * cfg.d + 1).astype(np.float32)
    m_np = rng.standard_normal(cfg.T * cfg.d + 1).astype(np.float32)
    x = torch.from_numpy(x_np).to("cuda:0")[1:]     # 4-byte aligned views
    m = torch.from_numpy(m_np).to("cuda:0")[1:]
    out = torch.empty(cfg.T * cfg.d + 1, dtype=torch.float32, device="cuda:0")[1:]
    B.moe_rev_couple(dm, x, m, out, -1)
    torch.cuda.synchronize()
    want = (x_np[1:].astype(np.float64) - m_np[1:].astype(np.float64)).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("r", [4, 8, 32])
def test_matrix_core_ranks(cuda_ok, r):
    """Adapter ranks other than 16 on the matrix-core path (their epilogues
    read Z and the adapter factors from global memory, masked to the rank;
    rank 32 takes two K steps), forward and backward against the oracle."""
    cfg = cfg_of(r=r, cfg_id=300 + r)
    rep, _ = full_parity(cfg, inputs.generate(cfg, 0))
    show(f"rank {r}", rep)


def _bf16_pow2(bits: np.ndarray, e: int) -> np.ndarray:
    """bf16 bit patterns times 2^e (exact: exponent field moved by e)."""
    b = bits.astype(np.int32)
    nz = (b & 0x7F80) != 0
    return np.where(nz, b + (e << 7), b).astype(np.uint16)


def test_group_scales_zero_and_spread(cuda_ok):
    """Group scales on the matrix-core path: columns with an all-zero group
    (q = 0, s = 0) and columns whose group scales span 2^48 (one group's
    scale times 2^24, the next zero, the next times 2^-24), in the gate and
    down matrices of every expert.  The forward telescopes group scales
    through ratios, so this is where a zero scale or a large spread could
    overflow; the backward scales its activations instead.  Forward and
    backward against the oracle, y also column by column."""
    cfg = cfg_of(T=200, E=12, k=3, d=384, f=384, cfg_id=310)
    inp = inputs.generate(cfg, 0)
    for m in ("gate", "down"):
        q, sc = inp[f"q_{m}"].copy(), inp[f"s_{m}"].copy()
        N = q.shape[1]
        spread = np.arange(N) % 7 == 0
        zero = np.arange(N) % 7 == 3
        sc[:, spread, 0] = _bf16_pow2(sc[:, spread, 0], 24)
        sc[:, spread, 2] = _bf16_pow2(sc[:, spread, 2], -24)
        for sel in (spread, zero):
            sc[:, sel, 1] = 0
            q[:, sel, 64:128] = 0
        inp[f"q_{m}"], inp[f"s_{m}"] = q, sc
    rep, gpu = full_parity(cfg, inp)
    ref = oracle.forward(inp, cfg.k, cfg.group, cfg.lora_scale, topk_idx=gpu["topk_idx"])
    ecol = rel_l2_cols = [rel_l2(oracle.to_f64(gpu["y"])[:, c], ref["y"][:, c])
                          for c in range(cfg.d)]
    assert np.all(np.isfinite(oracle.to_f64(gpu["y"])))
    assert max(ecol) <= 1e-2, (int(np.argmax(ecol)), max(ecol))
    rep["y_column_max"] = float(max(rel_l2_cols))
    show("group scales", rep)


def test_nan_input_row_keeps_routing_valid(cuda_ok):
    """A NaN in a row of x makes that token's logits NaN: the router still
    writes k distinct experts in [0, E) for it (NaN competes as -inf), every
    other token is routed as the oracle routes it, and the permutation stays
    a bijection."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(T=100, E=20, k=6, cfg_id=320, train=False)
    inp = inputs.generate(cfg, 0)
    bad = [5, 77]
    x = inp["x"].copy()
    x[5, 17] = 0x7FC0                      # bf16 quiet NaN
    x[77, :] = 0x7FC0
    inp["x"] = x
    L = DeviceLayer(cfg, inp, device="cuda:0", want_logits=True, with_backward=False)
    L.forward()
    torch.cuda.synchronize()
    idx = to_numpy(L.topk_idx)
    assert idx.min() >= 0 and idx.max() < cfg.E
    for t in range(cfg.T):
        assert len(set(idx[t].tolist())) == cfg.k, t
    for t in bad:                          # all logits NaN: lowest indices, in order
        assert idx[t].tolist() == list(range(cfg.k)), idx[t]
    good = np.setdiff1d(np.arange(cfg.T), bad)
    l64 = oracle.router_logits(inp["x"][good], inp["w_router"], inp.get("b_router"))
    ref = oracle.topk(l64, cfg.k)
    b, o = oracle.near_ties(l64, cfg.k)
    assert np.all((idx[good] == ref).all(axis=1) | b | o)
    ps = to_numpy(L.perm_src)
    assert np.array_equal(np.sort(ps), np.arange(cfg.S))
    y = oracle.to_f64(to_numpy(L.y))
    assert np.all(np.isfinite(y[good]))


def test_permute_repairs_invalid_caller_indices(cuda_ok):
    """moe_permute fed indices outside [0, E) and repeated within a token: each
    token's entries are made valid in j order (clamped; a repeat becomes the
    lowest unused expert), and the placement is that of the repaired routing
    (bit-exact against the oracle's permutation of it)."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(T=300, E=10, k=4, d=128, f=128, cfg_id=330, train=False)
    inp = inputs.generate(cfg, 0)
    rng = np.random.default_rng(3)
    idx = rng.integers(-3, 14, size=(cfg.T, cfg.k)).astype(np.int32)
    idx[0] = [2, 2, 2, 2]
    idx[1] = [-1, -5, 20, 9]
    L = DeviceLayer(cfg, inp, with_backward=False)
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.permute()
    torch.cuda.synchronize()
    fixed = np.empty_like(idx)
    for t in range(cfg.T):
        used = []
        for j in range(cfg.k):
            e = min(max(int(idx[t, j]), 0), cfg.E - 1)
            if e in used:
                e = min(set(range(cfg.E)) - set(used))
            used.append(e)
        fixed[t] = used
    assert fixed[0].tolist() == [2, 0, 1, 3] and fixed[1].tolist() == [0, 1, 9, 2]
    ref = oracle.permutation(fixed, cfg.E)
    for name, r in zip(("counts", "offsets", "perm_src", "slot_pos"), ref):
        assert np.array_equal(to_numpy(getattr(L, name)), r), name
