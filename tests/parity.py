"""Shared helpers of the GPU parity tests: run the HIP library through the C
ABI and the fp64 oracle on the same seeded inputs, and compare them under
the rules of the layer: routing bit-exact except near-ties (k-th and
(k+1)-th logits closer than 1e-5, counted and reported), outputs and adapter
gradients within a relative L2 error (1e-5 float32, 1e-2 bf16)."""
from __future__ import annotations

import numpy as np

import oracle
from sparse_moe_expert_fp32_amd import configs, inputs

ADAPTERS = ("dA_gate", "dB_gate", "dA_up", "dB_up", "dA_down", "dB_down")
TIE = 1e-5


def tol(cfg):
    return 1e-5 if cfg.act == "f32" else 1e-2


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return num / den if den > 0 else num


def f64(a):
    return oracle.to_f64(a)


def check_routing(cfg, gpu: dict, logits64: np.ndarray) -> dict:
    """Routing parity against the oracle's fp64 logits.  Returns the routing
    the oracle is to be evaluated on (the oracle's own, with the GPU's row
    substituted on near-tie tokens) and the near-tie statistics."""
    k = cfg.k
    ref_idx = oracle.topk(logits64, k)
    boundary, order = oracle.near_ties(logits64, k, TIE)
    flagged = boundary | order
    g_idx = gpu["topk_idx"]
    same = np.all(g_idx == ref_idx, axis=1)
    bad = ~same & ~flagged
    assert not bad.any(), f"routing differs on {bad.sum()} non-tie tokens, first {np.nonzero(bad)[0][:5]}"
    # on flagged tokens the GPU's set must still be a valid top-k within the tie band
    for t in np.nonzero(~same)[0]:
        kth = np.sort(logits64[t])[::-1][k - 1]
        assert len(set(g_idx[t].tolist())) == k
        assert np.all(logits64[t, g_idx[t]] >= kth - TIE)
    use_idx = np.where(same[:, None], ref_idx, g_idx).astype(np.int32)
    # permutation: bit-exact function of the routing
    counts, offsets, perm_src, slot_pos = oracle.permutation(use_idx, cfg.E)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], offsets)
    assert np.array_equal(gpu["perm_src"], perm_src)
    assert np.array_equal(gpu["slot_pos"], slot_pos)
    gam = oracle.gates(logits64, use_idx)
    err_g = rel_l2(gpu["gates"], gam)
    assert err_g <= 1e-5, f"gates rel L2 {err_g:.3e}"
    return {"topk_idx": use_idx, "near_ties": int(flagged.sum()),
            "substituted": int((~same).sum()), "gates_err": err_g}


def run_gpu(cfg, inp, backward=True, want_logits=True):
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    L = DeviceLayer(cfg, inp, want_logits=want_logits, with_backward=backward)
    L.forward()
    if backward:
        L.adapter_bwd()
    torch.cuda.synchronize()
    out = L.routing()
    out["y"] = to_numpy(L.y)
    out["e_out"] = to_numpy(L.e_out)
    if backward:
        out["dx"] = to_numpy(L.dx)
        for n in ADAPTERS:
            out[n] = to_numpy(L.grads[n])
    return out, L


def per_row_rel(got, ref) -> np.ndarray:
    """Relative L2 error of every row (leading index) of got against ref."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = got.reshape(got.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def compare_layer(cfg, gpu: dict, ref: dict, backward: bool, report: dict, seed_note=""):
    """Whole-tensor relative L2 of y, dX and the six adapter gradients, plus
    the per-unit rules: every token's y and dX row and every expert's block
    of each adapter gradient within the same tolerance of its own norm, and
    experts with no rows exactly zero.  The per-expert maximum is reported.
    An expert whose reference block is below 1e-30 of the largest block's
    norm (every gate it received underflows float32) is held to the
    tolerance times that largest norm instead: float32 cannot carry it."""
    t = tol(cfg)
    report["y"] = rel_l2(f64(gpu["y"]), ref["y"])
    assert report["y"] <= t, f"y rel L2 {report['y']:.3e} > {t} {seed_note}"
    ey = per_row_rel(f64(gpu["y"]), ref["y"])
    report["y_token_max"] = float(ey.max())
    assert ey.max() <= t, f"y of token {int(ey.argmax())}: rel L2 {ey.max():.3e} {seed_note}"
    if not backward:
        return report
    report["dx"] = rel_l2(f64(gpu["dx"]), ref["dx"])
    assert report["dx"] <= t, f"dx rel L2 {report['dx']:.3e}"
    ex = per_row_rel(f64(gpu["dx"]), ref["dx"])
    report["dx_token_max"] = float(ex.max())
    assert ex.max() <= t, f"dx of token {int(ex.argmax())}: rel L2 {ex.max():.3e}"
    counts = np.diff(np.asarray(ref["offsets"]))
    empty = counts == 0
    worst = (0.0, None, None)
    for n in ADAPTERS:
        report[n] = rel_l2(gpu[n], ref[n])
        assert report[n] <= t, f"{n} rel L2 {report[n]:.3e}"
        assert np.all(gpu[n][empty] == 0.0), f"{n} of an empty expert is not zero"
        rn = np.linalg.norm(np.asarray(ref[n], np.float64).reshape(cfg.E, -1), axis=1)
        tiny = ~empty & (rn < 1e-30 * rn.max())
        if tiny.any():
            gn = np.linalg.norm(np.asarray(gpu[n], np.float64).reshape(cfg.E, -1)[tiny], axis=1)
            assert gn.max() <= t * rn.max(), f"{n}: an underflowing expert has norm {gn.max():.3e}"
        keep = ~empty & ~tiny
        ee = per_row_rel(gpu[n][keep], ref[n][keep])
        if ee.size and ee.max() > worst[0]:
            worst = (float(ee.max()), n, int(np.nonzero(keep)[0][ee.argmax()]))
        assert ee.size == 0 or ee.max() <= t, \
            f"{n} of expert {int(np.nonzero(keep)[0][ee.argmax()])}: rel L2 {ee.max():.3e}"
    report["expert_max"] = worst[0]
    report["expert_max_at"] = f"{worst[1]}[{worst[2]}] ({int(counts[worst[2]])} rows)" \
        if worst[1] else "-"
    return report


def full_parity(cfg, inp, backward=True, seed_note=""):
    """Whole-layer comparison for shapes the oracle finishes in seconds."""
    gpu, _ = run_gpu(cfg, inp, backward)
    logits64 = oracle.router_logits(inp["x"], inp["w_router"], inp.get("b_router"))
    R = check_routing(cfg, gpu, logits64)
    lam = cfg.lora_scale
    fwd = oracle.forward(inp, cfg.k, cfg.group, lam, topk_idx=R["topk_idx"], keep=backward)
    report = {"near_ties": R["near_ties"], "gates": R["gates_err"]}
    ref = dict(fwd)
    if backward:
        ref.update(oracle.backward(inp, fwd, cfg.k, cfg.group, lam))
    compare_layer(cfg, gpu, ref, backward, report, seed_note)
    return report, gpu
