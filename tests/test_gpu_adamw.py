"""GPU parity of the adapter optimizer step (moe_adamw_step) against the fp64
oracle, through the C ABI: the 16-byte vector path with a ragged tail, the
scalar path (a tensor that starts off 16-byte alignment), both copies of the
new parameter (float32, bf16), several steps in a row, and one step of the
layer's six adapters after a training step."""
import numpy as np
import pytest

import oracle
from sparse_moe_expert_fp32_amd import configs, inputs

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
# the call takes its hyperparameters as float32: the oracle gets those values
HP32 = {k: float(np.float32(v)) for k, v in HP.items()}
EPS32 = 2.0 ** -23


def _check(p_gpu, m_gpu, v_gpu, p_ref, m_ref, v_ref, p_old, m_old, v_old, g, step):
    """float32 arithmetic from float32 inputs, bounded term by term: each
    result may carry a few roundings of the magnitudes that were added (sums
    can cancel, so the bound is not relative to the result)."""
    h = HP32
    p_old, m_old, v_old, g = (np.asarray(a, np.float64) for a in (p_old, m_old, v_old, g))
    tol_m = 4 * EPS32 * (h["beta1"] * np.abs(m_old) + (1 - h["beta1"]) * np.abs(g)) + 1e-38
    tol_v = 4 * EPS32 * (h["beta2"] * v_old + (1 - h["beta2"]) * g * g) + 1e-38
    assert np.all(np.abs(m_gpu - m_ref) <= tol_m), step
    assert np.all(np.abs(v_gpu - v_ref) <= tol_v), step
    bc1, bc2 = 1 - h["beta1"] ** step, 1 - h["beta2"] ** step
    den = np.sqrt(v_ref / bc2) + h["eps"]
    ratio = np.abs(m_ref) / bc1 / den
    # the GPU's own moment errors, carried into the step
    carried = (tol_m / bc1 + ratio * 0.5 * (tol_v / np.maximum(v_ref, 1e-38)) * np.sqrt(v_ref / bc2)) / den
    tol_p = (2 * EPS32 * np.maximum(np.abs(p_ref), np.abs(p_old))
             + h["lr"] * (16 * EPS32 * (ratio + h["weight_decay"] * np.abs(p_old)) + carried) + 1e-38)
    err = np.abs(p_gpu.astype(np.float64) - p_ref)
    assert np.all(err <= tol_p), (step, float((err / tol_p).max()))


@pytest.mark.parametrize("n,offset,copy", [(4 * 1000 + 3, 0, "bf16"), (4099, 1, "f32"),
                                           (1, 0, None), (70000, 0, "bf16")])
def test_adamw_steps_match_oracle(cuda_ok, n, offset, copy):
    import torch
    from sparse_moe_expert_fp32_amd import binding as B
    rng = np.random.default_rng(n + offset)
    dev = torch.device("cuda:0")
    p = rng.standard_normal(n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    # the tensors live at `offset` elements into their allocations
    mk = lambda a: torch.from_numpy(np.concatenate([np.zeros(offset, np.float32), a])).to(dev)[offset:]
    tp, tm, tv = mk(p), mk(m), mk(v)
    tout = None
    if copy == "bf16":
        tout = torch.empty(n, dtype=torch.bfloat16, device=dev)
    elif copy == "f32":
        tout = torch.empty(n + offset, dtype=torch.float32, device=dev)[offset:]
    pr, mr, vr = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    for step in range(1, 4):
        g = (rng.standard_normal(n) * (0.1 if step == 2 else 1.0)).astype(np.float32)
        if step == 3:
            g[: n // 7] = 0.0          # zero gradients: pure decay of p, decay of moments
        tg = mk(g)
        # the oracle starts from the GPU's own float32 state of the previous step
        p_old = tp.cpu().numpy().astype(np.float64)
        m_old, v_old = tm.cpu().numpy(), tv.cpu().numpy()
        B.moe_adamw_step(B.adamw_hparams(step=step, **HP), tp, tg, tm, tv, tout)
        torch.cuda.synchronize()
        pr, mr, vr = oracle.adamw_step(p_old, g, m_old, v_old, step=step, **HP32)
        pg, mg, vg = tp.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy()
        _check(pg, mg, vg, pr, mr, vr, p_old, m_old, v_old, g, step)
        if copy == "bf16":
            # the copy is the new master rounded to nearest even
            want = torch.from_numpy(pg).to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(tout.cpu().view(torch.int16).numpy(), want)
        elif copy == "f32":
            assert np.array_equal(tout.cpu().numpy(), pg)
    print(f"[adamw] n={n} offset={offset} copy={copy}: ok", flush=True)


def test_layer_adapters_one_step(cuda_ok):
    # after a training step, one optimizer step over the six adapters: the
    # masters follow the oracle and the bf16 adapters the forward reads are
    # the new masters rounded to nearest even
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = configs.LayerConfig(name="t", cfg_id=210, T=200, d=256, E=8, k=2, f=256, r=16,
                              group=128, act="bf16", router_bias_var=0.0, train=True)
    inp = inputs.generate(cfg, 0)
    L = DeviceLayer(cfg, inp, device="cuda:0")
    L.train_step()
    L.init_optimizer()
    torch.cuda.synchronize()
    grads = {k: to_numpy(v) for k, v in L.grads.items()}
    L.optimizer_step(**HP)
    torch.cuda.synchronize()
    for gname, pname in L.ADAPTERS:
        p0 = oracle.to_f64(inp[pname])
        pr, mr, vr = oracle.adamw_step(p0, grads[gname], np.zeros_like(p0), np.zeros_like(p0),
                                       step=1, **HP32)
        master, m, v = (to_numpy(t) for t in L.opt[pname])
        z = np.zeros_like(p0)
        _check(master, m, v, pr, mr, vr, p0, z, z, grads[gname], 1)
        want = torch.from_numpy(master).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(L.t[pname].cpu().view(torch.int16).numpy(), want), pname
