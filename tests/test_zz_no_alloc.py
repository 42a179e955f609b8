"""moe_expert_fwd_noalloc (the forward without a workspace, on the library's
fixed device scratch) against moe_expert_fwd with a workspace, through the C
ABI: the same inputs give the same bits, on two calls in a row of which the
second is smaller (the fixed array keeps the first call's contents), with and
without a save buffer."""
import numpy as np
import pytest

from sparse_moe_expert_fp32_amd import configs, inputs

pytestmark = pytest.mark.gpu


def _pair(cfg, seed, with_save):
    """The routed layer on the GPU, then its expert forward through both entry
    points (outputs and save buffers from each)."""
    import torch
    from sparse_moe_expert_fp32_amd import binding as B
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    L = DeviceLayer(cfg, inputs.generate(cfg, seed), device="cuda:0", with_backward=with_save)
    L.route()
    L.permute()
    outs = []
    for noalloc in (False, True):
        e_out = torch.full_like(L.e_out, float("nan"))
        save = torch.full_like(L.save, 0xFF) if with_save else None
        args = (L.dm, L.t["x"], L.offsets, L.perm_src, L.w["gate"], L.w["up"], L.w["down"],
                e_out, save)
        if noalloc:
            B.moe_expert_fwd_noalloc(*args)
        else:
            B.moe_expert_fwd(*args, L.ws[B.CALL_EXPERT_FWD])
        torch.cuda.synchronize()
        outs.append((to_numpy(e_out), None if save is None else save.cpu().numpy()))
    return outs


@pytest.mark.parametrize("with_save", [False, True])
def test_noalloc_forward_matches_workspace_forward(cuda_ok, with_save):
    big = configs.LayerConfig("noalloc_a", 400, T=600, d=512, E=24, k=4, f=384, r=16,
                              group=128, act="bf16", router_bias_var=0.5)
    small = big.with_(name="noalloc_b", cfg_id=401, T=70, E=24, k=3)
    for cfg in (big, small):            # the second call smaller than the first
        (ref, ref_save), (got, got_save) = _pair(cfg, 0, with_save)
        assert not np.isnan(inputs.bf16_to_f32(ref)).any()   # every row written
        assert np.array_equal(got, ref), cfg.name
        if with_save:
            assert np.array_equal(got_save, ref_save), cfg.name
        print(f"[noalloc] {cfg.name} save={with_save}: e_out {ref.shape} bitwise equal",
              flush=True)
