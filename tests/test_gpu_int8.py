"""GPU parity of the int8-base layer against the fp64 oracle, through the C
ABI ("Int8 or Int4": skill card "Reversible Sparse MoE Single Node",
Implementation Considerations, TQP Quantization).  The float32 kernels read
the bytes directly; the matrix-core path runs an int8 base as two int4 planes
(h = q >> 4 with scale 16 s, l - 8 with scale s, l = q & 15)."""
import numpy as np
import pytest

from parity import ADAPTERS, full_parity
from sparse_moe_expert_fp32_amd import configs, inputs

pytestmark = pytest.mark.gpu


def cfg_of(**kw):
    base = dict(name="i8", cfg_id=600, T=300, d=256, E=16, k=4, f=384, r=16, group=128,
                act="bf16", router_bias_var=0.3, train=True, bits=8)
    base.update(kw)
    return configs.LayerConfig(**base)


def show(name, rep):
    print(f"[parity int8] {name}: " + " ".join(
        f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}" for k, v in rep.items()), flush=True)


def test_int8_tiny_f32(cuda_ok):
    cfg = configs.C1.with_(name="tiny_f32_int8", cfg_id=601, bits=8)
    rep, _ = full_parity(cfg, inputs.generate(cfg, 0))
    show("C1 int8", rep)


@pytest.mark.parametrize("kw", [
    dict(cfg_id=610),                                   # matrix-core path, ragged tails
    dict(group=32, cfg_id=611),                         # float32 kernels with bf16 storage
    dict(d=384, T=200, cfg_id=612),                     # partial last column tile
    dict(T=64, E=64, k=12, d=1024, f=512, cfg_id=613, router_bias_var=0.0),  # decode-shaped
    dict(E=70, k=5, T=129, cfg_id=614),                 # empty experts, E not a multiple of 64
])
def test_int8_bf16_forward_backward(cuda_ok, kw):
    cfg = cfg_of(**kw)
    rep, gpu = full_parity(cfg, inputs.generate(cfg, 0))
    show(str(kw), rep)


def test_int8_packed_matches_per_call_packing(cuda_ok):
    """An int8 base packed once by the caller (moe_pack_base_f / _t) gives the
    same bits as the layer that packs it in its workspace on every call."""
    import torch
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, to_numpy
    cfg = cfg_of(cfg_id=620, E=24)
    inp = inputs.generate(cfg, 0)
    out = []
    for pack in (False, True):
        L = DeviceLayer(cfg, inp, device="cuda:0", pack_base=pack)
        assert bool(L.packed_f) == pack
        L.train_step()
        torch.cuda.synchronize()
        out.append({"y": to_numpy(L.y), "dx": to_numpy(L.dx),
                    **{n: to_numpy(L.grads[n]) for n in ADAPTERS}})
    for n in out[0]:
        assert np.array_equal(out[0][n], out[1][n]), n


def test_int8_full_range_values(cuda_ok):
    """Bytes over the whole int8 range, including -128 (never produced by the
    quantiser but decodable), and zero scales."""
    cfg = cfg_of(cfg_id=630, T=160)
    inp = inputs.generate(cfg, 0)
    rng = np.random.default_rng(3)
    for m in ("gate", "up", "down"):
        q = inp[f"q_{m}"]
        q[...] = rng.integers(0, 256, size=q.shape, dtype=np.uint8)
        s = inp[f"s_{m}"]
        # scales of the quantiser's size for these bytes (max |q| ~ 128)
        sf = inputs.bf16_to_f32(s) * np.float32(127.0 / 128.0)
        sf[0, :3, 0] = 0.0                               # zero groups
        inp[f"s_{m}"] = inputs.bf16_bits(sf)
    rep, _ = full_parity(cfg, inp)
    show("full range", rep)
