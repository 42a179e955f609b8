"""Device buffers for one layer and the call sequence of the five entry points.

This is plumbing around the C ABI: it uploads the (numpy) inputs once,
allocates outputs and workspaces with torch, and calls the library in the
order route -> permute -> expert_fwd -> combine [-> adapter_bwd].  No
arithmetic of the layer happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

MATS = ("gate", "up", "down")


def to_device(a, device):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_numpy(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceLayer:
    def __init__(self, cfg, inputs: dict, device: str = "cuda", want_logits: bool = False,
                 want_x_perm: bool = False, with_backward: bool | None = None,
                 pack_base: bool = True):
        self.cfg = cfg
        self.dev = torch.device(device)
        self.dm = B.dims_of(cfg)
        T, d, E, k, f, r = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.r
        S = T * k
        act = torch.float32 if cfg.act == "f32" else torch.bfloat16
        self.t = {key: to_device(v, self.dev) for key, v in inputs.items()}
        self.w = {m: B.qlora(self.t[f"q_{m}"], self.t[f"s_{m}"], self.t[f"A_{m}"],
                             self.t[f"B_{m}"]) for m in MATS}
        z = lambda *shape, dtype=act: torch.empty(shape, dtype=dtype, device=self.dev)
        i32, f32 = torch.int32, torch.float32
        self.topk_idx, self.gates = z(T, k, dtype=i32), z(T, k, dtype=f32)
        self.logits = z(T, E, dtype=f32) if want_logits else None
        self.counts, self.offsets = z(E, dtype=i32), z(E + 1, dtype=i32)
        self.perm_src, self.slot_pos = z(S, dtype=i32), z(S, dtype=i32)
        self.x_perm = z(S, d) if want_x_perm else None
        self.e_out, self.y = z(S, d), z(T, d)
        bwd = cfg.train if with_backward is None else with_backward
        self.save = (torch.empty(B.moe_save_size(self.dm), dtype=torch.uint8, device=self.dev)
                     if bwd else None)
        # the frozen base re-laid out once (matrix-core path): stage-major for
        # the forward, transposed for the backward
        self.packed, self.packed_f = {}, {}
        packing = pack_base and B.pack_base_supported(self.dm)
        # workspaces sized for what this layer supplies (a save buffer when
        # it trains, the packed bases when it packs)
        flags = {B.CALL_EXPERT_FWD: (B.WS_SAVE_GIVEN if bwd else 0) |
                 (B.WS_PACKED_GIVEN if packing else 0),
                 B.CALL_ADAPTER_BWD: B.WS_PACKED_GIVEN if packing else 0}
        calls = (B.CALL_ROUTE, B.CALL_PERMUTE, B.CALL_EXPERT_FWD, B.CALL_COMBINE) + \
            ((B.CALL_ADAPTER_BWD,) if bwd else ())
        self.ws = {c: torch.empty(max(1, B.moe_workspace_size(self.dm, c | flags.get(c, 0))),
                                  dtype=torch.uint8, device=self.dev) for c in calls}
        if packing:
            nbf = B.moe_pack_base_f_size(self.dm)
            nbt = B.moe_pack_base_t_size(self.dm) if bwd else 0
            for m in MATS:
                mat = B.MAT_DOWN if m == "down" else B.MAT_GATE_UP
                self.packed_f[m] = torch.empty(nbf, dtype=torch.uint8, device=self.dev)
                B.moe_pack_base_f(self.dm, mat, self.t[f"q_{m}"], self.t[f"s_{m}"],
                                  self.packed_f[m])
                if bwd:
                    self.packed[m] = torch.empty(nbt, dtype=torch.uint8, device=self.dev)
                    B.moe_pack_base_t(self.dm, mat, self.t[f"q_{m}"], self.t[f"s_{m}"],
                                      self.packed[m])
            self.w = {m: B.qlora(self.t[f"q_{m}"], self.t[f"s_{m}"], self.t[f"A_{m}"],
                                 self.t[f"B_{m}"], self.packed.get(m), self.packed_f[m])
                      for m in MATS}
        if bwd:
            self.dx = z(T, d)
            self.grads = {"dA_gate": z(E, r, d, dtype=f32), "dB_gate": z(E, f, r, dtype=f32),
                          "dA_up": z(E, r, d, dtype=f32), "dB_up": z(E, f, r, dtype=f32),
                          "dA_down": z(E, r, f, dtype=f32), "dB_down": z(E, d, r, dtype=f32)}

    # ---- the five calls
    def route(self, stream=None):
        t = self.t
        B.moe_route(self.dm, t["x"], t["w_router"], t.get("b_router"), self.topk_idx, self.gates,
                    self.logits, self.ws[B.CALL_ROUTE], stream)

    def permute(self, stream=None):
        B.moe_permute(self.dm, self.topk_idx, self.t["x"], self.counts, self.offsets,
                      self.perm_src, self.slot_pos, self.x_perm, self.ws[B.CALL_PERMUTE], stream)

    def expert_fwd(self, stream=None):
        B.moe_expert_fwd(self.dm, self.t["x"], self.offsets, self.perm_src, self.w["gate"],
                         self.w["up"], self.w["down"], self.e_out, self.save,
                         self.ws[B.CALL_EXPERT_FWD], stream)

    def combine(self, stream=None):
        B.moe_combine(self.dm, self.e_out, self.slot_pos, self.gates, self.y, None, stream)

    def adapter_bwd(self, stream=None):
        t, g = self.t, self.grads
        B.moe_adapter_bwd(self.dm, t["dy"], t["x"], self.topk_idx, self.gates, self.offsets,
                          self.perm_src, self.slot_pos, t["w_router"], self.w["gate"],
                          self.w["up"], self.w["down"], self.e_out, self.save, self.dx,
                          g["dA_gate"], g["dB_gate"], g["dA_up"], g["dB_up"], g["dA_down"],
                          g["dB_down"], self.ws[B.CALL_ADAPTER_BWD], stream)

    def forward(self, stream=None):
        self.route(stream)
        self.permute(stream)
        self.expert_fwd(stream)
        self.combine(stream)

    def train_step(self, stream=None):
        self.forward(stream)
        self.adapter_bwd(stream)

    # ---- reversible residual block around the layer: the layer input x is
    # the block's stream y1, m = MoE(y1) is self.y after forward()
    def rev_forward(self, x2, y2, stream=None):
        """y2 = x2 + MoE(y1)."""
        self.forward(stream)
        B.moe_rev_couple(self.dm, x2, self.y, y2, +1, stream)

    def rev_inverse(self, y2, x2, stream=None):
        """x2 = y2 - MoE(y1), MoE(y1) recomputed from y1 (stateless routing)."""
        self.forward(stream)
        B.moe_rev_couple(self.dm, y2, self.y, x2, -1, stream)

    # ---- adapter optimizer (AdamW through moe_adamw_step)
    ADAPTERS = (("dA_gate", "A_gate"), ("dB_gate", "B_gate"), ("dA_up", "A_up"),
                ("dB_up", "B_up"), ("dA_down", "A_down"), ("dB_down", "B_down"))

    def init_optimizer(self):
        """float32 master copies of the six adapters and zero moments."""
        self.opt = {}
        for gname, pname in self.ADAPTERS:
            master = self.t[pname].float().contiguous()
            self.opt[pname] = (master, torch.zeros_like(master), torch.zeros_like(master))
        self.opt_step = 0

    def optimizer_step(self, lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0,
                       stream=None):
        """One AdamW step on every adapter; the act-dtype adapters that the
        forward reads are rewritten from the updated masters."""
        self.opt_step += 1
        h = B.adamw_hparams(lr, beta1, beta2, eps, weight_decay, self.opt_step)
        for gname, pname in self.ADAPTERS:
            master, m, v = self.opt[pname]
            B.moe_adamw_step(h, master, self.grads[gname], m, v, self.t[pname], stream)

    # ---- results on the host
    def routing(self) -> dict:
        out = {n: to_numpy(getattr(self, n)) for n in
               ("topk_idx", "gates", "counts", "offsets", "perm_src", "slot_pos")}
        if self.logits is not None:
            out["logits"] = to_numpy(self.logits)
        return out


def grow_inputs(t: dict, cfg, factor: int, noise=None, noise_scale: float = 0.0):
    """Few -> many growth of a layer's device tensors through moe_grow_copy /
    moe_grow_router: returns the grown config (E and k times `factor`) and
    tensors (expert e * factor + c is a copy of expert e; router copies c >= 1
    moved by noise_scale * noise, noise [d][E * factor] float32)."""
    out = {}
    for key, v in t.items():
        if v is not None and key.startswith(("q_", "s_", "A_", "B_")):
            dst = torch.empty((v.shape[0] * factor,) + tuple(v.shape[1:]), dtype=v.dtype,
                              device=v.device)
            B.moe_grow_copy(v, dst, v[0].numel() * v.element_size(), v.shape[0], factor)
            out[key] = dst
        else:
            out[key] = v
    w, b = t["w_router"], t.get("b_router")
    d, E = w.shape
    w_out = torch.empty((d, E * factor), dtype=torch.float32, device=w.device)
    b_out = torch.empty(E * factor, dtype=torch.float32, device=w.device) if b is not None else None
    z = to_device(noise, w.device) if noise is not None else None
    B.moe_grow_router(d, E, factor, w, b, z, float(noise_scale), w_out, b_out)
    out["w_router"], out["b_router"] = w_out, b_out
    return cfg.with_(E=E * factor, k=cfg.k * factor), out
