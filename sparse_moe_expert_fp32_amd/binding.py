"""ctypes binding of libmoe_tqp.so (see include/moe_tqp.h).

Argument marshalling only: torch tensors are passed by device pointer and the
current HIP stream; every step of the layer runs in the library's kernels.
Importing this module loads the library and raises if it was not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_tqp.so")

MOE_F32, MOE_BF16 = 0, 1
CALL_ROUTE, CALL_PERMUTE, CALL_EXPERT_FWD, CALL_COMBINE, CALL_ADAPTER_BWD = range(5)
# workspace flags OR-ed into a call id of moe_workspace_size
WS_SAVE_GIVEN, WS_PACKED_GIVEN = 0x100, 0x200
MAT_GATE_UP, MAT_DOWN = 0, 1


class MoeError(RuntimeError):
    pass


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group", ctypes.c_int32), ("act", ctypes.c_int32),
                ("lora_scale", ctypes.c_float), ("base_bits", ctypes.c_int32)]


class QLora(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("qt", ctypes.c_void_p),
                ("qf", ctypes.c_void_p)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is missing: build it with "
                       "`python -m sparse_moe_expert_fp32_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(Dims)
    sig = {
        "moe_route": [DP, P, P, P, P, P, P, P, SZ, P],
        "moe_permute": [DP, P, P, P, P, P, P, P, P, SZ, P],
        "moe_expert_fwd": [DP, P, P, P, QLora, QLora, QLora, P, P, P, SZ, P],
        "moe_expert_fwd_noalloc": [DP, P, P, P, QLora, QLora, QLora, P, P, P],
        "moe_combine": [DP, P, P, P, P, P, SZ, P],
        "moe_adapter_bwd": [DP, P, P, P, P, P, P, P, P, QLora, QLora, QLora, P, P, P,
                            P, P, P, P, P, P, P, SZ, P],
        "moe_workspace_size": [DP, I32, ctypes.POINTER(SZ)],
        "moe_save_size": [DP, ctypes.POINTER(SZ)],
        "moe_status_string": [I32],
        "moe_last_error": [],
        "moe_abi_version": [],
        "moe_timer_start": [I32],
        "moe_timer_stop": [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I32)],
        "moe_adamw_step": [ctypes.POINTER(AdamWHparams), ctypes.c_int64, P, P, P, P, P, I32, P],
        "moe_pack_base_t_size": [DP, ctypes.POINTER(SZ)],
        "moe_pack_base_t": [DP, I32, P, P, P, SZ, P],
        "moe_pack_base_f_size": [DP, ctypes.POINTER(SZ)],
        "moe_pack_base_f": [DP, I32, P, P, P, SZ, P],
        "moe_rev_couple": [DP, P, P, P, I32, P],
        "moe_grow_copy": [P, P, ctypes.c_int64, I32, I32, P],
        "moe_grow_router": [I32, I32, I32, P, P, P, ctypes.c_float, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I32
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()
EXPORTS = ("moe_route", "moe_permute", "moe_expert_fwd", "moe_expert_fwd_noalloc", "moe_combine",
           "moe_adapter_bwd",
           "moe_workspace_size", "moe_save_size", "moe_status_string", "moe_last_error",
           "moe_abi_version", "moe_timer_start", "moe_timer_stop", "moe_adamw_step",
           "moe_pack_base_t_size", "moe_pack_base_t", "moe_pack_base_f_size", "moe_pack_base_f",
           "moe_rev_couple", "moe_grow_copy", "moe_grow_router")

# kernel tags of moe_timer_start (moe_kernel_tag)
KT = {"router_logits": 0, "router_topk": 1, "permute": 2, "gateup": 3, "down": 4, "combine": 5,
      "gate_grad": 6, "bwd_down": 7, "bwd_gateup": 8}


def _check(status: int, name: str):
    if status != 0:
        raise MoeError(f"{name}: {LIB.moe_status_string(status).decode()}: "
                       f"{LIB.moe_last_error().decode()}")


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims(T, d, E, k, f, r, group, act, lora_scale=1.0, bits=4) -> Dims:
    a = {"f32": MOE_F32, "bf16": MOE_BF16}.get(act, act)
    return Dims(T, d, E, k, f, r, group, a, lora_scale, bits)


def dims_of(cfg, T: int | None = None) -> Dims:
    return dims(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.r, cfg.group,
                cfg.act, cfg.lora_scale, getattr(cfg, "bits", 4))


def qlora(q, scale, A, B, qt=None, qf=None) -> QLora:
    return QLora(_p(q), _p(scale), _p(A), _p(B), _p(qt), _p(qf))


def moe_workspace_size(dm: Dims, call: int) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.moe_workspace_size(ctypes.byref(dm), call, ctypes.byref(out)), "moe_workspace_size")
    return out.value


def moe_save_size(dm: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.moe_save_size(ctypes.byref(dm), ctypes.byref(out)), "moe_save_size")
    return out.value


def moe_abi_version() -> int:
    return LIB.moe_abi_version()


def moe_timer_start(tag) -> None:
    _check(LIB.moe_timer_start(KT.get(tag, tag)), "moe_timer_start")


def moe_timer_stop():
    ms, n = ctypes.c_float(0), ctypes.c_int32(0)
    _check(LIB.moe_timer_stop(ctypes.byref(ms), ctypes.byref(n)), "moe_timer_stop")
    return ms.value, n.value


def moe_route(dm, x, w_router, b_router, topk_idx, gates, logits, ws, stream=None):
    _check(LIB.moe_route(ctypes.byref(dm), _p(x), _p(w_router), _p(b_router), _p(topk_idx),
                         _p(gates), _p(logits), _p(ws), ws.numel() if ws is not None else 0,
                         _stream(stream)), "moe_route")


def moe_permute(dm, topk_idx, x, counts, offsets, perm_src, slot_pos, x_perm, ws, stream=None):
    _check(LIB.moe_permute(ctypes.byref(dm), _p(topk_idx), _p(x), _p(counts), _p(offsets),
                           _p(perm_src), _p(slot_pos), _p(x_perm), _p(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "moe_permute")


def moe_expert_fwd(dm, x, offsets, perm_src, gate, up, down, e_out, save, ws, stream=None):
    _check(LIB.moe_expert_fwd(ctypes.byref(dm), _p(x), _p(offsets), _p(perm_src), gate, up, down,
                              _p(e_out), _p(save), _p(ws), ws.numel() if ws is not None else 0,
                              _stream(stream)), "moe_expert_fwd")


def moe_expert_fwd_noalloc(dm, x, offsets, perm_src, gate, up, down, e_out, save, stream=None):
    _check(LIB.moe_expert_fwd_noalloc(ctypes.byref(dm), _p(x), _p(offsets), _p(perm_src), gate,
                                      up, down, _p(e_out), _p(save), _stream(stream)),
           "moe_expert_fwd_noalloc")


def moe_combine(dm, e_out, slot_pos, gates, y, ws=None, stream=None):
    _check(LIB.moe_combine(ctypes.byref(dm), _p(e_out), _p(slot_pos), _p(gates), _p(y), _p(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "moe_combine")


def moe_adapter_bwd(dm, dy, x, topk_idx, gates, offsets, perm_src, slot_pos, w_router, gate, up,
                    down, e_out, save, dx, dA_gate, dB_gate, dA_up, dB_up, dA_down, dB_down, ws,
                    stream=None):
    _check(LIB.moe_adapter_bwd(ctypes.byref(dm), _p(dy), _p(x), _p(topk_idx), _p(gates),
                               _p(offsets), _p(perm_src), _p(slot_pos), _p(w_router), gate, up,
                               down, _p(e_out), _p(save), _p(dx), _p(dA_gate), _p(dB_gate),
                               _p(dA_up), _p(dB_up), _p(dA_down), _p(dB_down), _p(ws),
                               ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_adapter_bwd")


def pack_base_supported(dm: Dims) -> bool:
    """Whether these dims have a packed transposed base (the matrix-core path)."""
    out = ctypes.c_size_t(0)
    return LIB.moe_pack_base_t_size(ctypes.byref(dm), ctypes.byref(out)) == 0


def moe_pack_base_t_size(dm: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.moe_pack_base_t_size(ctypes.byref(dm), ctypes.byref(out)), "moe_pack_base_t_size")
    return out.value


def moe_pack_base_t(dm: Dims, matrix: int, q, scale, packed, stream=None):
    _check(LIB.moe_pack_base_t(ctypes.byref(dm), matrix, _p(q), _p(scale), _p(packed),
                               packed.numel() if packed is not None else 0, _stream(stream)),
           "moe_pack_base_t")


def moe_rev_couple(dm: Dims, x, m, out, sign: int, stream=None):
    _check(LIB.moe_rev_couple(ctypes.byref(dm), _p(x), _p(m), _p(out), sign, _stream(stream)),
           "moe_rev_couple")


def moe_grow_copy(src, dst, block_bytes: int, n_experts: int, factor: int, stream=None):
    _check(LIB.moe_grow_copy(_p(src), _p(dst), block_bytes, n_experts, factor, _stream(stream)),
           "moe_grow_copy")


def moe_grow_router(d: int, n_experts: int, factor: int, w, b, noise, noise_scale: float,
                    w_out, b_out, stream=None):
    _check(LIB.moe_grow_router(d, n_experts, factor, _p(w), _p(b), _p(noise), noise_scale,
                               _p(w_out), _p(b_out), _stream(stream)), "moe_grow_router")


def moe_pack_base_f_size(dm: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.moe_pack_base_f_size(ctypes.byref(dm), ctypes.byref(out)), "moe_pack_base_f_size")
    return out.value


def moe_pack_base_f(dm: Dims, matrix: int, q, scale, packed, stream=None):
    _check(LIB.moe_pack_base_f(ctypes.byref(dm), matrix, _p(q), _p(scale), _p(packed),
                               packed.numel() if packed is not None else 0, _stream(stream)),
           "moe_pack_base_f")


def adamw_hparams(lr, beta1, beta2, eps, weight_decay, step) -> AdamWHparams:
    return AdamWHparams(lr, beta1, beta2, eps, weight_decay, step)


def moe_adamw_step(h: AdamWHparams, master, grad, m, v, param=None, stream=None):
    if param is None:
        pdt = MOE_F32
    else:
        pdt = MOE_BF16 if param.dtype == torch.bfloat16 else MOE_F32
    n = master.numel()
    _check(LIB.moe_adamw_step(ctypes.byref(h), n, _p(master), _p(grad), _p(m), _p(v), _p(param),
                              pdt, _stream(stream)), "moe_adamw_step")
