"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects bad arguments with the
documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_tqp.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*|int32_t)\s*(moe_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def B():
    from sparse_moe_expert_fp32_amd import binding
    return binding


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for name in ("moe_route", "moe_permute", "moe_expert_fwd", "moe_combine", "moe_adapter_bwd"):
        assert name in fns


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(B.EXPORTS)
    assert B.moe_abi_version() == 4
    import __graft_entry__
    assert __graft_entry__.header_abi_version() == B.moe_abi_version()


def good(B, **kw):
    base = dict(T=64, d=128, E=8, k=2, f=256, r=4, group=32, act="f32")
    base.update(kw)
    return B.dims(**base)


def test_workspace_and_save_sizes(B):
    dm = good(B)
    for c in range(5):
        assert B.moe_workspace_size(dm, c) >= 0
    assert B.moe_save_size(dm) > 0
    big = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    assert B.moe_save_size(big) >= 8192 * 12 * 768 * 2 * 3


def test_workspace_flags_shrink_and_validate(B):
    """A caller that supplies the save buffer and the packed bases needs less
    workspace (the 8K shape: without the save region and the ratio tables in
    the forward, without the transposed-base slots in the backward); unknown
    flag bits are rejected."""
    big = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    fw = B.moe_workspace_size(big, B.CALL_EXPERT_FWD)
    fw_s = B.moe_workspace_size(big, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN)
    fw_sp = B.moe_workspace_size(big, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN | B.WS_PACKED_GIVEN)
    assert fw - fw_s >= B.moe_save_size(big)
    assert fw_s - fw_sp >= 3 * 460 * 768 * 16 * 4
    assert fw_sp < 16 << 20
    bw = B.moe_workspace_size(big, B.CALL_ADAPTER_BWD)
    bw_p = B.moe_workspace_size(big, B.CALL_ADAPTER_BWD | B.WS_PACKED_GIVEN)
    assert bw - bw_p >= 2 * (460 * 2048 * 768 // 2)
    out = ctypes.c_size_t(7)
    assert B.LIB.moe_workspace_size(ctypes.byref(big), B.CALL_EXPERT_FWD | 0x400,
                                    ctypes.byref(out)) == -1
    assert out.value == 7


def test_int8_base_sizes_and_validation(B):
    """An int8 base ("Int8 or Int4") doubles the packed base sizes (its two
    int4 planes), the forward workspace holds the planes when the caller does
    not pack them, and a base width other than 4 or 8 is unsupported."""
    i4 = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    i8 = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16", bits=8)
    assert B.moe_pack_base_f_size(i8) == 2 * B.moe_pack_base_f_size(i4)
    assert B.moe_pack_base_t_size(i8) == 2 * B.moe_pack_base_t_size(i4)
    f8 = B.moe_workspace_size(i8, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN)
    assert f8 >= 3 * B.moe_pack_base_f_size(i8)
    f8p = B.moe_workspace_size(i8, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN | B.WS_PACKED_GIVEN)
    f4p = B.moe_workspace_size(i4, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN | B.WS_PACKED_GIVEN)
    assert f8p > f4p and f8p < 16 << 20     # only the doubled start-value tables
    for bad in (1, 5, 16, -4):
        dm = B.dims(64, 128, 8, 2, 256, 4, 32, "f32", bits=bad)
        out = ctypes.c_size_t(7)
        assert B.LIB.moe_workspace_size(ctypes.byref(dm), 0, ctypes.byref(out)) == -2
        assert out.value == 7
    assert B.moe_workspace_size(B.dims(64, 128, 8, 2, 256, 4, 32, "f32", bits=0), 0) >= 0


def test_noalloc_forward_rejects_before_any_hip_call(B):
    """moe_expert_fwd_noalloc validates like moe_expert_fwd and refuses,
    with MOE_ERR_WORKSPACE and before touching the GPU, a call whose scratch
    would exceed its fixed 64 MiB (the 8K shape without a save buffer)."""
    big = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    P = 0x10000
    q = B.QLora(P, P, P, P, None, None)
    f = B.LIB.moe_expert_fwd_noalloc
    assert f(ctypes.byref(big), P, P, P, q, q, q, P, None, None) == -3
    assert "64" in B.LIB.moe_last_error().decode() or "67108864" in B.LIB.moe_last_error().decode()
    assert f(ctypes.byref(big), None, P, P, q, q, q, P, P, None) == -1
    bad = B.QLora(P, None, P, P, None, None)
    assert f(ctypes.byref(big), P, P, P, bad, q, q, P, P, None) == -1
    need = B.moe_workspace_size(big, B.CALL_EXPERT_FWD | B.WS_SAVE_GIVEN | B.WS_PACKED_GIVEN)
    assert need < 64 << 20


BAD = [
    (dict(T=0), -1), (dict(E=0), -1), (dict(E=1025), -1), (dict(k=0), -1), (dict(k=9), -1),
    (dict(E=64, k=33), -1), (dict(r=0), -1), (dict(r=33), -1), (dict(group=16), -2),
    (dict(group=48), -2), (dict(act=7), -2), (dict(d=80), -1), (dict(f=200), -1),
    (dict(T=1 << 24, k=8, E=16), -1), (dict(d=0), -1),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_invalid_dims_rejected(B, kw, code):
    dm = good(B, **kw)
    out = ctypes.c_size_t(12345)
    st = B.LIB.moe_workspace_size(ctypes.byref(dm), 0, ctypes.byref(out))
    assert st == code
    assert out.value == 12345                       # nothing written
    assert B.LIB.moe_last_error().decode()


def test_nonfinite_scale_rejected(B):
    dm = good(B, lora_scale=float("nan"))
    assert B.LIB.moe_save_size(ctypes.byref(dm), ctypes.byref(ctypes.c_size_t())) == -1


FAKE = 0x1000  # never dereferenced: validation fails before any HIP call


def test_null_pointers_rejected_before_launch(B):
    dm = good(B)
    L = B.LIB
    P = FAKE
    q = B.QLora(P, P, P, P)
    qnull = B.QLora(P, None, P, P)
    assert L.moe_route(ctypes.byref(dm), None, P, None, P, P, None, P, 1 << 30, None) == -1
    assert L.moe_permute(ctypes.byref(dm), P, None, P, P, None, P, None, P, 1 << 30, None) == -1
    assert L.moe_permute(ctypes.byref(dm), P, None, P, P, P, P, P, P, 1 << 30, None) == -1
    assert L.moe_expert_fwd(ctypes.byref(dm), P, P, P, q, qnull, q, P, None, P, 1 << 30,
                            None) == -1
    assert "up" in L.moe_last_error().decode()
    assert L.moe_combine(ctypes.byref(dm), P, None, P, P, None, 0, None) == -1
    assert L.moe_adapter_bwd(ctypes.byref(dm), P, P, P, P, P, P, P, P, q, q, q, P, None, P,
                             P, P, P, P, P, P, P, 1 << 30, None) == -1
    assert L.moe_route(None, P, P, None, P, P, None, P, 1 << 30, None) == -1


def test_unaligned_expert_fwd_buffers_rejected(B):
    """x, e_out and save are read and written in 16-byte pieces: a pointer
    off a 16-byte boundary is refused on the host, before any launch."""
    dm = good(B)
    L = B.LIB
    P = FAKE
    q = B.QLora(P, P, P, P)
    for x, e_out, save in ((P + 8, P, None), (P, P + 2, None), (P, P, P + 4)):
        assert L.moe_expert_fwd(ctypes.byref(dm), x, P, P, q, q, q, e_out, save, P, 1 << 30,
                                None) == -1
        assert "16-byte" in L.moe_last_error().decode()
        assert L.moe_expert_fwd_noalloc(ctypes.byref(dm), x, P, P, q, q, q, e_out, save,
                                        None) == -1


def test_unaligned_adapter_or_base_rejected(B):
    """q, A and B are streamed in 16-byte pieces: each must be 16-byte
    aligned, in the forward and in the backward."""
    dm = good(B)
    L = B.LIB
    P = FAKE
    q = B.QLora(P, P, P, P)
    for bad in (B.QLora(P + 4, P, P, P), B.QLora(P, P, P + 2, P), B.QLora(P, P, P, P + 8)):
        assert L.moe_expert_fwd(ctypes.byref(dm), P, P, P, q, bad, q, P, None, P, 1 << 30,
                                None) == -1
        assert "16-byte" in L.moe_last_error().decode()
        assert L.moe_adapter_bwd(ctypes.byref(dm), P, P, P, P, P, P, P, P, q, q, bad, P, P, P,
                                 P, P, P, P, P, P, P, 1 << 30, None) == -1
        assert "16-byte" in L.moe_last_error().decode()


def test_small_workspace_rejected(B):
    dm = good(B)
    L = B.LIB
    P = FAKE
    need = B.moe_workspace_size(dm, B.CALL_ROUTE)
    assert need > 0
    assert L.moe_route(ctypes.byref(dm), P, P, None, P, P, None, P, need - 1, None) == -3
    assert L.moe_route(ctypes.byref(dm), P, P, None, P, P, None, None, need, None) == -3
    q = B.QLora(P, P, P, P)
    need = B.moe_workspace_size(dm, B.CALL_EXPERT_FWD)
    assert L.moe_expert_fwd(ctypes.byref(dm), P, P, P, q, q, q, P, None, P, need - 1, None) == -3
    assert "workspace" in L.moe_last_error().decode()


def test_status_strings(B):
    assert B.LIB.moe_status_string(0) == b"MOE_OK"
    assert B.LIB.moe_status_string(-3) == b"MOE_ERR_WORKSPACE"
    assert B.LIB.moe_status_string(-99) == b"MOE_ERR_UNKNOWN"


# ---- adapter optimizer step: host-side validation (nothing reaches the GPU)

def adamw_call(B, n=16, ptrs=(0x1000, 0x2000, 0x3000, 0x4000), param=None, pdt=0, **kw):
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    hp.update(kw)
    h = B.adamw_hparams(**hp)
    return B.LIB.moe_adamw_step(ctypes.byref(h), n, *ptrs, param, pdt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(step=0), -1), (dict(beta1=1.0), -1), (dict(beta2=-0.1), -1), (dict(eps=0.0), -1),
    (dict(eps=float("nan")), -1), (dict(lr=float("inf")), -1),
    (dict(weight_decay=float("nan")), -1), (dict(n=-1), -1),
    (dict(ptrs=(None, 0x2000, 0x3000, 0x4000)), -1),
    (dict(ptrs=(0x1000, 0x1000, 0x3000, 0x4000)), -1),
    (dict(ptrs=(0x1000, 0x2000, 0x3000, 0x3000)), -1),
    (dict(param=0x5000, pdt=7), -2),
])
def test_adamw_rejects_bad_arguments(B, kw, status):
    assert adamw_call(B, **kw) == status
    assert B.LIB.moe_last_error().decode().startswith("moe_adamw_step")


def test_adamw_empty_tensor_is_a_no_op(B):
    assert adamw_call(B, n=0, ptrs=(None, None, None, None)) == 0


# ---- packed transposed base: host-side validation

def test_pack_size_and_support(B):
    big = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    E, d, f = 460, 2048, 768
    assert B.moe_pack_base_t_size(big) == E * d * f // 2 + E * d * f // 128 * 4
    assert B.pack_base_supported(big)
    for dm in (good(B), good(B, act="bf16"), B.dims(64, 192, 8, 2, 256, 4, 64, "bf16")):
        out = ctypes.c_size_t(7)
        assert B.LIB.moe_pack_base_t_size(ctypes.byref(dm), ctypes.byref(out)) == -2
        assert out.value == 7
        assert not B.pack_base_supported(dm)


@pytest.mark.parametrize("matrix,q,s,packed,nbytes,status", [
    (2, FAKE, FAKE, FAKE, 1 << 40, -1),          # no such matrix
    (0, None, FAKE, FAKE, 1 << 40, -1),          # null q
    (1, FAKE, FAKE, None, 1 << 40, -1),          # null output
    (0, FAKE, FAKE, FAKE + 8, 1 << 40, -1),      # misaligned output
    (0, FAKE, FAKE, FAKE, 1024, -3),             # output too small
])
def test_pack_rejects_bad_arguments(B, matrix, q, s, packed, nbytes, status):
    dm = B.dims(256, 256, 8, 2, 128, 16, 128, "bf16")
    assert B.LIB.moe_pack_base_t(ctypes.byref(dm), matrix, q, s, packed, nbytes, None) == status
    assert B.LIB.moe_last_error().decode()


def test_misaligned_packed_base_rejected(B):
    dm = B.dims(256, 256, 8, 2, 128, 16, 128, "bf16")
    P = FAKE
    q, qbad = B.QLora(P, P, P, P, P), B.QLora(P, P, P, P, P + 4)
    assert B.LIB.moe_adapter_bwd(ctypes.byref(dm), P, P, P, P, P, P, P, P, q, qbad, q, P, P, P,
                                 P, P, P, P, P, P, P, 1 << 40, None) == -1
    assert "qt" in B.LIB.moe_last_error().decode()


# ---- stage-major packed base for the forward: host-side validation

def test_pack_f_size_and_support(B):
    big = B.dims(8192, 2048, 460, 12, 768, 16, 128, "bf16")
    assert B.moe_pack_base_f_size(big) == 460 * 2048 * 768 // 2 + 460 * 2048 * 768 // 128 * 4
    for dm in (good(B), good(B, act="bf16"), B.dims(64, 192, 8, 2, 256, 4, 64, "bf16")):
        out = ctypes.c_size_t(7)
        assert B.LIB.moe_pack_base_f_size(ctypes.byref(dm), ctypes.byref(out)) == -2
        assert out.value == 7


@pytest.mark.parametrize("matrix,q,s,packed,nbytes,status", [
    (2, FAKE, FAKE, 1 << 32, 1 << 40, -1),          # no such matrix
    (0, None, FAKE, 1 << 32, 1 << 40, -1),          # null q
    (0, FAKE, None, 1 << 32, 1 << 40, -1),          # null scale
    (1, FAKE, FAKE, None, 1 << 40, -1),             # null output
    (0, FAKE, FAKE, (1 << 32) + 8, 1 << 40, -1),    # misaligned output
    (0, FAKE + 4, FAKE, 1 << 32, 1 << 40, -1),      # misaligned q
    (0, FAKE, FAKE, FAKE + 64, 1 << 40, -1),        # output overlaps q
    (0, FAKE, FAKE, 1 << 32, 1024, -3),             # output too small
])
def test_pack_f_rejects_bad_arguments(B, matrix, q, s, packed, nbytes, status):
    dm = B.dims(256, 256, 8, 2, 128, 16, 128, "bf16")
    assert B.LIB.moe_pack_base_f(ctypes.byref(dm), matrix, q, s, packed, nbytes, None) == status
    assert B.LIB.moe_last_error().decode().startswith("moe_pack_base_f")


def test_misaligned_forward_packed_base_rejected(B):
    dm = B.dims(256, 256, 8, 2, 128, 16, 128, "bf16")
    P = FAKE
    q, qbad = B.QLora(P, P, P, P), B.QLora(P, P, P, P, None, P + 8)
    need = B.moe_workspace_size(dm, B.CALL_EXPERT_FWD)
    assert B.LIB.moe_expert_fwd(ctypes.byref(dm), P, P, P, q, qbad, q, P, P, P, need,
                                None) == -1
    assert "qf" in B.LIB.moe_last_error().decode()


# ---- reversible coupling: host-side validation

@pytest.mark.parametrize("x,m,out,sign", [
    (None, FAKE, FAKE + 4096, 1), (FAKE, None, FAKE + 4096, 1), (FAKE, FAKE + 64, None, 1),
    (FAKE, FAKE + 64, FAKE + 4096, 0), (FAKE, FAKE + 64, FAKE + 4096, 2),
    (FAKE, FAKE + 64, FAKE + 64, -1),    # out aliases m
])
def test_rev_couple_rejects_bad_arguments(B, x, m, out, sign):
    dm = good(B)
    assert B.LIB.moe_rev_couple(ctypes.byref(dm), x, m, out, sign, None) == -1
    assert B.LIB.moe_last_error().decode().startswith("moe_rev_couple")


# ---- expert growth: host-side validation

@pytest.mark.parametrize("src,dst,nb,E,F", [
    (None, 1 << 32, 64, 4, 2), (FAKE, None, 64, 4, 2), (FAKE, 1 << 32, 0, 4, 2),
    (FAKE, 1 << 32, 64, 0, 2), (FAKE, 1 << 32, 64, 4, 0), (FAKE, 1 << 32, 64, 600, 2),
    (FAKE, FAKE + 64, 64, 4, 2),          # dst overlaps src
])
def test_grow_copy_rejects_bad_arguments(B, src, dst, nb, E, F):
    assert B.LIB.moe_grow_copy(src, dst, nb, E, F, None) == -1
    assert B.LIB.moe_last_error().decode().startswith("moe_grow_copy")


@pytest.mark.parametrize("d,E,F,w,b,wo,bo,s", [
    (64, 8, 2, None, None, FAKE, None, 0.0), (64, 8, 2, FAKE, None, None, None, 0.0),
    (64, 8, 2, FAKE, FAKE, FAKE, None, 0.0), (0, 8, 2, FAKE, None, FAKE, None, 0.0),
    (64, 8, 200, FAKE, None, FAKE, None, 0.0), (64, 8, 2, FAKE, None, FAKE, None, float("nan")),
])
def test_grow_router_rejects_bad_arguments(B, d, E, F, w, b, wo, bo, s):
    assert B.LIB.moe_grow_router(d, E, F, w, b, None, s, wo, bo, None) == -1
    assert B.LIB.moe_last_error().decode().startswith("moe_grow_router")
