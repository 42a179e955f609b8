"""Plain fp64 CPU oracle of the TQP routed-expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: it exists so that tests, the package smoke check and the benchmark's
CPU baseline can compare the HIP library against an obviously correct
definition.  It imports nothing from the HIP library or its binding and shares
no helper with them; the only thing both sides see is the input tensors.

What is computed (cited by page title and section):
  * "Reversible Sparse MoE Single Node" (skill card), Principle 3 "TQP
    Optimizer Strategy" and Implementation Considerations "TQP Quantization":
    expert base weights are quantized and fixed, low-rank adapters are full
    precision and trained, the router is full precision.  So every expert
    matrix is W_eff = dequant(q, s) + lam * B @ A, the base receives no
    gradient and the adapters do.
  * Same card, Architecture Details, and the abstract of "Reversible
    Foundations: Training a 120B Sparse MoE through State-Preserving Scaling":
    routed experts with top-k routing (460 experts, top-12 at the largest
    stage).
  * Same card, Implementation Considerations "Reversibility": routing is a
    stateless function of the layer input.
  * Same card, Related Methods: LoRA, i.e. the adapter product of a row with
    two low-rank factors; stored out x in here (A [r, K], B [N, r]).
Readings where the pages are silent (each is listed with its reason in the
design notes of the repository): symmetric int4 (or int8) with bf16 group scales; top-k
over the logits with ties to the lower expert index; gates = softmax over the
selected logits (= softmax over all experts renormalised over the selected);
dropless routing; SwiGLU experts without biases, silu(z) = z / (1 + e^-z);
LoRA on gate, up and down; loss L = sum_t <dY_t, y_t>; the top-k choice is
held constant in the backward and the router receives no weight gradient but
does pass gradient to x through the gates.

Everything is evaluated in float64 from the exact stored inputs: bf16 bit
patterns and float32 values convert to float64 exactly, int4 nibbles and
int8 bytes become integers and bf16 scales become float64.  Parity pins for every function are
in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------- storage --


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor: uint16 arrays are bf16 bit
    patterns, float32 arrays are float32 values."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def unpack_int4(q_packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> int64 [..., K] signed values.

    Word layout: every aligned 32-bit little-endian word covers an 8-wide
    block of K; nibble slot j (bits 4j..4j+3) holds element 2j for j < 4 and
    element 2(j-4)+1 for j >= 4; nibbles are two's complement."""
    q_packed = np.ascontiguousarray(q_packed, dtype=np.uint8)
    lead = q_packed.shape[:-1]
    words = q_packed.reshape(lead + (q_packed.shape[-1] // 4, 4)).astype(np.int64)
    word = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    out = np.empty(lead + (word.shape[-1], 8), dtype=np.int64)
    for slot in range(8):
        nib = (word >> (4 * slot)) & 0xF
        val = np.where(nib >= 8, nib - 16, nib)
        elem = 2 * slot if slot < 4 else 2 * (slot - 4) + 1
        out[..., elem] = val
    return out.reshape(lead + (word.shape[-1] * 8,))


def unpack_int8(q_bytes: np.ndarray) -> np.ndarray:
    """uint8 [..., K] -> int64 [..., K]: each byte is one two's-complement
    value, in k order."""
    return np.ascontiguousarray(q_bytes, dtype=np.uint8).view(np.int8).astype(np.int64)


def dequantize(q_packed: np.ndarray, scale_bits: np.ndarray, group: int) -> np.ndarray:
    """W_hat[n, c] = s[n, c // group] * q[n, c]  (float64, exact).

    The storage width follows from the shapes: with K = (scale columns) *
    group, q holds K bytes per row for int8 and K/2 for int4 ("Int8 or Int4",
    skill card "Reversible Sparse MoE Single Node", Implementation
    Considerations, TQP Quantization)."""
    K = scale_bits.shape[-1] * group
    if q_packed.shape[-1] == K:
        q = unpack_int8(q_packed)
    elif 2 * q_packed.shape[-1] == K:
        q = unpack_int4(q_packed)
    else:
        raise ValueError("q holds neither K int8 nor K/2 int4 bytes per row")
    s = to_f64(scale_bits)
    return q * np.repeat(s, group, axis=-1)


# --------------------------------------------------------------- routing --


def router_logits(x, w_router, b_router=None) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] W_r[c, e] + b[e]  (full-precision router)."""
    l = to_f64(x) @ to_f64(w_router)
    if b_router is not None:
        l = l + to_f64(b_router)[None, :]
    return l


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """First k experts of each row under the order (logit descending, expert
    index ascending); returned in that order, int32 [T, k]."""
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    experts = np.arange(E)
    for t in range(T):
        order = np.lexsort((experts, -logits[t]))
        idx[t] = order[:k]
    return idx


def gates(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """gamma[t, j] = exp(l[t, S_j]) / sum_i exp(l[t, S_i]) over the selected
    experts S (computed relative to the largest selected logit)."""
    sel = np.take_along_axis(logits, topk_idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def near_ties(logits: np.ndarray, k: int, thr: float = 1e-5):
    """(boundary, order) boolean masks per token.  boundary: the k-th and
    (k+1)-th largest logits differ by less than thr, so the selected set can
    legitimately differ between precisions.  order: two adjacent selected
    logits differ by less than thr, so their slot order can differ."""
    srt = -np.sort(-logits, axis=1)
    T, E = logits.shape
    boundary = np.zeros(T, bool)
    if k < E:
        boundary = (srt[:, k - 1] - srt[:, k]) < thr
    order = np.zeros(T, bool)
    if k > 1:
        order = (np.diff(-srt[:, :k], axis=1) < thr).any(axis=1)
    return boundary, order


# ----------------------------------------------------------- permutation --


def permutation(topk_idx: np.ndarray, E: int):
    """Expert-contiguous placement of the T*k routed slots, stable in token
    order: counts[e], offsets[e] (exclusive scan, offsets[E] = T*k),
    perm_src[p] = t*k + j and slot_pos[t*k + j] = p."""
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    perm_src = np.empty(T * k, dtype=np.int64)
    slot_pos = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = flat[t * k + j]
            p = cursor[e]
            cursor[e] += 1
            perm_src[p] = t * k + j
            slot_pos[t * k + j] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm_src.astype(np.int32), slot_pos.astype(np.int32))


# ---------------------------------------------------------------- experts --


def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


class Expert:
    """Float64 view of one expert's frozen base and adapters."""

    def __init__(self, inputs: dict, e: int, group: int):
        self.e = e
        self.W = {m: dequantize(inputs[f"q_{m}"][e], inputs[f"s_{m}"][e], group)
                  for m in ("gate", "up", "down")}
        self.A = {m: to_f64(inputs[f"A_{m}"][e]) for m in ("gate", "up", "down")}
        self.B = {m: to_f64(inputs[f"B_{m}"][e]) for m in ("gate", "up", "down")}


def expert_forward(ex: Expert, X: np.ndarray, lam: float) -> dict:
    """SwiGLU expert with adapters on every matrix, rows X [M, d].  Adapters
    are stored out x in like the base (A [r, K], B [N, r]), so the adapted
    matrix is W_hat + lam * B A and its product with a row is
    x W_hat^T + lam (x A^T) B^T:
    G = X W_g^T + lam (X A_g^T) B_g^T, U likewise, H = silu(G) * U,
    O = H W_d^T + lam (H A_d^T) B_d^T."""
    Zg = X @ ex.A["gate"].T
    Zu = X @ ex.A["up"].T
    G = X @ ex.W["gate"].T + lam * (Zg @ ex.B["gate"].T)
    U = X @ ex.W["up"].T + lam * (Zu @ ex.B["up"].T)
    H = silu(G) * U
    Zd = H @ ex.A["down"].T
    O = H @ ex.W["down"].T + lam * (Zd @ ex.B["down"].T)
    return {"G": G, "U": U, "H": H, "O": O, "Zg": Zg, "Zu": Zu, "Zd": Zd}


def expert_backward(ex: Expert, X: np.ndarray, fw: dict, dO: np.ndarray, lam: float) -> dict:
    """Adapter-only backward of expert_forward for upstream dO [M, d]:
    gradients of A and B of each matrix, and dX [M, d].  The base is frozen,
    so no gradient of W is formed."""
    G, U, H = fw["G"], fw["U"], fw["H"]
    dB_down = lam * dO.T @ fw["Zd"]
    dZd = lam * dO @ ex.B["down"]
    dA_down = dZd.T @ H
    dH = dO @ ex.W["down"] + dZd @ ex.A["down"]
    sg = sigmoid(G)
    dG = dH * U * sg * (1.0 + G * (1.0 - sg))
    dU = dH * G * sg
    dB_gate = lam * dG.T @ fw["Zg"]
    dB_up = lam * dU.T @ fw["Zu"]
    dZg = lam * dG @ ex.B["gate"]
    dZu = lam * dU @ ex.B["up"]
    dA_gate = dZg.T @ X
    dA_up = dZu.T @ X
    dX = (dG @ ex.W["gate"] + dU @ ex.W["up"]
          + dZg @ ex.A["gate"] + dZu @ ex.A["up"])
    return {"dA_gate": dA_gate, "dB_gate": dB_gate, "dA_up": dA_up, "dB_up": dB_up,
            "dA_down": dA_down, "dB_down": dB_down, "dX": dX}


# ------------------------------------------------------------ whole layer --


def route(inputs: dict, k: int, topk_idx: np.ndarray | None = None) -> dict:
    """Logits, selection, gates and permutation.  A caller may pass the
    selection to evaluate the layer on a given routing."""
    l = router_logits(inputs["x"], inputs["w_router"], inputs.get("b_router"))
    idx = topk(l, k) if topk_idx is None else np.asarray(topk_idx, np.int32)
    E = l.shape[1]
    counts, offsets, perm_src, slot_pos = permutation(idx, E)
    return {"logits": l, "topk_idx": idx, "gates": gates(l, idx), "counts": counts,
            "offsets": offsets, "perm_src": perm_src, "slot_pos": slot_pos}


def expert_rows(inputs: dict, R: dict, e: int, k: int, group: int, lam: float = 1.0,
                backward: bool = False, fw: dict | None = None) -> dict:
    """Expert e over its segment of the permutation R (as from route()): the
    forward of its rows ("fw", with the outputs "O") and, with backward, the
    adapter-only backward for the upstream gradient of those rows,
    dO[p] = gamma[t(p), j(p)] dY[t(p)]: the six adapter gradients and "dX".
    A saved forward may be passed as fw."""
    lo, hi = R["offsets"][e], R["offsets"][e + 1]
    src = R["perm_src"][lo:hi]
    rows, js = src // k, src % k
    ex = Expert(inputs, e, group)
    X = to_f64(inputs["x"][rows])
    if fw is None:
        fw = expert_forward(ex, X, lam)
    out = {"fw": fw, "O": fw["O"]}
    if backward:
        dO = R["gates"][rows, js][:, None] * to_f64(inputs["dy"][rows])
        out.update(expert_backward(ex, X, fw, dO, lam))
    return out


def combine(gam: np.ndarray, O: np.ndarray, slot_pos: np.ndarray) -> np.ndarray:
    """y[t] = sum_j gamma[t, j] O[slot_pos[t k + j]], j ascending."""
    T, k = gam.shape
    slot = np.asarray(slot_pos).reshape(T, k)
    y = np.zeros((T, O.shape[1]))
    for j in range(k):
        y += gam[:, j:j + 1] * O[slot[:, j]]
    return y


def gate_backward(dy, O: np.ndarray, gam: np.ndarray, topk_idx: np.ndarray,
                  slot_pos: np.ndarray, w_router) -> tuple:
    """The gate path of the backward with the selection held fixed:
    dgamma[t, j] = <dY_t, O_(t,j)>, the softmax over the selected logits
    dl = gamma (dgamma - <gamma, dgamma>), and the router-input gradient
    dx_r[t] = sum_j dl[t, j] W_r[:, e(t, j)] (the router itself is frozen)."""
    dy = to_f64(dy)
    wr = to_f64(w_router)
    T, k = gam.shape
    slot = np.asarray(slot_pos).reshape(T, k)
    dgam = np.einsum("td,tjd->tj", dy, O[slot])
    dl = gam * (dgam - (gam * dgam).sum(axis=1, keepdims=True))
    dx_r = np.zeros(dy.shape)
    for j in range(k):
        dx_r += dl[:, j:j + 1] * wr[:, topk_idx[:, j]].T
    return dgam, dl, dx_r


def forward(inputs: dict, k: int, group: int, lam: float = 1.0,
            topk_idx: np.ndarray | None = None, keep: bool = False) -> dict:
    """y[t] = sum_j gamma[t, j] * O_{e(t,j)}(x_t), j ascending."""
    R = route(inputs, k, topk_idx)
    T, d = inputs["x"].shape
    E = R["logits"].shape[1]
    O = np.zeros((T * k, d))
    saved = {}
    for e in range(E):
        lo, hi = R["offsets"][e], R["offsets"][e + 1]
        if hi == lo:
            continue
        res = expert_rows(inputs, R, e, k, group, lam)
        O[lo:hi] = res["O"]
        if keep:
            saved[e] = res["fw"]
    out = dict(R)
    out.update({"e_out": O, "y": combine(R["gates"], O, R["slot_pos"])})
    if keep:
        out["saved"] = saved
    return out


ADAPTER_GRADS = ("dA_gate", "dB_gate", "dA_up", "dB_up", "dA_down", "dB_down")


def adapter_grad_shapes(inputs: dict) -> dict:
    E, f, d = inputs["q_gate"].shape[0], inputs["q_gate"].shape[1], inputs["q_down"].shape[1]
    r = inputs["A_gate"].shape[1]
    return {"dA_gate": (E, r, d), "dB_gate": (E, f, r), "dA_up": (E, r, d), "dB_up": (E, f, r),
            "dA_down": (E, r, f), "dB_down": (E, d, r)}


def backward(inputs: dict, fwd: dict, k: int, group: int, lam: float = 1.0) -> dict:
    """Gradients of L = sum_t <dY_t, y_t> with the top-k choice held fixed:
    dX (through the experts and through the gates into the router input) and
    the six adapter gradients per expert.  The router and base are frozen."""
    T, d = inputs["x"].shape
    E = inputs["w_router"].shape[1]
    slot = fwd["slot_pos"].reshape(T, k)
    dgam, dl, dx_r = gate_backward(inputs["dy"], fwd["e_out"], fwd["gates"], fwd["topk_idx"],
                                   fwd["slot_pos"], inputs["w_router"])
    grads = {n: np.zeros(shape) for n, shape in adapter_grad_shapes(inputs).items()}
    dXp = np.zeros((T * k, d))
    for e in range(E):
        lo, hi = fwd["offsets"][e], fwd["offsets"][e + 1]
        if hi == lo:
            continue
        res = expert_rows(inputs, fwd, e, k, group, lam, backward=True,
                          fw=fwd.get("saved", {}).get(e))
        for name in grads:
            grads[name][e] = res[name]
        dXp[lo:hi] = res["dX"]
    dx = dx_r.copy()
    for j in range(k):
        dx += dXp[slot[:, j]]
    out = {"dx": dx, "dx_router": dx_r, "dgates": dgam, "dlogits_sel": dl}
    out.update(grads)
    return out


# ------------------------------------------------- sampled evaluation --
# The same definitions evaluated on a subset, for shapes where the whole
# layer is too slow on the CPU: outputs of chosen tokens and gradients of
# chosen experts are exact functions of their own rows.


def forward_tokens(inputs: dict, tokens, k: int, group: int, lam: float = 1.0,
                   topk_idx: np.ndarray | None = None, cache: dict | None = None) -> dict:
    """Routing and y for the listed tokens only (topk_idx, if given, holds the
    selection of those tokens, one row each)."""
    tokens = np.asarray(tokens)
    x = to_f64(inputs["x"][tokens])
    l = router_logits(inputs["x"][tokens], inputs["w_router"], inputs.get("b_router"))
    idx = topk(l, k) if topk_idx is None else np.asarray(topk_idx, np.int32)
    gam = gates(l, idx)
    cache = {} if cache is None else cache
    y = np.zeros_like(x)
    O = np.zeros((len(tokens), k, x.shape[1]))
    for i in range(len(tokens)):
        for j in range(k):
            e = int(idx[i, j])
            if e not in cache:
                cache[e] = Expert(inputs, e, group)
            O[i, j] = expert_forward(cache[e], x[i:i + 1], lam)["O"][0]
            y[i] += gam[i, j] * O[i, j]
    return {"logits": l, "topk_idx": idx, "gates": gam, "O": O, "y": y}


def backward_tokens(inputs: dict, tokens, k: int, group: int, lam: float = 1.0,
                    topk_idx: np.ndarray | None = None, cache: dict | None = None) -> np.ndarray:
    """dX rows of the listed tokens (each is a function of that token alone)."""
    tokens = np.asarray(tokens)
    fw = forward_tokens(inputs, tokens, k, group, lam, topk_idx, cache)
    cache = {} if cache is None else cache
    x = to_f64(inputs["x"][tokens])
    dy = to_f64(inputs["dy"][tokens])
    wr = to_f64(inputs["w_router"])
    idx, gam, O = fw["topk_idx"], fw["gates"], fw["O"]
    dgam = np.einsum("id,ijd->ij", dy, O)
    dl = gam * (dgam - (gam * dgam).sum(axis=1, keepdims=True))
    dx = np.zeros_like(x)
    for i in range(len(tokens)):
        for j in range(k):
            e = int(idx[i, j])
            ex = cache.setdefault(e, Expert(inputs, e, group))
            dx[i] += dl[i, j] * wr[:, e]
            f1 = expert_forward(ex, x[i:i + 1], lam)
            g = expert_backward(ex, x[i:i + 1], f1, gam[i, j] * dy[i:i + 1], lam)
            dx[i] += g["dX"][0]
    return dx


def expert_grads(inputs: dict, R: dict, e: int, k: int, group: int, lam: float = 1.0) -> dict:
    """The six adapter gradients (and dX rows) of expert e given the full
    routing R (as returned by route())."""
    return expert_rows(inputs, R, e, k, group, lam, backward=True)


# --------------------------------------------------- adapter optimizer step --
# "Reversible Sparse MoE Single Node" (skill card), Principle 3 "TQP Optimizer
# Strategy" and Pattern 3: the optimizer state lives on the low-rank adapters
# only (the quantized base is fixed).  The pages do not name the optimizer;
# the reading taken here is AdamW as published ("Decoupled Weight Decay
# Regularization", Loshchilov and Hutter, over Adam of Kingma and Ba): float32
# master parameters with two float32 moments, bias-corrected moments, and
# weight decay applied to the parameter directly (not through the gradient).

def adamw_step(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int):
    """One AdamW step at step number t = `step` (t >= 1), in float64:
        m' = beta1 m + (1 - beta1) g
        v' = beta2 v + (1 - beta2) g^2
        p' = p - lr (  (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)
                     + weight_decay p )
    Returns (p', m', v') as float64 arrays."""
    p, g, m, v = (np.asarray(a, dtype=np.float64) for a in (p, g, m, v))
    m1 = beta1 * m + (1.0 - beta1) * g
    v1 = beta2 * v + (1.0 - beta2) * g * g
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    p1 = p - lr * (mhat / (np.sqrt(vhat) + eps) + weight_decay * p)
    return p1, m1, v1


# ---------------------------------------------- reversible residual block --
# "Reversible Sparse MoE Single Node" (skill card), Principle 1 "Reversible
# Recurrence Stack" and Pattern 1 "Reversible Layer Implementation": a block
# reconstructs its input from its output instead of storing it, through
# invertible operations such as addition and subtraction; Implementation
# Considerations: reversible residual blocks, stateless routing.  The layer is
# the block's function G: with streams (y1, x2),
#     y2 = x2 + G(y1),        x2 = y2 - G(y1).

def rev_forward(inputs: dict, x2, k: int, group: int, lam: float = 1.0,
                topk_idx: np.ndarray | None = None) -> np.ndarray:
    """y2 = x2 + MoE(y1), y1 = inputs["x"], in float64."""
    return to_f64(x2) + forward(inputs, k, group, lam, topk_idx=topk_idx)["y"]


def rev_inverse(inputs: dict, y2, k: int, group: int, lam: float = 1.0,
                topk_idx: np.ndarray | None = None) -> np.ndarray:
    """x2 = y2 - MoE(y1), MoE(y1) recomputed from y1, in float64."""
    return to_f64(y2) - forward(inputs, k, group, lam, topk_idx=topk_idx)["y"]


# ------------------------------------------------- few -> many growth --
# "Reversible Sparse MoE Single Node" (skill card), Principle 2
# "State-Preserving Growth": the few -> many expansion duplicates experts and
# reinitialises routing; Pattern 2: expansions are initialised from the
# smaller model and must preserve its state.  Grown expert e F + c
# (c = 0 .. F-1) is expert e; router column e F + c is column e, moved for
# c >= 1 by s * z[:, e F + c] in float32 with one rounding.  With s = 0 and
# F k experts per token the grown layer computes the original function.

PER_EXPERT_PREFIXES = ("q_", "s_", "A_", "B_")


def grow(inputs: dict, factor: int, noise=None, noise_scale: float = 0.0) -> dict:
    """The grown layer's tensors (the dict layout of the inputs)."""
    out = dict(inputs)
    for key, v in inputs.items():
        if v is not None and key.startswith(PER_EXPERT_PREFIXES):
            out[key] = np.repeat(v, factor, axis=0)
    w = np.repeat(np.asarray(inputs["w_router"], np.float32), factor, axis=1)
    if noise is not None and noise_scale != 0.0:
        moved = (w.astype(np.float64) + np.float64(np.float32(noise_scale))
                 * np.asarray(noise, np.float64)).astype(np.float32)
        copies = (np.arange(w.shape[1]) % factor) != 0
        w[:, copies] = moved[:, copies]
    out["w_router"] = w
    if inputs.get("b_router") is not None:
        out["b_router"] = np.repeat(np.asarray(inputs["b_router"], np.float32), factor)
    return out


def routing_load(topk_idx: np.ndarray, E: int) -> dict:
    """Routing-collapse statistics of one routing: the most loaded expert's
    share over the mean load, and the number of experts that get no token."""
    counts = np.bincount(np.asarray(topk_idx).ravel(), minlength=E)
    return {"max_over_mean": float(counts.max() / counts.mean()), "empty": int((counts == 0).sum())}
