"""The fp64 oracle over the whole layer, with its per-expert work spread over
worker processes (test infrastructure).

The layer's experts are independent given the routing, so the oracle's own
per-expert function (oracle.expert_rows) can run for different experts in
different processes; the routing (oracle.route), the combine
(oracle.combine) and the gate path of the backward (oracle.gate_backward)
run in the calling process, exactly as oracle.forward / oracle.backward
chain them.  No arithmetic of the layer is written here.

The workers are fresh Python processes that import only numpy and the
oracle (never torch or the HIP library), so they are safe to start from a
process that already uses the GPU.  Inputs, routing and results are shared
through .npy files in a temporary directory under /dev/shm (memory-mapped on
both sides), and every worker runs single-threaded BLAS.

    layer(inputs, cfg, topk_idx=None, backward=True, workers=None) -> dict

returns the keys of oracle.forward (routing, "e_out", "y") and, with
backward, those of oracle.backward ("dx", "dx_router", the six adapter
gradients).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

ROUTE_KEYS = ("offsets", "perm_src", "gates")


def default_workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _assign(counts: np.ndarray, workers: int) -> list:
    """Experts with rows, largest first, each to the least-loaded worker
    (cost ~ rows + a fixed per-expert dequantisation cost)."""
    order = np.argsort(-counts, kind="stable")
    load = np.zeros(workers)
    parts = [[] for _ in range(workers)]
    for e in order:
        if counts[e] == 0:
            continue
        w = int(np.argmin(load))
        parts[w].append(int(e))
        load[w] += counts[e] + 64
    return parts


def layer(inputs: dict, cfg, topk_idx=None, backward: bool = True, workers: int | None = None,
          log=None) -> dict:
    workers = workers or default_workers()
    k, group, lam = cfg.k, cfg.group, cfg.lora_scale
    t0 = time.perf_counter()
    R = oracle.route(inputs, k, topk_idx)
    T, d = inputs["x"].shape
    S = T * k
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    with tempfile.TemporaryDirectory(dir=shm, prefix="moe_oracle_") as tmp:
        for key, v in inputs.items():
            if v is not None:
                np.save(os.path.join(tmp, f"in_{key}.npy"), np.ascontiguousarray(v))
        for key in ROUTE_KEYS:
            np.save(os.path.join(tmp, f"R_{key}.npy"), R[key])
        O = np.lib.format.open_memmap(os.path.join(tmp, "out_O.npy"), "w+", np.float64, (S, d))
        outs = {"O": O}
        if backward:
            outs["dX"] = np.lib.format.open_memmap(os.path.join(tmp, "out_dX.npy"), "w+",
                                                   np.float64, (S, d))
            for n, shape in oracle.adapter_grad_shapes(inputs).items():
                outs[n] = np.lib.format.open_memmap(os.path.join(tmp, f"out_{n}.npy"), "w+",
                                                    np.float64, shape)
        for a in outs.values():
            a.flush()
        parts = _assign(R["counts"], workers)
        for w, p in enumerate(parts):
            np.save(os.path.join(tmp, f"part_{w}.npy"), np.array(p, np.int64))
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1",
                   MKL_NUM_THREADS="1", BLIS_NUM_THREADS="1")
        procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), tmp, str(w),
                                   str(k), str(group), repr(float(lam)), str(int(backward))],
                                  env=env) for w in range(len(parts))]
        rcs = [p.wait() for p in procs]
        if any(rcs):
            raise RuntimeError(f"oracle workers failed: exit codes {rcs}")
        if log:
            log(f"oracle experts on {len(parts)} workers: {time.perf_counter() - t0:.1f} s")
        res = dict(R)
        res["e_out"] = np.array(O)
        res["y"] = oracle.combine(R["gates"], res["e_out"], R["slot_pos"])
        if backward:
            dgam, dl, dx_r = oracle.gate_backward(inputs["dy"], res["e_out"], R["gates"],
                                                  R["topk_idx"], R["slot_pos"],
                                                  inputs["w_router"])
            dXp = np.array(outs["dX"])
            dx = dx_r.copy()
            slot = R["slot_pos"].reshape(T, k)
            for j in range(k):
                dx += dXp[slot[:, j]]
            res.update({"dx": dx, "dx_router": dx_r, "dgates": dgam, "dlogits_sel": dl})
            for n in oracle.ADAPTER_GRADS:
                res[n] = np.array(outs[n])
        del O, outs
    if log:
        log(f"oracle whole layer: {time.perf_counter() - t0:.1f} s")
    return res


def _worker(tmp: str, wid: int, k: int, group: int, lam: float, backward: bool) -> None:
    ld = lambda name, mode="r": np.load(os.path.join(tmp, name), mmap_mode=mode)
    inputs = {}
    for f in os.listdir(tmp):
        if f.startswith("in_"):
            inputs[f[3:-4]] = ld(f)
    inputs.setdefault("b_router", None)
    R = {key: ld(f"R_{key}.npy") for key in ROUTE_KEYS}
    O = ld("out_O.npy", "r+")
    outs = {}
    if backward:
        outs["dX"] = ld("out_dX.npy", "r+")
        for n in oracle.ADAPTER_GRADS:
            outs[n] = ld(f"out_{n}.npy", "r+")
    for e in ld(f"part_{wid}.npy"):
        lo, hi = R["offsets"][e], R["offsets"][e + 1]
        res = oracle.expert_rows(inputs, R, int(e), k, group, lam, backward=backward)
        O[lo:hi] = res["O"]
        if backward:
            outs["dX"][lo:hi] = res["dX"]
            for n in oracle.ADAPTER_GRADS:
                outs[n][e] = res[n]
    O.flush()
    for a in outs.values():
        a.flush()


if __name__ == "__main__":
    a = sys.argv[1:]
    _worker(a[0], int(a[1]), int(a[2]), int(a[3]), float(a[4]), bool(int(a[5])))
