"""Parity metrics and small drivers shared by the GPU tests.

Tolerances (fp32 state, bf16 q/k/v, fp64 oracle fed the same bf16/fp32 values):

* fp32 tensors (states, checkpoints): ``rel(x, r) = max|x - r| / max|r| <= 2e-3``.
* bf16 outputs o: storing a value in bf16 alone moves it by up to half an ulp (relative
  2^-8 near a power of two), which on its own can exceed 2e-3 of max|r|. So o is scored on
  the error beyond that mandatory rounding:
  ``rel_bf16(x, r) = max(max(0, |x - r| - ulp_bf16(r) / 2)) / max|r| <= 2e-3``;
  a kernel whose fp32 result is exact scores 0.

Both are taken twice: over the whole tensor, and per (sequence, head) -- normalised by that
group's own scale (for outputs, the larger of its reference and value magnitudes; for states,
the state's own largest entry) -- so that a wrong head or sequence of small magnitude cannot
hide under a large one. ``check_out`` / ``check_state`` assert both and append the
measured values to the JSON-lines file named by the environment variable KDA_PARITY_LOG (when
set), one record per check, tagged with the running test.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

TOL = 2e-3


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel(x, r) -> float:
    x, r = f64(x), f64(r)
    den = np.max(np.abs(r)) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - r)) / den)


def half_ulp_bf16(r: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(r))            # |r| = m 2^e, m in [0.5, 1): ulp_bf16 = 2^(e-8)
    h = np.ldexp(1.0, e - 9)
    return np.where(r == 0, 0.0, h)


def rel_bf16(x, r) -> float:
    x, r = f64(x), f64(r)
    den = np.max(np.abs(r)) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    excess = np.maximum(0.0, np.abs(x - r) - half_ulp_bf16(r))
    return float(np.max(excess) / den)


def _log(kind: str, what: str, shape, err_all: float, err_group: float, n_groups: int) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    rec = {"test": test, "what": what, "kind": kind, "shape": list(shape),
           "global": err_all, "per_group": err_group, "groups": n_groups, "tol": TOL}
    print(f"[parity] {test} {what}: global {err_all:.3e}, worst (sequence, head) "
          f"{err_group:.3e} over {n_groups} groups", flush=True)
    path = os.environ.get("KDA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _rel_bf16_scaled(x, r, v) -> float:
    """rel_bf16 with the denominator max(max|r|, max|v|): the error beyond the bf16 rounding of
    the output, against the larger of the output's and its value inputs' magnitudes."""
    den = max(float(np.max(np.abs(r))) if r.size else 0.0,
              float(np.max(np.abs(v))) if v is not None and v.size else 0.0)
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.maximum(0.0, np.abs(x - r) - half_ulp_bf16(r))) / den)


def check_out(x, r, cu=None, what: str = "o", v=None) -> tuple[float, float]:
    """bf16 outputs against the oracle, over the whole tensor (rel_bf16) and per (sequence,
    head).

    Shapes: [n_seq, ..., H, dv] (axis 0 = sequence, axis -2 = head; any axes between, such as
    verify positions, belong to the group), or packed [N, H, dv] with ``cu`` giving the
    sequence boundaries along axis 0 (empty sequences are skipped). ``v`` (same shape: the
    value inputs of the same tokens) sets each group's scale: its error is taken against
    max(max|o_ref|, max|v|) of that group, so that a group whose outputs are small because q
    and the state nearly cancel (one token from a zero state reads b (q.k) v) is measured
    against the magnitude of what it read, while a wrong head or sequence of small magnitude
    still cannot hide under a large one."""
    x, r = f64(x), f64(r)
    vv = None if v is None else f64(v)
    assert x.shape == r.shape, (x.shape, r.shape)
    assert vv is None or vv.shape == x.shape, (vv.shape, x.shape)
    e_all = rel_bf16(x, r)
    groups = []
    if cu is not None:
        cu = [int(c) for c in cu]
        for lo, hi in zip(cu[:-1], cu[1:]):
            if hi > lo:
                groups += [(x[lo:hi, h], r[lo:hi, h], None if vv is None else vv[lo:hi, h])
                           for h in range(x.shape[1])]
    else:
        xm, rm = np.moveaxis(x, -2, 1), np.moveaxis(r, -2, 1)
        vm = None if vv is None else np.moveaxis(vv, -2, 1)
        groups = [(xm[i, h], rm[i, h], None if vm is None else vm[i, h])
                  for i in range(xm.shape[0]) for h in range(xm.shape[1])]
    e_grp = max((_rel_bf16_scaled(a, b, c) for a, b, c in groups), default=0.0)
    _log("bf16", what, x.shape, e_all, e_grp, len(groups))
    assert e_all <= TOL and e_grp <= TOL, (what, e_all, e_grp)
    return e_all, e_grp


def check_state(x, r, what: str = "state") -> tuple[float, float]:
    """fp32 states [..., dk, dv] against the oracle, whole tensor and per matrix (every
    leading index: slot, head)."""
    x, r = f64(x), f64(r)
    assert x.shape == r.shape, (x.shape, r.shape)
    e_all = rel(x, r)
    xm = x.reshape((-1,) + x.shape[-2:])
    rm = r.reshape((-1,) + r.shape[-2:])
    e_grp = max((rel(xm[i], rm[i]) for i in range(xm.shape[0])), default=0.0)
    _log("fp32", what, x.shape, e_all, e_grp, xm.shape[0])
    assert e_all <= TOL and e_grp <= TOL, (what, e_all, e_grp)
    return e_all, e_grp


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def meta_equal(gpu_meta: np.ndarray, oracle_meta: np.ndarray, slots) -> None:
    slots = list(slots)
    np.testing.assert_array_equal(gpu_meta[slots], oracle_meta[slots])
