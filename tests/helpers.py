"""Shared helpers for the GPU parity tests: uploads, oracle comparisons, tolerances.

Tolerances (the bar every parity test applies):
  * relayout: byte-equal;
  * fp32 attention: max-abs <= 1e-5 on O, lse, dQ, dK, dV;
  * bf16 attention: O max-abs <= 1e-2; dQ, dK, dV relative L2 <= 2e-2 per tensor;
    lse max-abs <= 1e-3 (lse is fp32 computed from bf16 inputs);
  * bf16 O elements with |O*| >= 4 may exceed 1e-2 by bf16 output rounding alone; such an
    element is accepted only if |err| <= half a bf16 ulp of O* + 1e-3 (reported).
"""

from __future__ import annotations

import numpy as np

from oracle import attention as OA

TOL_F32 = 1e-5
TOL_BF16_O = 1e-2
TOL_BF16_GRAD_RL2 = 2e-2
TOL_BF16_LSE = 1e-3


def to_device(arr: np.ndarray, dtype: str):
    """Stored host array -> torch device tensor of the workload dtype (bits unchanged)."""
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16)).view(torch.bfloat16).cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    raise ValueError(dtype)


def to_f64(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact widening)."""
    import torch

    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((x - ref).ravel()) / (den if den > 0 else 1.0))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - 8)


def check_o_bf16(o: np.ndarray, ref: np.ndarray, what: str = "O") -> dict:
    err = np.abs(o - ref)
    worst = float(err.max()) if err.size else 0.0
    over = err > TOL_BF16_O
    if over.any():
        big = np.abs(ref) >= 4.0
        ok = big & (err <= bf16_half_ulp(ref) + 1e-3)
        bad = over & ~ok
        assert not bad.any(), f"{what}: max-abs {worst:.3g} > {TOL_BF16_O} at {np.argwhere(bad)[:5]}"
    return {"max_abs": worst, "n_rounding_edge": int(over.sum())}


def check_max_abs(x: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    worst = float(np.abs(x - ref).max()) if x.size else 0.0
    assert worst <= tol, f"{what}: max-abs {worst:.3g} > {tol}"
    return worst


def check_rel_l2(x: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    r = rel_l2(x, ref)
    assert r <= tol, f"{what}: rel-L2 {r:.3g} > {tol}"
    return r


def widen_inputs(st: dict, dtype: str) -> dict:
    return {n: OA.widen(a, dtype) for n, a in st.items()}
