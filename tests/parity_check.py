"""Element-by-element parity checks shared by the GPU tests (test infrastructure).

Two bars hold for every compared output (o and the final state):

  * per unit: the relative L2 error ||x - x_ref|| / ||x_ref|| over each (sequence, value head)
    unit is <= tol (bf16 io 5e-3, fp32 io 1e-4). A unit whose reference is exactly zero must
    come out exactly zero.
  * per row: every row (one token of o, one key row of the final state; V values) satisfies
        ||x_row - ref_row|| <= tol_row * (||ref_row|| + rms_unit)
    with rms_unit the root-mean-square row norm of the reference over the unit's rows.

Why the row bound has that form. Rounding o to bf16 moves each element by at most 2^-8 of its
magnitude (bf16 keeps 8 significant bits; round to nearest), so the rounding alone gives
||x_row - ref_row|| <= 2^-8 ||ref_row|| = 3.9e-3 ||ref_row||. The arithmetic before the final
rounding (fp16 operands with 2^-11 unit roundoff, fp32 accumulation) adds an error that scales
with the magnitudes of the state and the chunk operands rather than with the row's own norm, so
it is bounded relative to the unit's typical row norm. tol_row = 5e-3 (bf16) covers the
rounding term with margin and allows an arithmetic error up to 5e-3 of the unit's rms row norm
(the measured arithmetic error is about 5e-4 of it); fp32 io has no output rounding and uses
1e-4. A row that is wrong as a whole (zero, stale, another token's or another head's) differs by
about its own norm and fails for every row whose norm exceeds 0.5% of the unit's rms.

One global relative L2 over a whole tensor would not see such a row: at 16 heads x 4096 tokens a
single zeroed row adds 1/256 = 3.9e-3 to the global error.
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 5e-3, "fp32": 1e-4}
TOL_ROW = {"bf16": 5e-3, "fp32": 1e-4}


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def _segments_sum(x: np.ndarray, bounds) -> np.ndarray:
    """Sums of x [T_total, ...] over the token ranges [a, b) of `bounds` -> [N, ...]."""
    out = np.zeros((len(bounds),) + x.shape[1:], np.float64)
    for i, (a, b) in enumerate(bounds):
        if b > a:
            out[i] = x[a:b].sum(axis=0)
    return out


def o_errors(o, o_ref, bounds, units=None):
    """Per-unit relative L2 errors and per-row error ratios of o.

    o, o_ref: [B, T, HV, V] (any float dtype); bounds: [(bos, eos)] per sequence on the packed
    token axis; units: optional list of (s, j) to restrict the comparison to.
    Returns (unit_err [N, HV] (nan where not compared), row_ratio [T_total, HV] (0 where not
    compared): ||d_row|| / (||ref_row|| + rms_unit), rms [N, HV]).
    """
    HV, V = o_ref.shape[2], o_ref.shape[3]
    x = np.asarray(o).reshape(-1, HV, V)
    r = np.asarray(o_ref).reshape(-1, HV, V)
    N = len(bounds)
    if units is None:
        d2 = np.zeros(x.shape[:2], np.float64)
        r2 = np.zeros(x.shape[:2], np.float64)
        for j in range(HV):            # head by head: bounded temporary memory
            dj = x[:, j].astype(np.float64) - r[:, j].astype(np.float64)
            d2[:, j] = np.einsum("tv,tv->t", dj, dj)
            rj = r[:, j].astype(np.float64)
            r2[:, j] = np.einsum("tv,tv->t", rj, rj)
        mask = np.ones((N, HV), bool)
    else:
        d2 = np.zeros(x.shape[:2], np.float64)
        r2 = np.zeros(x.shape[:2], np.float64)
        mask = np.zeros((N, HV), bool)
        for (s, j) in units:
            a, b = bounds[s]
            dj = x[a:b, j].astype(np.float64) - r[a:b, j].astype(np.float64)
            rj = r[a:b, j].astype(np.float64)
            d2[a:b, j] = np.einsum("tv,tv->t", dj, dj)
            r2[a:b, j] = np.einsum("tv,tv->t", rj, rj)
            mask[s, j] = True
    D = _segments_sum(d2, bounds)                  # [N, HV] squared error per unit
    R = _segments_sum(r2, bounds)
    lens = np.array([b - a for a, b in bounds], np.float64)[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        unit_err = np.where(R > 0, np.sqrt(D / np.where(R > 0, R, 1)), np.sqrt(D))
        rms = np.sqrt(np.where(lens > 0, R / np.maximum(lens, 1), 0.0))
    unit_err = np.where(mask & (lens > 0), unit_err, np.nan)
    rms_tok = np.zeros_like(d2)
    for i, (a, b) in enumerate(bounds):
        rms_tok[a:b] = rms[i]
    den = np.sqrt(r2) + rms_tok
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(den > 0, np.sqrt(d2) / np.where(den > 0, den, 1),
                         np.where(d2 > 0, np.inf, 0.0))
    return unit_err, ratio, rms


def state_errors(fin, f_ref, units=None):
    """Per-unit relative L2 errors and per-key-row error ratios of the final state
    [N, HV, K, V]; same conventions as o_errors (rows are the K rows of each unit)."""
    x = np.asarray(fin, np.float64)
    r = np.asarray(f_ref, np.float64)
    d2 = ((x - r) ** 2).sum(-1)                    # [N, HV, K]
    r2 = (r ** 2).sum(-1)
    D, R = d2.sum(-1), r2.sum(-1)                  # [N, HV]
    with np.errstate(invalid="ignore", divide="ignore"):
        unit_err = np.where(R > 0, np.sqrt(D / np.where(R > 0, R, 1)), np.sqrt(D))
    rms = np.sqrt(R / max(1, r.shape[2]))
    den = np.sqrt(r2) + rms[..., None]
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(den > 0, np.sqrt(d2) / np.where(den > 0, den, 1),
                         np.where(d2 > 0, np.inf, 0.0))
    if units is not None:
        mask = np.zeros(unit_err.shape, bool)
        for (s, j) in units:
            mask[s, j] = True
        unit_err = np.where(mask, unit_err, np.nan)
        ratio = np.where(mask[..., None], ratio, 0.0)
    return unit_err, ratio


def check_outputs(o, fin, o_ref, f_ref, bounds, dtype, units=None, what=""):
    """Assert both bars on o (and on the final state when fin is not None). Returns a dict of
    the worst values (for the error log)."""
    tol, tol_row = TOL[dtype], TOL_ROW[dtype]
    assert np.isfinite(np.asarray(o, np.float32)).all(), f"{what}: non-finite o"
    ue, ratio, _ = o_errors(o, o_ref, bounds, units)
    worst = {"o_unit": float(np.nanmax(ue)) if np.isfinite(ue).any() else 0.0,
             "o_row": float(ratio.max()) if ratio.size else 0.0}
    if fin is not None:
        assert np.isfinite(fin).all(), f"{what}: non-finite final state"
        fe, fr = state_errors(fin, f_ref, units)
        worst["final_unit"] = float(np.nanmax(fe)) if np.isfinite(fe).any() else 0.0
        worst["final_row"] = float(fr.max()) if fr.size else 0.0
    bad_units = np.argwhere(np.nan_to_num(ue, nan=0.0) > tol)
    assert bad_units.size == 0, (
        f"{what}: o rel L2 above {tol} in {len(bad_units)} unit(s), first (s, j) = "
        f"{tuple(int(i) for i in bad_units[0])}: {ue[tuple(bad_units[0])]:.3e}")
    bad_rows = np.argwhere(ratio > tol_row)
    assert bad_rows.size == 0, (
        f"{what}: o row error above {tol_row} x (row norm + unit rms) in {len(bad_rows)} "
        f"row(s), first (token, head) = {tuple(int(i) for i in bad_rows[0])}: {ratio[tuple(bad_rows[0])]:.3e}")
    if fin is not None:
        bad_units = np.argwhere(np.nan_to_num(fe, nan=0.0) > tol)
        assert bad_units.size == 0, (
            f"{what}: final-state rel L2 above {tol} in {len(bad_units)} unit(s), first "
            f"(s, j) = {tuple(int(i) for i in bad_units[0])}: {fe[tuple(bad_units[0])]:.3e}")
        bad_rows = np.argwhere(fr > tol_row)
        assert bad_rows.size == 0, (
            f"{what}: final-state row error above {tol_row} x (row norm + unit rms) in "
            f"{len(bad_rows)} row(s), first (s, j, key row) = {tuple(int(i) for i in bad_rows[0])}: "
            f"{fr[tuple(bad_rows[0])]:.3e}")
    return worst


# ----------------------------------------------------------------------------- gradients

GRAD_TOL = 1e-4          # the backward computes in fp32 from the exact inputs (either io)
GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def check_grads(got, ref, bounds, what=""):
    """Both bars on every gradient tensor, per unit and per row, as for o and the final state:
    dq and dk per (sequence, q/k head) with token rows of K values; dv and dg per (sequence,
    value head) with token rows; dbeta per (sequence, value head) with one value per token;
    dh0 per (sequence, value head) with its K key rows. got and ref are (dq, dk, dv, dg, dbeta,
    dh0) in the layouts of the inputs ([B, T, heads, D], [B, T, HV], [N, HV, K, V]). Returns
    the worst unit and row values per tensor."""
    worst = {}
    for name, a, b in zip(GRAD_NAMES, got, ref):
        if name == "dh0":
            if a is None:
                continue
            assert np.isfinite(a).all(), f"{what}: non-finite {name}"
            ue, ratio = state_errors(a, np.asarray(b).reshape(a.shape))
        else:
            a = np.asarray(a)
            b = np.asarray(b).reshape(a.shape)
            if name == "dbeta":
                a, b = a[..., None], b[..., None]
            assert np.isfinite(a).all(), f"{what}: non-finite {name}"
            ue, ratio, _ = o_errors(a, b, bounds)
        worst[name + "_unit"] = float(np.nanmax(ue)) if np.isfinite(ue).any() else 0.0
        worst[name + "_row"] = float(ratio.max()) if ratio.size else 0.0
        bad = np.argwhere(np.nan_to_num(ue, nan=0.0) > GRAD_TOL)
        assert bad.size == 0, (
            f"{what}: {name} rel L2 above {GRAD_TOL} in {len(bad)} unit(s), first "
            f"{tuple(int(i) for i in bad[0])}: {ue[tuple(bad[0])]:.3e}")
        bad = np.argwhere(ratio > GRAD_TOL)
        assert bad.size == 0, (
            f"{what}: {name} row error above {GRAD_TOL} x (row norm + unit rms) in {len(bad)} "
            f"row(s), first {tuple(int(i) for i in bad[0])}: {ratio[tuple(bad[0])]:.3e}")
    return worst
