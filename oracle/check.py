"""Tolerance checker -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Compares results of the HIP library with the float64 oracle under the stated
tolerances:
  * codes: equal to the oracle's, except where the oracle's distance to the
    chosen codeword is within a relative 1e-4 of its best distance (a near
    tie, where several codes are correct).  After any accepted choice the
    oracle continues the residual chain from that choice (teacher forcing), so
    one near tie does not make later stages look wrong;
  * scalar codes: the same rule on the scalar distances: equal to the
    oracle's nearest level, except where the candidate level's squared
    distance is within a relative 1e-4 of the best one; stage 2 is checked on
    the residual of the candidate's stage-1 choice;
  * reconstructed vectors: within 1e-6 absolute;
  * attention outputs: within 2e-3 max-abs and 1e-3 relative L2.
"""
from __future__ import annotations

import numpy as np

from .kvq_oracle import fwht, nearest, scalar_nearest

CODE_REL_TOL = 1e-4
RECON_ATOL = 1e-6
ATTN_ATOL = 2e-3
ATTN_REL_L2 = 1e-3


def check_codes(x, codebooks, codes, *, rotate=True, rel_tol=CODE_REL_TOL, block=4096):
    """Teacher-forced comparison of candidate codes [N][S][G] with the oracle.

    Returns counts of exact matches, accepted near ties and hard mismatches
    over all N*S*G decisions, and the worst relative excess
    d(z_candidate)/d1 - 1 seen among non-exact decisions."""
    S, G, C, dsub = codebooks.shape
    x = np.asarray(x, dtype=np.float64)
    codes = np.asarray(codes)
    cb = np.asarray(codebooks, dtype=np.float64)
    n_exact = n_tie = n_hard = 0
    worst = 0.0
    hard_at = []
    for lo in range(0, x.shape[0], block):
        hi = min(x.shape[0], lo + block)
        y = fwht(x[lo:hi]) if rotate else x[lo:hi]
        for g in range(G):
            r = y[:, g * dsub:(g + 1) * dsub].copy()
            for s in range(S):
                z_o, d = nearest(r, cb[s, g])
                z_c = codes[lo:hi, s, g].astype(np.int64)
                if np.any(z_c >= C):
                    raise ValueError("candidate code out of range")
                rows = np.arange(hi - lo)
                d1 = d[rows, z_o]
                dc = d[rows, z_c]
                exact = z_c == z_o
                ok = dc <= (1.0 + rel_tol) * d1
                n_exact += int(exact.sum())
                n_tie += int((~exact & ok).sum())
                bad = ~exact & ~ok
                n_hard += int(bad.sum())
                if (~exact).any():
                    with np.errstate(divide="ignore", invalid="ignore"):
                        ex = np.where(d1 > 0, dc / d1 - 1.0, np.where(dc > 0, np.inf, 0.0))
                    worst = max(worst, float(ex[~exact].max()))
                if bad.any() and len(hard_at) < 16:
                    for i in np.nonzero(bad)[0][:16 - len(hard_at)]:
                        hard_at.append((lo + int(i), s, g, int(z_c[i]), int(z_o[i])))
                r = r - cb[s, g][z_c]          # follow the candidate's choice
    total = x.shape[0] * S * G
    return {"total": total, "exact": n_exact, "near_tie": n_tie, "hard": n_hard,
            "worst_rel_excess": worst, "hard_examples": hard_at}


def check_scalar_codes(y, levels1, levels2, z1, z2, *, rel_tol=CODE_REL_TOL):
    """Teacher-forced check of candidate scalar indices z1, z2 [N][D] against
    the nearest levels of the rotated vectors y [N][D] (float64), under the
    code rule of the vector quantiser: a non-matching index is accepted when
    its squared distance to the element is at most (1 + rel_tol) times the
    best level's (the best two distances within rel_tol relative)."""
    y = np.asarray(y, dtype=np.float64)
    l1 = np.asarray(levels1, dtype=np.float64)
    l2 = np.asarray(levels2, dtype=np.float64)
    out = {"total": 2 * y.size, "exact": 0, "near_tie": 0, "hard": 0, "worst_rel_excess": 0.0}
    r = y
    for lv, zc in ((l1, np.asarray(z1)), (l2, np.asarray(z2))):
        zo = scalar_nearest(r, lv)
        dc = (r - lv[zc]) ** 2
        do = (r - lv[zo]) ** 2
        exact = zc == zo
        ok = dc <= (1.0 + rel_tol) * do
        out["exact"] += int(exact.sum())
        out["near_tie"] += int((~exact & ok).sum())
        out["hard"] += int((~exact & ~ok).sum())
        if (~exact).any():
            with np.errstate(divide="ignore", invalid="ignore"):
                ex = np.where(do > 0, dc / do - 1.0, np.where(dc > 0, np.inf, 0.0))
            out["worst_rel_excess"] = max(out["worst_rel_excess"], float(ex[~exact].max()))
        r = r - lv[zc]
    return out


def check_recon(got, ref, atol=RECON_ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return {"max_abs": err, "ok": err <= atol}


def check_attn(got, ref, atol=ATTN_ATOL, rel_l2=ATTN_REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    flat = np.abs(diff).reshape(-1, diff.shape[-1]).max(axis=1)
    worst = int(np.argmax(flat)) if flat.size else -1
    return {"max_abs": max_abs, "rel_l2": rel, "worst_row": worst,
            "ok": max_abs <= atol and rel <= rel_l2}
