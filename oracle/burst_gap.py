"""Burst-Gap issue-time model and its parameter fit (test infrastructure).

Source: X-Stage explainer (gist.science, arXiv 2607.23264), technical summary,
"Methodology": the issuer-visible time to issue a burst of aggregate volume V from K
producers, separated from the previous burst by a useful gap G, is

    T_iss(G; K, V) = max(T0_iss(K, V), V / R - G)

with T0_iss the backpressure-free issue time, R the effective drain rate and Q the
effective pending capacity.  Two regimes: drain-dominated (short G, T_iss = V/R - G) and
backpressure-free (long G, T_iss = T0_iss).  "Contributions" (characterisation item):
T0_iss, R and Q are measured with parameterised microbenchmarks.

The printed formula does not contain Q.  ``t_iss_fluid`` is a labelled reading that gives
Q a role (a fluid queue of capacity Q drained at R whenever it is non-empty); it equals
the printed formula whenever G <= Q / R.
"""

from __future__ import annotations

import numpy as np


def t_iss(G, T0, V, R):
    """The printed Burst-Gap formula, evaluated in float64 (broadcasts over arrays)."""
    G = np.asarray(G, dtype=np.float64)
    return np.maximum(np.asarray(T0, dtype=np.float64), np.asarray(V, dtype=np.float64) / np.float64(R) - G)


def regime(G, T0, V, R):
    """'drain' where V/R - G exceeds T0 (drain-dominated), else 'free' (backpressure-free)."""
    drain = np.asarray(V, dtype=np.float64) / np.float64(R) - np.asarray(G, dtype=np.float64) > np.asarray(T0, dtype=np.float64)
    return np.where(drain, "drain", "free")


def t_iss_fluid(G, T0, V, R, Q):
    """Reading with capacity Q (an extension, not printed on the pages).

    Producer issues its burst of V at the free rate V / T0; accepted volume waits in a
    queue of capacity Q that drains at R whenever non-empty.  Periodic steady state:

    * G < Q/R: the queue never empties, so each period drains exactly V at R:
      T_iss + G = V / R, i.e. the printed drain-dominated branch;
    * G >= Q/R: the gap empties the queue; a burst fills Q, then issues the remaining
      V - Q at R: T_iss = (V - Q) / R (in the limit of a free rate much faster than R).

    Both branches are max(T0, V/R - min(G, Q/R)).
    """
    G = np.asarray(G, dtype=np.float64)
    eff_gap = np.minimum(G, np.float64(Q) / np.float64(R))
    return np.maximum(np.asarray(T0, dtype=np.float64), np.asarray(V, dtype=np.float64) / np.float64(R) - eff_gap)


def t0_linear(K, V, c, f1):
    """Backpressure-free issue time read as a fixed cost plus V/K bytes at a per-producer rate f1.

    The pages make T0_iss a function of (K, V) without giving its form; this affine form
    is a reading used only by the fluid fit.
    """
    return np.float64(c) + np.asarray(V, dtype=np.float64) / (np.asarray(K, dtype=np.float64) * np.float64(f1))


def t_iss_isolated(T0, V, R, Q):
    """Capacity reading for a burst that starts on an empty queue (the previous burst drained
    long before): the first Q bytes are absorbed, the rest issue at the drain rate, so
    T_iss = max(T0, (V - Q) / R).  This is the G -> infinity limit of ``t_iss_fluid``."""
    V = np.asarray(V, dtype=np.float64)
    return np.maximum(np.asarray(T0, dtype=np.float64), (V - np.float64(Q)) / np.float64(R))


def fit_isolated(V, T, T0, R=None, margin=1.5):
    """Capacity Q (and a drain rate) from isolated bursts, per the capacity reading.

    V, T: volumes (bytes) and issue times (s) of bursts issued on an empty queue; T0: their
    backpressure-free issue times.  Points with T > margin * T0 lie on T = (V - Q) / R:
    * a least-squares line T = a + b V over those points gives R_iso = 1 / b and
      Q_iso = -a / b (both from the isolated bursts alone);
    * with a drain rate R measured elsewhere (the drain branch of periodic bursts),
      Q = median(V - R T) over the same points.
    Needs at least two distinct volumes above the margin."""
    V = np.asarray(V, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    sel = T > margin * np.asarray(T0, dtype=np.float64)
    out = {"n_used": int(sel.sum())}
    if len(set(V[sel].tolist())) < 2:
        return out
    b, a = np.polyfit(V[sel], T[sel], 1)
    out["R_iso"] = float(1.0 / b)
    out["Q_iso"] = float(-a / b)
    if R is not None:
        out["Q"] = float(np.median(V[sel] - np.float64(R) * T[sel]))
    return out


def fit_burst_gap(points, drain_margin=1.1):
    """Fit the Burst-Gap parameters to measured (K, V_bytes, G_s, T_iss_s) points.

    Page formula (no Q), in the order the model is stated:
      1. T0(K, V) = median T_iss at the longest gap measured for that (K, V), where the
         formula says the issuer is backpressure-free;
      2. R: points with T_iss > drain_margin * T0 lie on the drain branch T_iss + G = V/R;
         least squares of (T_iss + G) on V through the origin gives 1/R;
      3. relative error |T_meas - T_model| / T_meas of every point.
    Fluid reading (extension): parameters (c, f1, R, Q) of
      T_iss = max(c + V/(K f1), V/R - min(G, Q/R))
    by least squares on log T over all points, started from the page-formula fit.
    """
    from scipy.optimize import least_squares

    pts = np.asarray(list(points), dtype=np.float64)
    if pts.ndim != 2 or pts.shape[0] == 0:
        raise ValueError("no points")
    K, V, G, T = pts.T
    T0 = {}
    for kv in sorted(set(zip(K.tolist(), V.tolist()))):
        sel = (K == kv[0]) & (V == kv[1])
        at = sel & (G == G[sel].max())
        T0[kv] = float(np.median(T[at]))
    t0_arr = np.array([T0[(k, v)] for k, v in zip(K.tolist(), V.tolist())])
    drain = T > drain_margin * t0_arr
    out = {"T0": T0, "R": None, "n_points": int(len(T)), "n_drain": int(drain.sum())}
    if not drain.any():
        return out
    x = V[drain]
    y = T[drain] + G[drain]
    R = float(np.dot(x, x) / np.dot(x, y))
    out["R"] = R
    rel = np.abs(T - t_iss(G, t0_arr, V, R)) / T
    out["rel_err_median"] = float(np.median(rel))
    out["rel_err_max"] = float(rel.max())

    # fluid reading: start c, f1 from the long-gap T0 of the smallest volume per K
    vmin = V.min()
    small = [(k, T0[(k, vmin)]) for k in sorted(set(K.tolist()))]
    f1_0 = float(np.median([vmin / (k * t) for k, t in small]))
    p0 = np.log([min(t for _, t in small) * 0.1 + 1e-12, f1_0, R, max(V.max() * 0.1, 1.0)])

    def resid(lp):
        c, f1, r, q = np.exp(lp)
        return np.log(t_iss_fluid(G, t0_linear(K, V, c, f1), V, r, q)) - np.log(T)

    sol = least_squares(resid, p0, method="trf", x_scale="jac", max_nfev=4000)
    c, f1, r, q = (float(v) for v in np.exp(sol.x))
    relq = np.abs(T - t_iss_fluid(G, t0_linear(K, V, c, f1), V, r, q)) / T
    out["fluid"] = {"c": c, "f1": f1, "R": r, "Q": q,
                    "rel_err_median": float(np.median(relq)), "rel_err_max": float(relq.max())}
    return out
