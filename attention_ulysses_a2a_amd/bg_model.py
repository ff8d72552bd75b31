"""Burst-Gap model and fit used by the microbenchmark driver (host-side analysis).

Model (X-Stage explainer, gist.science, arXiv 2607.23264, technical summary,
"Methodology"): the issuer-visible time to issue a burst of aggregate volume V from K
producers after a useful gap G is T_iss(G; K, V) = max(T0_iss(K, V), V / R - G).  The
formula itself is evaluated by the library (``xstage_bg_t_iss``); this module fits its
parameters to measured sweeps and, as a labelled extension, fits a capacity Q through a
fluid-queue reading T_iss = max(T0, V/R - min(G, Q/R)) with T0 = c + V / (K f1).
"""

from __future__ import annotations

import numpy as np

from . import xstage_bg_t_iss


def t_iss(G, T0, V, R):
    """Vectorised wrapper of the library's Burst-Gap formula."""
    G, T0, V = np.broadcast_arrays(np.asarray(G, float), np.asarray(T0, float), np.asarray(V, float))
    out = np.empty(G.shape)
    for idx in np.ndindex(G.shape):
        out[idx] = xstage_bg_t_iss(G[idx], T0[idx], V[idx], R)
    return out


def t_iss_capacity(G, T0, V, R, Q):
    """Fluid-queue reading with pending capacity Q (extension; equals the formula for G <= Q/R)."""
    return t_iss(np.minimum(np.asarray(G, float), Q / R), T0, V, R)


def fit(points, drain_margin: float = 1.1):
    """Fit (T0 per (K, V), R) of the printed formula, then (c, f1, R, Q) of the reading.

    points: iterable of (K, V_bytes, G_s, T_iss_s).
    1. T0(K, V): median issue time at the longest measured gap for that (K, V).
    2. R: the points above drain_margin * T0 sit on T_iss + G = V / R; least squares
       through the origin of (T_iss + G) on V.
    3. Capacity reading: least squares on log T_iss of max(c + V/(K f1), V/R - min(G, Q/R)).
    """
    from scipy.optimize import least_squares

    pts = np.asarray(list(points), dtype=float)
    K, V, G, T = pts.T
    t0 = {}
    for k, v in sorted(set(zip(K.tolist(), V.tolist()))):
        sel = (K == k) & (V == v)
        gmax = G[sel].max()
        t0[(k, v)] = float(np.median(T[sel & (G == gmax)]))
    t0_arr = np.array([t0[(k, v)] for k, v in zip(K.tolist(), V.tolist())])
    drain = T > drain_margin * t0_arr
    res = {"T0": {f"K{int(k)}_V{int(v)}": val for (k, v), val in t0.items()}, "n_points": int(len(T)),
           "n_drain": int(drain.sum()), "R": None}
    if not drain.any():
        return res
    R = float(np.dot(V[drain], V[drain]) / np.dot(V[drain], T[drain] + G[drain]))
    res["R"] = R
    rel = np.abs(T - t_iss(G, t0_arr, V, R)) / T
    res["rel_err_median"] = float(np.median(rel))
    res["rel_err_max"] = float(rel.max())
    gmax_of = np.array([G[(K == k) & (V == v)].max() for k, v in zip(K.tolist(), V.tolist())])
    pred = G < gmax_of  # points not used to read T0
    if pred.any():
        res["rel_err_median_predicted"] = float(np.median(rel[pred]))
        res["rel_err_p90_predicted"] = float(np.percentile(rel[pred], 90))

    vmin = V.min()
    f1_0 = float(np.median([vmin / (k * t0[(k, vmin)]) for k in sorted(set(K.tolist()))]))
    c_0 = max(1e-9, 0.1 * min(t0[(k, vmin)] for k in sorted(set(K.tolist()))))

    def model(p):
        c, f1, r, q = np.exp(p)
        base = c + V / (K * f1)
        return np.maximum(base, V / r - np.minimum(G, q / r))

    sol = least_squares(lambda p: np.log(model(p)) - np.log(T), np.log([c_0, f1_0, R, max(1.0, 0.1 * V.max())]),
                        method="trf", x_scale="jac", max_nfev=4000)
    c, f1, r, q = (float(x) for x in np.exp(sol.x))
    relq = np.abs(T - model(sol.x)) / T
    res["capacity_reading"] = {"c_s": c, "f1_Bps": f1, "R_Bps": r, "Q_bytes": q,
                               "rel_err_median": float(np.median(relq)), "rel_err_max": float(relq.max())}
    return res


def fit_isolated(V, T, T0, R=None, margin: float = 1.5):
    """Capacity Q from bursts issued on an empty queue (capacity reading: T = max(T0, (V - Q)/R)).

    Points with T > margin * T0 lie on T = (V - Q) / R: a least-squares line T = a + b V
    gives R_iso = 1/b and Q_iso = -a/b; with a drain rate R from the periodic sweep,
    Q = median(V - R T)."""
    V, T, T0 = (np.asarray(x, float) for x in (V, T, T0))
    use = T > margin * T0
    res = {"n_used": int(use.sum())}
    if len(set(V[use].tolist())) < 2:
        return res
    b, a = np.polyfit(V[use], T[use], 1)
    res["R_iso_Bps"] = float(1.0 / b)
    res["Q_iso_bytes"] = float(-a / b)
    if R is not None:
        res["Q_bytes_at_R"] = float(np.median(V[use] - R * T[use]))
    return res


def fit_synchronized(large, isolated, c, f1, K, margin: float = 1.5):
    """Fits of the series whose producers start every round together (one aggregate burst).

    large: (V, G, T) of periodic bursts; isolated: (V, T[, start spread]) of bursts on a
    drained queue; T0 = c + V / (K f1), the backpressure-free issue time from the
    unsynchronised sweep (plus, for an isolated burst, the spread of its producers' starts).
    * R_agg: least squares of V = R T over the zero-gap periodic points;
    * the printed formula max(T0, V/R_agg - G) and the capacity reading
      max(T0, V/R_agg - min(G, Q/R_agg)) against the periodic points with G > 0 (median
      relative error each; Q from the isolated fit);
    * the isolated fit (``fit_isolated``) with R = R_agg."""
    L = np.asarray(large, float)
    V, G, T = L.T
    z = G == 0
    R = float(np.dot(V[z], V[z]) / np.dot(V[z], T[z]))
    iso = np.asarray(isolated, float)
    # An aggregate burst cannot be issued before its last producer has started and issued
    # its own share freely: its free time is the start spread plus c + V / (K f1).
    spread = iso[:, 2] if iso.shape[1] > 2 else 0.0
    t0_iso = c + iso[:, 0] / (K * f1) + spread
    fi = fit_isolated(iso[:, 0], iso[:, 1], t0_iso, R=R, margin=margin)
    res = {"R_agg_Bps": R, "isolated": fi}
    Q = fi.get("Q_bytes_at_R")
    g = G > 0
    t0 = c + V[g] / (K * f1)
    page = np.maximum(t0, V[g] / R - G[g])
    res["page_formula_rel_err_median"] = float(np.median(np.abs(T[g] - page) / T[g]))
    if Q is not None:
        cap = np.maximum(t0, V[g] / R - np.minimum(G[g], max(Q, 0.0) / R))
        res["capacity_reading_rel_err_median"] = float(np.median(np.abs(T[g] - cap) / T[g]))
    return res
