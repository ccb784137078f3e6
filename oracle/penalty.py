"""Oracle for the contextual-penalty logit pass (penalty, temperature, top-p, min-p).

Test infrastructure only (see the package docstring).

Definition: TokenSwift summary §3.4 "Contextual Penalty and Random N-gram
Selection" (a penalty on the tokens of the most recent W positions, instead of
on every generated token), Appendix D.1 "Introduction of Different Sampling
Algorithms" (top-p: with tokens sorted by probability, the shortest head of
that order whose mass is above p, then renormalised; min-p: the tokens with
p_i >= p_base * max_j p_j), Appendix F.1 (temperature). Hyper-parameters from the
TokenSwift reproducibility checklist, Table 11 (penalty 1.2, penalty length
1024, temperature 1.0, top-p 0.9, min-p 0.05).

Readings taken where the pages are silent:

* Penalty form (repetition penalty of the CTRL line of work, listed in the
  citation map): for each DISTINCT id w in the window, a positive logit is
  divided by theta and a non-positive one multiplied by theta. Ids outside
  [0, V) are padding and ignored.
* Order: penalty, then temperature, then the top-p and min-p masks, which
  are intersected (min-p is scale-free, so applying it to the top-p
  renormalised distribution gives the same set).
* Top-p boundary: with tokens ordered by (probability desc, id asc) and E(i)
  the mass strictly before token i, keep i iff E(i) <= top_p.
* Min-p boundary is inclusive: keep i iff p_i >= min_p * max(p).
* Sampling: with caller-supplied u in [0,1), the token is the smallest id t
  whose cumulative renormalised probability (ascending ids) exceeds u.

The eta-sampling variant (Appendix D.1: the pool is the tokens whose
probability reaches eta, a quantity built from the entropy and two
constants alpha and epsilon) replaces the top-p and min-p masks. Readings:
eta = min(epsilon, alpha * exp(-H)) with H = -sum p ln p in nats (the form of
the truncation-sampling paper the citation map lists), and the most probable
token is always kept, so the pool is {i : p_i >= min(eta, max p)}.
"""

from dataclasses import dataclass

import numpy as np


@dataclass
class PenaltyResult:
    z: np.ndarray        # float64 [rows][V]; penalised, tempered logits
    p: np.ndarray        # float64 [rows][V]; softmax(z)
    keep: np.ndarray     # bool [rows][V]
    probs: np.ndarray    # float64 [rows][V]; renormalised kept probabilities
    token: np.ndarray    # int64 [rows]; -1 when no u was given
    excl_mass: np.ndarray  # float64 [rows][V]; E(i), mass strictly before i
    ratio: np.ndarray    # float64 [rows][V]; p_i / max p


def apply_penalty(x, window_ids, V, theta):
    """Windowed repetition penalty on one row (float64)."""
    y = np.array(x, dtype=np.float64)
    ids = np.asarray(window_ids, dtype=np.int64)
    ids = ids[(ids >= 0) & (ids < V)]
    w = np.unique(ids)
    vals = y[w]
    y[w] = np.where(vals > 0, vals / theta, vals * theta)
    return y


def penalty_sample(logits, window, penalty, temperature, top_p, min_p, u=None):
    """Run the logit pass on every row.

    logits: float [rows][V]. window: int [rows][W] or [W] (shared by all rows).
    u: optional float [rows] in [0, 1).
    """
    x = np.asarray(logits, dtype=np.float64)
    rows, V = x.shape
    win = np.asarray(window, dtype=np.int64)
    if win.ndim == 1:
        win = np.broadcast_to(win, (rows, win.shape[0]))
    if not (penalty > 0 and temperature > 0 and 0 <= top_p <= 1 and 0 <= min_p <= 1):
        raise ValueError("parameter out of range")

    z = np.empty_like(x)
    p = np.empty_like(x)
    keep = np.zeros(x.shape, dtype=bool)
    probs = np.zeros_like(x)
    token = np.full(rows, -1, dtype=np.int64)
    excl = np.empty_like(x)
    ratio = np.empty_like(x)
    ids = np.arange(V, dtype=np.int64)
    for r in range(rows):
        y = apply_penalty(x[r], win[r], V, float(penalty))
        zr = y / float(temperature)
        e = np.exp(zr - zr.max())
        pr = e / e.sum()
        # (p desc, id asc) order; E(i) = mass strictly before i in that order.
        order = np.lexsort((ids, -pr))
        csum = np.cumsum(pr[order])
        e_sorted = np.concatenate([[0.0], csum[:-1]])
        er = np.empty(V)
        er[order] = e_sorted
        keep_top = er <= top_p
        keep_min = pr >= min_p * pr.max()
        kr = keep_top & keep_min
        qr = np.where(kr, pr, 0.0)
        qr = qr / qr.sum()
        z[r], p[r], keep[r], probs[r], excl[r] = zr, pr, kr, qr, er
        ratio[r] = pr / pr.max()
        if u is not None:
            cdf = np.cumsum(qr)
            hits = np.nonzero(cdf > float(u[r]))[0]
            # u < 1 and the kept mass sums to 1; the guard covers rounding.
            token[r] = int(hits[0]) if len(hits) else int(np.nonzero(kr)[0][-1])
    return PenaltyResult(z=z, p=p, keep=keep, probs=probs, token=token, excl_mass=excl, ratio=ratio)


@dataclass
class EtaResult:
    z: np.ndarray        # float64 [rows][V]
    p: np.ndarray        # float64 [rows][V]
    keep: np.ndarray     # bool [rows][V]
    probs: np.ndarray    # float64 [rows][V]
    token: np.ndarray    # int64 [rows]; -1 when no u was given
    entropy: np.ndarray  # float64 [rows]; H in nats
    eta: np.ndarray      # float64 [rows]
    ratio: np.ndarray    # float64 [rows][V]; p_i / min(eta, max p), 1 at the cutoff


def eta_sample(logits, window, penalty, temperature, epsilon, alpha, u=None):
    """The logit pass with eta-sampling in place of top-p and min-p."""
    x = np.asarray(logits, dtype=np.float64)
    rows, V = x.shape
    win = np.asarray(window, dtype=np.int64)
    if win.ndim == 1:
        win = np.broadcast_to(win, (rows, win.shape[0]))
    if not (penalty > 0 and temperature > 0 and 0 < epsilon <= 1 and alpha >= 0):
        raise ValueError("parameter out of range")
    out = dict(z=np.empty_like(x), p=np.empty_like(x), keep=np.zeros(x.shape, dtype=bool), probs=np.zeros_like(x),
               token=np.full(rows, -1, dtype=np.int64), entropy=np.empty(rows), eta=np.empty(rows),
               ratio=np.empty_like(x))
    for r in range(rows):
        zr = apply_penalty(x[r], win[r], V, float(penalty)) / float(temperature)
        e = np.exp(zr - zr.max())
        pr = e / e.sum()
        nz = pr > 0
        H = -np.sum(pr[nz] * np.log(pr[nz]))
        eta = min(float(epsilon), float(alpha) * np.exp(-H))
        thr = min(eta, pr.max())
        kr = pr >= thr
        qr = np.where(kr, pr, 0.0)
        qr = qr / qr.sum()
        out["z"][r], out["p"][r], out["keep"][r], out["probs"][r] = zr, pr, kr, qr
        with np.errstate(divide="ignore"):   # thr = 0 when alpha = 0: every ratio is +inf, far from the cutoff
            out["entropy"][r], out["eta"][r], out["ratio"][r] = H, eta, pr / thr
        if u is not None:
            cdf = np.cumsum(qr)
            hits = np.nonzero(cdf > float(u[r]))[0]
            out["token"][r] = int(hits[0]) if len(hits) else int(np.nonzero(kr)[0][-1])
    return EtaResult(**out)
