"""Oracle for calibrated and static scheduling (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (by page title and section):

* "UraionSpec: A Faithful Implementation of Confidence-Scheduled Speculative
  Decoding", section "Sequential Temperature Scaling" (both places it appears):
  the calibrated score of position k is c~_k = c_k^(1/T_k).  T_k is fitted left
  to right: with the positions before k already calibrated, the cumulative
  survival a_k(T) = prod_{j<k} c~_j * c_k^(1/T) is compared with the empirical
  cumulative acceptance labels.  The fit keeps the T of a 100-point grid over
  (0.1, 10) with the least expected calibration error over 15 bins.  The
  scaling preserves order.  The same page provides a static scheduler with a
  fixed-length mode and a static-threshold mode.
* "breaking down dspark and its lineage", section "Verify smarter, not
  longer": a static threshold on the per-position confidence.  Threshold zero
  is fixed-length verification.

Readings (also in the design doc):

* 0-based positions: conf[:, k] is the confidence of draft k+1, and its
  cumulative label is 1 when at least k+1 drafts were accepted (acc_len > k).
* c~ = float32(2^(log2(c) / T)), the power formed in float64 and rounded to
  float32, the precision the schedulers read confidences in.  c = 0 gives 0,
  c = 1 gives 1.
* The grid is numpy.linspace(0.1, 10.0, 100), step 0.1 with T = 1 on it, each
  point taken as the float32 the library is given.  Equal ECE keeps the first
  (smallest) T.
* ECE over 15 equal-width bins on [0, 1]: bin = min(floor(15 a), 14).
  ECE = (1/N) sum_bins |sum_{i in bin} a_i - sum_{i in bin} y_i|, the
  count-weighted gap between mean prediction and mean label.  The survival
  used for later positions is the float64 product of the fitted powers, not
  rounded to float32.
* The fit takes confidences clamped into [0, 1] (NaN as 0).
* Static threshold: a request keeps its leading drafts whose (calibrated)
  confidence exceeds tau.  len_b = the first k with c~[b, k] <= tau, else G.
* Fixed length: len_b = min(L, G) for every request.
"""

import numpy as np


def power(c, T):
    """c^(1/T) in float64 as 2^(log2(c) / T) (0 -> 0, 1 -> 1)."""
    c = np.asarray(c, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.exp2(np.log2(c) / np.float64(T))


def sts_apply(conf, temps):
    """Calibrated confidences c~[b, k] = float32(c[b, k]^(1/T_k))."""
    c = np.asarray(conf, np.float32)
    T = np.asarray(temps, np.float32).astype(np.float64)
    out = np.empty(c.shape, np.float32)
    for k in range(c.shape[1]):
        out[:, k] = power(c[:, k], T[k]).astype(np.float32)
    return out


def grid(lo=0.1, hi=10.0, n=100):
    return np.linspace(lo, hi, n)


def ece(pred, label, bins=15):
    """Expected calibration error of predictions in [0, 1] against 0/1 labels."""
    a = np.asarray(pred, np.float64)
    y = np.asarray(label, np.float64)
    idx = np.minimum(np.floor(a * bins).astype(np.int64), bins - 1)
    total = 0.0
    for bi in range(bins):
        m = idx == bi
        if m.any():
            total = total + abs(float(a[m].sum()) - float(y[m].sum()))
    return total / len(a)


def sts_fit(conf, acc_len, temps=None, bins=15, return_ece=False):
    """Fit T_k left to right (Sequential Temperature Scaling).

    conf [N, G] raw confidences, acc_len [N] accepted draft counts (0..G).
    Returns T [G] (float64 grid values), and the ECE of every grid point per
    position if return_ece.
    """
    c = np.asarray(conf, np.float32).astype(np.float64)
    c = np.clip(np.where(np.isnan(c), 0.0, c), 0.0, 1.0)
    L = np.asarray(acc_len, np.int64)
    N, G = c.shape
    temps = np.asarray(grid() if temps is None else temps, np.float32).astype(np.float64)
    prefix = np.ones(N, np.float64)
    fitted = np.empty(G, np.float64)
    table = np.empty((G, len(temps)), np.float64)
    for k in range(G):
        y = (L > k).astype(np.float64)
        best, best_t = None, 0
        for ti, T in enumerate(temps):
            e = ece(prefix * power(c[:, k], T), y, bins)
            table[k, ti] = e
            if best is None or e < best:
                best, best_t = e, ti
        fitted[k] = temps[best_t]
        prefix = prefix * power(c[:, k], fitted[k])
    return (fitted, table) if return_ece else fitted


def static_fixed(B, G, length):
    """Fixed-length mode: every request verifies min(L, G) drafts."""
    return np.full(B, min(max(int(length), 0), G), np.int64)


def static_threshold(conf, tau):
    """Static-threshold mode: leading drafts whose confidence exceeds tau."""
    c = np.asarray(conf, np.float32).astype(np.float64)
    B, G = c.shape
    out = np.empty(B, np.int64)
    for b in range(B):
        n = 0
        while n < G and c[b, n] > float(np.float32(tau)):
            n += 1
        out[b] = n
    return out
