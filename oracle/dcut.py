"""Oracle for ratio-budgeted verification (D-cut) and packed verification (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "AngelSpec: Towards Real-World High Performance Inference with
Speculative Decoding", section 4.1 (a request keeping n drafts contributes
n + 1 verification positions; the batch budget is K = sum (n + 1)) and
section 4.2, "D-cut: Adaptive Verification Budgeting":

* Eq. 20: the score of position k of request i is the prefix product of the
  drafter's confidences, s_{i,k} = prod_{t=1..k} c_{i,t}, with s_{i,0} = 1 for
  the bonus position;
* Eq. 21: keeping n drafts has estimated progress A_i(n) = sum_{k=0..n} s_{i,k};
* the budget is spent on the K best scores of the whole batch, equal scores
  going to shallower positions first; with non-increasing scores this keeps a
  contiguous prefix of every request;
* Eq. 22: the budget of ratio rho is K_rho(B) = max(B, ceil(rho * B * (D + 1)));
* Eq. 23: the batch progress of rho is U(B, rho) = sum_i A_i(n_i^(rho));
* Eq. 24: the ratio used is the argmax over rho of U(B, rho) / C(B, rho), with
  C a cost profiled ahead of time per (B, rho);
* "Packing and correctness": the kept prefixes form one dense batch of
  K_{rho*} positions for the target; every kept token is verified exactly as
  before, so packing changes which rows exist, not how a row is verified.

Readings (also in the design doc):

* 0-based drafts: confidence[b, t], t = 0..D-1, is the page's c_{i,t+1}.
  scores[b, 0] = 1 (bonus) and scores[b, k] = prod_{t<k} confidence[b, t] for
  k = 1..D, a left-to-right float64 product.
* A confidence outside [0, 1] is clamped into it and a NaN counts as 0, so the
  scores never increase along a request (the page's contiguity argument needs
  confidences that are probabilities).
* Order of the top-K selection: score descending, then position ascending
  (the page's shallow rule), then request ascending.
* rho is taken as given (a float32 ratio); rho * B * (D + 1) is formed in
  float64, which is exact for these sizes, then rounded up.
* The chosen ratio is the first one, in the order given, that attains the
  largest U / C (U and C in float64).
* Packed layout: request b owns rows row_offsets[b] .. row_offsets[b+1] - 1,
  its positions 0..n_b in order; row_offsets[0] = 0, row_offsets[B] = K.
"""

import math

import numpy as np

from .verify import _as_f64, verify


def clamp_confidence(confidence):
    """Confidences as float64 in [0, 1]; NaN -> 0."""
    c = np.asarray(confidence, dtype=np.float64)
    return np.where(np.isnan(c), 0.0, np.clip(c, 0.0, 1.0))


def scores(confidence):
    """Eq. 20: [B, D+1] with column 0 = 1 and column k = prod_{t<k} c[b, t], left to right."""
    c = clamp_confidence(confidence)
    B, D = c.shape
    s = np.empty((B, D + 1), dtype=np.float64)
    for b in range(B):
        acc = 1.0
        s[b, 0] = acc
        for k in range(D):
            acc = acc * c[b, k]
            s[b, k + 1] = acc
    return s


def ratio_budget(rho, B, D):
    """Eq. 22: K_rho(B) = max(B, ceil(rho * B * (D + 1))), rho taken as float32."""
    r = float(np.float32(rho))
    return max(int(B), int(math.ceil(r * float(B * (D + 1)))))


def top_k_lengths(s, K):
    """Keep depths n_b from the K best scores of s [B, D+1] (ties: shallower, then lower b)."""
    B, D1 = s.shape
    order = sorted(((b, k) for b in range(B) for k in range(D1)), key=lambda bk: (-s[bk[0], bk[1]], bk[1], bk[0]))
    kept = np.zeros((B, D1), dtype=bool)
    for b, k in order[:K]:
        kept[b, k] = True
    n = kept.sum(axis=1).astype(np.int64) - 1
    for b in range(B):
        # The kept positions of a request form the prefix 0..n_b.
        assert kept[b, : n[b] + 1].all() and not kept[b, n[b] + 1:].any(), "top-K left a hole"
    return n


def progress(s, n):
    """Eq. 21 per request: A_b(n_b) = s[b,0] + ... + s[b,n_b], summed in position order."""
    B = s.shape[0]
    out = np.empty(B, dtype=np.float64)
    for b in range(B):
        acc = 0.0
        for k in range(int(n[b]) + 1):
            acc = acc + s[b, k]
        out[b] = acc
    return out


def utility(s, n):
    """Eq. 23: U = sum over requests (in order) of their estimated progress."""
    acc = 0.0
    for a in progress(s, n):
        acc = acc + a
    return acc


def row_offsets(n):
    """Packed layout: request b owns rows off[b] .. off[b+1]-1 (n_b + 1 of them)."""
    off = np.zeros(len(n) + 1, dtype=np.int64)
    for b, nb in enumerate(n):
        off[b + 1] = off[b] + int(nb) + 1
    return off


def dcut(confidence, ratios, ratio_cost):
    """Choose the ratio budget and the keep depths (Eq. 20-24).

    confidence [B, D]; ratios [R] in (0, 1]; ratio_cost [R] > 0, the profiled
    cost C(B, rho) of each ratio at this batch size.  Returns a dict with
    verify_len [B], row_offsets [B+1], ratio_index, total_rows (K of the chosen
    ratio), and per ratio: budgets K_rho [R], utility U [R], lengths [R, B].
    """
    c = np.asarray(confidence, dtype=np.float64)
    B, D = c.shape
    s = scores(c)
    budgets, util, lens = [], [], []
    for rho in ratios:
        K = ratio_budget(rho, B, D)
        n = top_k_lengths(s, K)
        budgets.append(K)
        util.append(utility(s, n))
        lens.append(n)
    best, best_i = None, 0
    for i, cost in enumerate(ratio_cost):
        val = util[i] / float(np.float32(cost))
        if best is None or val > best:
            best, best_i = val, i
    n = lens[best_i]
    return {
        "verify_len": n,
        "row_offsets": row_offsets(n),
        "ratio_index": best_i,
        "total_rows": budgets[best_i],
        "budgets": np.asarray(budgets, dtype=np.int64),
        "utility": np.asarray(util, dtype=np.float64),
        "lengths": np.asarray(lens, dtype=np.int64).reshape(len(budgets), B),
    }


def pack_rows(target_logits, row_offsets_, rows=None):
    """Dense packed target rows: row off[b] + k holds target_logits[b, k], k = 0..n_b.

    `rows` (>= off[B]) sizes the buffer; rows past off[B] are zero.
    """
    z = np.asarray(target_logits)
    off = np.asarray(row_offsets_, dtype=np.int64)
    B = len(off) - 1
    K = int(off[B]) if rows is None else int(rows)
    out = np.zeros((K,) + z.shape[2:], dtype=z.dtype)
    for b in range(B):
        m = int(off[b + 1] - off[b])
        out[off[b]: off[b + 1]] = z[b, :m]
    return out


def verify_packed(packed_logits, row_offsets_, draft_probs, draft_tokens, uniforms, temperature):
    """Verification over packed target rows (section 4.2, "Packing and correctness").

    packed_logits [rows, V] (float, or uint16 bfloat16 bits); row_offsets [B+1]:
    request b's target rows are packed rows off[b] .. off[b+1]-1, its positions
    0..n_b with n_b = off[b+1] - off[b] - 1.  A request whose rows are not
    inside the buffer, or with n_b outside [0, D], is a data error (outputs -1).
    Each request is then verified exactly as an unpacked one with verify
    length n_b.
    """
    z = _as_f64(packed_logits)
    rows, V = z.shape
    off = np.asarray(row_offsets_, dtype=np.int64)
    B = len(off) - 1
    x = np.asarray(draft_tokens).reshape(B, -1)
    D = x.shape[1]
    full = np.zeros((B, D + 1, V), dtype=np.float64)
    n = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        lo, hi = int(off[b]), int(off[b + 1])
        nb = hi - lo - 1
        if 0 <= lo and hi <= rows and 0 <= nb <= D:
            full[b, : nb + 1] = z[lo:hi]
            n[b] = nb
    return verify(full, draft_probs, draft_tokens, uniforms, temperature, verify_len=n)
