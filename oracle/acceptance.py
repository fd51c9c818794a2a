"""Oracle for draft-logits verification and per-position acceptance diagnostics (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (by page title and section):

* "AngelSpec: Towards Real-World High Performance Inference with Speculative
  Decoding", section 2, Eq. 2: the drafter's distribution at depth k is a
  softmax over the vocabulary of its logits, and the draft token is taken from
  it; Eq. 4: TV(p, q) = 1/2 sum_v |p(v) - q(v)|; Eq. 5: under rejection-sampling
  verification the expected acceptance probability of one position is the
  overlap alpha(p, q) = sum_v min(p(v), q(v)) = 1 - TV(p, q).
* "breaking down dspark and its lineage", section "Preserving the target
  distribution during verification": the worked example's overlap is 0.8.
* "UraionSpec: A Faithful Implementation of Confidence-Scheduled Speculative
  Decoding", section on the confidence head: its training target is
  c*_k = 1 - 1/2 ||p_d - p_t||_1, the conditional probability that draft k is
  accepted, which is the same overlap.

Readings (also in the design doc):

* Draft-logits mode: the draft distribution is q_k = softmax(d_k / T) with the
  call's temperature T (the drafter samples at the temperature the target is
  verified at); with draft probabilities given instead, q is used as given.
* A verified draft row (k < n_b) that holds a NaN, whose maximum is +inf, or
  which is entirely -inf is a data error of its request, like a target row.
* The diagnostics cover the tested positions k < n_b.  alpha_k depends only on
  target row k and draft row k, so it is NaN when either of those rows is bad
  (NaN, maximum +inf, or all -inf), for k >= n_b, and for every position of a
  request whose verify length is outside [0, G].  TV and c* are 1 - alpha and
  alpha; only alpha is returned.  Draft ids play no part.
* Diagnostics are defined for T > 0 (at T = 0 p and q are one-hot).
"""

import numpy as np

from .verify import _as_f64, row_is_bad, target_probs, verify, verify_greedy


def draft_probs_from_logits(draft_logits, temperature):
    """q = softmax(d / T) along the last axis in float64 (Eq. 2 at temperature T)."""
    q, _ = target_probs(_as_f64(draft_logits), float(temperature))
    return q


def total_variation(p, q):
    """Eq. 4: 1/2 sum |p - q| along the last axis."""
    return 0.5 * np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum(axis=-1)


def overlap(p, q):
    """Eq. 5: sum min(p, q) along the last axis."""
    return np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum(axis=-1)


def _draft_rows_bad(d, n):
    """Per request: does a verified draft row (k < n_b) hold a bad row?"""
    B, G = d.shape[:2]
    used = np.arange(G)[None, :] < n[:, None]
    return (row_is_bad(d) & used).any(axis=1)


def acceptance(target_logits, draft, temperature, verify_len=None, draft_is_logits=False):
    """alpha[b, k] = sum_v min(p_k(v), q_k(v)) for k < n_b, else NaN.

    target_logits [B, G+1, V] (float or uint16 bfloat16 bits); draft [B, G, V]:
    draft probabilities, or draft logits when draft_is_logits (softmax at T).
    """
    z = _as_f64(target_logits)
    B, G1, V = z.shape
    G = G1 - 1
    T = float(temperature)
    if not T > 0.0:
        raise ValueError("acceptance diagnostics need T > 0")
    n = np.full(B, G, np.int64) if verify_len is None else np.asarray(verify_len, np.int64).reshape(B)
    tested = (np.arange(G)[None, :] < n[:, None]) & ((n >= 0) & (n <= G))[:, None]
    bad_pos = row_is_bad(z[:, :G])
    if draft_is_logits:
        d = _as_f64(draft).reshape(B, G, V)
        bad_pos = bad_pos | row_is_bad(d)
        q = draft_probs_from_logits(d, T)
    else:
        q = np.asarray(draft, np.float64).reshape(B, G, V)
    p, _ = target_probs(z[:, :G], T)
    alpha = overlap(p, q)
    return np.where(tested & ~bad_pos, alpha, np.nan)


def verify_logits(target_logits, draft_logits, draft_tokens, uniforms, temperature, verify_len=None):
    """Verification with the draft distribution given as logits: q = softmax(d / T).

    A verified draft row that is bad (NaN, max +inf, all -inf) is a data error
    of its request.  Temperature 0 ignores the draft logits (greedy limit).
    """
    if float(temperature) == 0.0:
        return verify_greedy(target_logits, draft_tokens, verify_len)
    z = np.asarray(target_logits)
    B, G1, V = z.shape
    G = G1 - 1
    d = _as_f64(draft_logits).reshape(B, G, V)
    q = draft_probs_from_logits(d, temperature) if G > 0 else np.zeros((B, 0, V))
    out = verify(target_logits, q, draft_tokens, uniforms, temperature, verify_len)
    n = np.full(B, G, np.int64) if verify_len is None else np.asarray(verify_len, np.int64).reshape(B)
    nn = np.clip(n, 0, G)
    bad = _draft_rows_bad(d, nn) & (n >= 0) & (n <= G)
    if bad.any():
        out["accepted"][bad] = -1
        out["tokens"][bad] = -1
        for key in ("lse", "p_draft", "q_draft"):
            out[key][bad] = np.nan
        out["resid_mass"][bad] = np.nan
    return out
