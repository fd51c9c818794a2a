"""Oracle for batched lossless speculative-sampling verification (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is used by
the HIP library; nothing here imports it.

What is computed (sources, by page title and section):

* "breaking down dspark and its lineage", section "Speculative decoding basics:
  drafting and verification": one causal target pass over
  [prefix, x_1..x_gamma] yields gamma+1 conditionals, so the target logits of
  one request are gamma+1 rows over the vocabulary; row k is the target's
  distribution for the token after k accepted drafts.
* same page, section "Preserving the target distribution during verification":
  the two-case rule -- p(x) >= q(x): keep the draft; p(x) < q(x): keep it with
  probability p(x)/q(x), otherwise reject and draw from the normalised part of
  p that sticks up above q, i.e. max(p - q, 0) / sum.
* "UraionSpec: A Faithful Implementation of Confidence-Scheduled Speculative
  Decoding", section "Speculative Decoding", Eq. (acceptance): accept x_k with
  probability min(1, p_t/p_d); the first rejection ends the accepted prefix.
* "AngelSpec: Towards Real-World High Performance Inference with Speculative
  Decoding", section 1 and section 4.1: the verified prefix is committed
  together with one target-generated token; when every kept draft survives,
  that token is the bonus token drawn from the target at the next position.

Readings where the pages are silent (each also listed in the design doc):

* Temperature softmax of the target row: p_k(v) = exp((z_kv - m_k)/T) /
  sum_w exp((z_kw - m_k)/T) with m_k the row maximum; T applies to the target
  logits only, the draft probabilities are used as given (they are the
  distribution the drafter sampled from).
* Uniforms are laid out [B, G+1]: u[b, k] (k < G) decides draft k; u[b, G] is the
  single draw for the correction or bonus token, whatever the verify length.
* Accept iff u < p(x)/q(x) (strict, u in [0,1)); when q(x) is not positive the
  draft is accepted iff p(x) > 0.
* Inverse CDF over ascending token index: y = min{v : C(v) > u * R} with C the
  running sum and R = C(V-1); if no index qualifies (rounding at the top end)
  y is the largest index with positive mass.  Zero-mass tokens are never drawn.
* If the residual mass is zero (only possible through rounding) the draw falls
  back to p_j itself.
* Verify length n_b <= G: only positions k < n_b are tested, the bonus row is
  row n_b, rows beyond n_b are never used.
* Data errors (the request's outputs are all -1): n_b outside [0, G]; a draft
  id outside [0, V) at a tested position; a used row (k <= n_b) that holds a
  NaN, whose maximum is +inf, or which is entirely -inf.
* Temperature 0 is the greedy limit: a_k = lowest index attaining the row
  maximum (exact comparison), accept iff x_k == a_k, the emitted token is a_j
  at the first mismatch j (or a_n when all match).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bfloat16 values stored as uint16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _as_f64(logits):
    a = np.asarray(logits)
    if a.dtype == np.uint16:  # bfloat16 bit patterns
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def row_is_bad(z):
    """True where a logit row (last axis) holds a NaN, has max +inf, or is all -inf."""
    z = np.asarray(z, dtype=np.float64)
    has_nan = np.isnan(z).any(axis=-1)
    m = np.where(np.isnan(z), -np.inf, z).max(axis=-1)
    return has_nan | (m == np.inf) | (m == -np.inf)


def target_probs(z, temperature):
    """Temperature softmax over the last axis in float64; also returns log-sum-exp.

    p(v) = exp((z_v - m)/T) / S,  S = sum_v exp((z_v - m)/T),  lse = m/T + ln S.
    """
    z = np.asarray(z, dtype=np.float64)
    T = float(temperature)
    with np.errstate(all="ignore"):
        m = z.max(axis=-1, keepdims=True)
        e = np.exp((z - m) / T)
        S = e.sum(axis=-1, keepdims=True)
        p = e / S
        lse = m[..., 0] / T + np.log(S[..., 0])
    return p, lse


def accept_draft(p_x, q_x, u):
    """Two-case acceptance: keep the draft iff u < p(x)/q(x); q(x) <= 0 keeps iff p(x) > 0."""
    p_x = np.asarray(p_x, dtype=np.float64)
    q_x = np.asarray(q_x, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(all="ignore"):
        return np.where(q_x > 0, u < p_x / q_x, p_x > 0)


def residual(p, q):
    """The part of p that sticks up above q: max(p - q, 0) (unnormalised)."""
    return np.maximum(np.asarray(p, np.float64) - np.asarray(q, np.float64), 0.0)


def inverse_cdf(r, u):
    """Draw from unnormalised masses r (last axis) with uniforms u.

    y = min{v : C(v) > u * C(V-1)}, C the running sum in ascending index order;
    when no index qualifies, the largest index with r > 0.  Returns (y, R).
    """
    r = np.asarray(r, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    C = np.cumsum(r, axis=-1)
    R = C[..., -1]
    t = u * R
    above = C > t[..., None]
    first = above.argmax(axis=-1)
    pos = r > 0
    V = r.shape[-1]
    last_pos = V - 1 - pos[..., ::-1].argmax(axis=-1)
    y = np.where(above.any(axis=-1), first, np.where(pos.any(axis=-1), last_pos, -1))
    return y.astype(np.int64), R


def _first_true(mask, default):
    """Index of the first True along the last axis, else `default` (works for zero length)."""
    if mask.shape[-1] == 0:
        return np.asarray(default, dtype=np.int64).copy()
    return np.where(mask.any(axis=-1), mask.argmax(axis=-1), default).astype(np.int64)


def _prepare(target_logits, draft_tokens, verify_len):
    z = _as_f64(target_logits)
    if z.ndim != 3:
        raise ValueError("target_logits must be [B, G+1, V]")
    B, G1, V = z.shape
    G = G1 - 1
    x = np.asarray(draft_tokens, dtype=np.int64).reshape(B, G)
    if verify_len is None:
        n = np.full(B, G, dtype=np.int64)
    else:
        n = np.asarray(verify_len, dtype=np.int64).reshape(B)
    bad = (n < 0) | (n > G)
    nn = np.clip(n, 0, G)
    rows_used = np.arange(G1)[None, :] <= nn[:, None]          # rows 0..n_b
    pos_used = np.arange(G)[None, :] < nn[:, None]             # drafts 0..n_b-1
    bad = bad | (row_is_bad(z) & rows_used).any(axis=1)
    bad = bad | (((x < 0) | (x >= V)) & pos_used).any(axis=1)
    return z, x, nn, pos_used, bad


def _emit(x, j, y, bad):
    B, G = x.shape
    acc = np.where(bad, -1, j).astype(np.int64)
    tok = np.full((B, G + 1), -1, dtype=np.int64)
    for b in range(B):
        if bad[b]:
            continue
        tok[b, : j[b]] = x[b, : j[b]]
        tok[b, j[b]] = y[b]
    return acc, tok


def verify(target_logits, draft_probs, draft_tokens, uniforms, temperature, verify_len=None):
    """Verify one batch of draft blocks.

    target_logits [B, G+1, V] (float array, or uint16 = bfloat16 bits);
    draft_probs [B, G, V]; draft_tokens [B, G]; uniforms [B, G+1];
    temperature T >= 0 (0 = greedy limit); verify_len [B] or None (= G).

    Returns a dict: accepted [B] (-1 on a data error), tokens [B, G+1]
    (accepted drafts, then the correction/bonus token, then -1), and the
    diagnostics lse [B, G+1], p_draft [B, G], q_draft [B, G] (NaN where not
    used), resid_mass [B] (R at the rejection row, -1 when nothing was rejected).
    """
    if float(temperature) == 0.0:
        return verify_greedy(target_logits, draft_tokens, verify_len)
    z, x, n, pos_used, bad = _prepare(target_logits, draft_tokens, verify_len)
    B, G1, V = z.shape
    G = G1 - 1
    T = float(temperature)
    if G > 0:
        q = np.asarray(draft_probs, dtype=np.float64).reshape(B, G, V)
    else:
        q = np.zeros((B, 0, V))
    u = np.asarray(uniforms, dtype=np.float64).reshape(B, G1)

    # Target conditionals for every row (rows beyond n_b are computed but unused).
    p, lse = target_probs(z, T)

    # Accept test at every drafted position.
    xs = np.clip(x, 0, V - 1)
    px = np.take_along_axis(p[:, :G, :], xs[..., None], axis=2)[..., 0]
    qx = np.take_along_axis(q, xs[..., None], axis=2)[..., 0]
    acc_k = accept_draft(px, qx, u[:, :G])

    # First rejection among the tested positions, else n_b.
    rej = ~acc_k & pos_used
    j = _first_true(rej, n)
    rejected = j < n

    # The one distribution the final token is drawn from.
    rows = np.arange(B)
    pj = p[rows, j]
    if G > 0:
        qj = q[rows, np.minimum(j, G - 1)]
        r = np.where(rejected[:, None], residual(pj, qj), pj)
    else:
        r = pj
    y, R = inverse_cdf(r, u[:, G])
    fallback = rejected & ~(R > 0)
    if fallback.any():
        y_fb, _ = inverse_cdf(pj, u[:, G])
        y = np.where(fallback, y_fb, y)

    acc, tok = _emit(x, j, y, bad)
    nanG1 = np.arange(G1)[None, :] > n[:, None]
    diag = {
        "lse": np.where(nanG1, np.nan, lse),
        "p_draft": np.where(pos_used, px, np.nan),
        "q_draft": np.where(pos_used, qx, np.nan),
        "resid_mass": np.where(rejected, R, -1.0),
    }
    for key in ("lse", "p_draft", "q_draft"):
        diag[key][bad] = np.nan
    diag["resid_mass"][bad] = np.nan
    return {"accepted": acc, "tokens": tok, **diag}


def verify_greedy(target_logits, draft_tokens, verify_len=None):
    """Temperature-0 limit: argmax match with lowest-index ties, first mismatch, target argmax."""
    z, x, n, pos_used, bad = _prepare(target_logits, draft_tokens, verify_len)
    B, G1, V = z.shape
    G = G1 - 1
    a = z.argmax(axis=2)                      # numpy returns the first maximal index
    miss = (x != a[:, :G]) & pos_used
    j = _first_true(miss, n)
    y = a[np.arange(B), j]
    acc, tok = _emit(x, j, y, bad)
    return {"accepted": acc, "tokens": tok, "argmax": a}
