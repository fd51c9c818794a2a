"""Oracle for confidence-scheduled verification depth (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (by page title and section):

* "AngelSpec: Towards Real-World High Performance Inference with Speculative
  Decoding", section 4.2, Eq. 19-21: expected progress of keeping n drafts is
  1 + sum_{k<=n} Pr(L >= k); the survival Pr(L >= k) is estimated by the
  prefix product of per-position confidences, s_k = prod_{t<=k} c_t, s_0 = 1;
  selecting the globally best scores with ties toward shallower positions
  keeps contiguous prefixes.  Section 4.1: keeping n_i drafts costs n_i + 1
  verification positions, and the batch total is K = sum (n_i + 1).
* "UraionSpec: A Faithful Implementation of Confidence-Scheduled Speculative
  Decoding", section "Hardware-Aware Prefix Scheduler", Algorithm 1: candidates
  with survival above epsilon, sorted by survival, extend a request's prefix
  only contiguously; start from one anchor per request; keep an extension
  while the throughput Theta = tau * SPS(tokens) strictly improves, stop at the
  first one that does not.
* "breaking down dspark and its lineage", section "Verify smarter, not longer":
  tokens are added only while their expected benefit outweighs the loss in
  steps per second of the larger verification batch.

Readings (also in the design doc):

* The loop index j of Algorithm 1 is 0-based: candidate (b, k) keeps draft k+1
  and carries s_{b,k} = prod_{t=0..k} c[b, t]; it is contiguous iff len_b == k.
* The token count T starts at B (one anchor per request) and grows by one per
  kept draft; SPS(T) = 1 / cost[T], so Theta = tau / cost[T].
* Sort key: survival descending, then position ascending, then request
  ascending.  Theta must improve strictly.  A batch token budget caps T: the
  scan stops (T only grows) once T + 1 would exceed it.
* Products, sums and ratios are float64 in the order the algorithm states.
"""

import itertools

import numpy as np


def survival(confidence):
    """s[b, k] = prod_{t=0..k} c[b, t] in float64, left to right."""
    c = np.asarray(confidence, dtype=np.float64)
    B, G = c.shape
    s = np.empty((B, G), dtype=np.float64)
    for b in range(B):
        acc = 1.0
        for k in range(G):
            acc = acc * c[b, k]
            s[b, k] = acc
    return s


def schedule(confidence, cost_table, token_budget, eps=0.0):
    """Greedy prefix scheduler.  Returns (len [B] int64, T int, tau float)."""
    c = np.asarray(confidence, dtype=np.float64)
    B, G = c.shape
    cost = [float(v) for v in np.asarray(cost_table, dtype=np.float64)]
    s = survival(c)
    cands = [(b, k) for b in range(B) for k in range(G) if s[b, k] > eps]
    cands.sort(key=lambda bk: (-s[bk[0], bk[1]], bk[1], bk[0]))
    length = [0] * B
    T = B
    tau = float(B)
    best = tau / cost[T]
    for b, k in cands:
        if length[b] != k:
            continue                      # not contiguous: skip
        if T + 1 > token_budget:
            break                         # budget reached
        theta = (tau + s[b, k]) / cost[T + 1]
        if theta > best:
            length[b] = k + 1
            T += 1
            tau = tau + s[b, k]
            best = theta
        else:
            break                         # throughput saturated
    return np.asarray(length, dtype=np.int64), T, tau


def schedule_value(confidence, cost_table, lengths):
    """Theta = (B + sum of kept survivals) / cost[T] for given lengths (exact objective)."""
    s = survival(confidence)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = s.shape[0]
    tau = float(B) + sum(float(s[b, :lengths[b]].sum()) for b in range(B))
    T = int(B + lengths.sum())
    return tau / float(np.asarray(cost_table, dtype=np.float64)[T]), T, tau


def brute_force(confidence, cost_table, token_budget):
    """Best Theta over every allocation len in {0..G}^B with T <= budget (tiny B, G only)."""
    c = np.asarray(confidence, dtype=np.float64)
    B, G = c.shape
    best = None
    for lens in itertools.product(range(G + 1), repeat=B):
        T = B + sum(lens)
        if T > token_budget:
            continue
        val, _, _ = schedule_value(c, cost_table, lens)
        if best is None or val > best[0]:
            best = (val, lens)
    return best
