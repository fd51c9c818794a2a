"""Oracle for greedy tree verification (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "breaking down dspark and its lineage", section "Tree attention"
(and "Prefill, decode, and trees on both sides"): a drafter may propose
several continuations per step, arranged as a tree rooted at the last
committed token, where a node's parent is the token it extends.  One target
pass over the flattened tree, with attention restricted to each node's
ancestors, gives every node the distribution it would get on its own
root-to-node path; verification then keeps the one candidate path the target
agrees with.
"UraionSpec", "Future work", names tree verification for autoregressive
drafters.

What is built is the acceptance walk after the target pass, in the greedy
(temperature 0) limit, which is the case the pages fix exactly:

* node 0 is the root (the last committed token); node i >= 1 carries token
  tok[i] and parent par[i] < i.  Row i of the target logits is the target's
  next-token distribution after the path root..i;
* from the root, the walk moves to the child of the current node whose token
  equals the target's lowest-index argmax at the current node (the
  lowest-numbered such child if several carry it), and stops when no child
  matches;
* the emitted tokens are the tokens of the accepted path, then the argmax at
  its last node (the bonus).  This is exactly what greedy decoding of the
  target would emit, for any tree.

Readings (also in the design doc):

* The walk visits rows root, path[1], ..., last node.  A visited row holding a
  NaN, whose maximum is +inf or which is entirely -inf is a data error (outputs
  -1), as is a parent outside [0, i) or a token outside [0, V) for some node
  i >= 1.  Rows that are not visited are not checked.
* Sampled (T > 0) lossless acceptance over several candidates per position
  needs a multi-candidate rejection rule that the pages do not give; it is not
  built.
"""

import numpy as np

from .verify import _as_f64, row_is_bad


def tree_verify_greedy(target_logits, parents, tokens):
    """Greedy walk over a candidate tree per request.

    target_logits [B, M, V] (float or uint16 bfloat16 bits); parents [B, M]
    (parents[:, 0] ignored); tokens [B, M] (tokens[:, 0] ignored).
    Returns a dict: accepted [B] (path length, -1 on a data error),
    tokens [B, M] (accepted tokens, then the bonus, then -1), path [B, M]
    (accepted node indices after the root, then -1).
    """
    z = _as_f64(target_logits)
    B, M, V = z.shape
    par = np.asarray(parents, np.int64).reshape(B, M)
    tok = np.asarray(tokens, np.int64).reshape(B, M)
    acc = np.full(B, -1, np.int64)
    out_tok = np.full((B, M), -1, np.int64)
    out_path = np.full((B, M), -1, np.int64)
    bad_row = row_is_bad(z)
    for b in range(B):
        nodes = range(1, M)
        if any(not (0 <= par[b, i] < i) or not (0 <= tok[b, i] < V) for i in nodes):
            continue
        cur, path, emitted, bad = 0, [], [], False
        while True:
            if bad_row[b, cur]:
                bad = True
                break
            a = int(np.argmax(z[b, cur]))          # the first maximal index
            nxt = next((i for i in nodes if par[b, i] == cur and tok[b, i] == a), None)
            if nxt is None:
                emitted.append(a)
                break
            path.append(nxt)
            emitted.append(a)
            cur = nxt
        if bad:
            continue
        acc[b] = len(path)
        out_tok[b, : len(emitted)] = emitted
        out_path[b, : len(path)] = path
    return {"accepted": acc, "tokens": out_tok, "path": out_path}


def chain(G):
    """Parents of a single chain of G drafts (node k+1 follows node k)."""
    return np.arange(-1, G, dtype=np.int64)
