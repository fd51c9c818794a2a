"""Seeded synthetic inputs for the verification and scheduling path.

Shared by the tests and bench.py, and by nothing else.  This module holds no
verification or scheduling arithmetic: it only draws random numbers and plays
the drafter (a temperature softmax of noisy logits, sampled with numpy's
``Generator.choice``; a greedy drafter's argmax).  Every stream is a separate
``numpy.random.Philox`` key derived from (seed, stream id), so the same seed
gives the same bytes.

Recipes (the value distributions are readings of the workload descriptions;
the design doc lists them):

  tiny       B=4, G=4, V=1024, fp32 logits ~ N(0, 2) (standard deviation 2);
             draft logits = target + N(0, 0.5); T = 1.  Plus the V=3 worked
             example p=(0.5,0.3,0.2), q=(0.4,0.5,0.1).
  mtp        B=16, G=3, V=32000, bf16 logits ~ N(0, 3); each row independently
             with probability 1/8 gets +8 on one uniformly chosen token; draft
             logits = target + N(0, 1); T = 0.7.
  block      B=64, G=15, V=129280, bf16 logits z = -1.1 ln(rank) over a fresh
             uniform permutation of ranks 1..V per row (Zipf(1.1) at T=1);
             draft logits = target + N(0, 0.75 * 1.05**k) at draft position k;
             T = 1.
  greedy     B=64, G=7, V=152064, bf16 logits ~ N(0, 4); T = 0; draft token k is
             the lowest-index argmax of bf16(z_k + N(0, 0.2)).
  scheduled  block logits at B in {4, 16, 64}; confidence c[b,k] =
             sigmoid(N(1.5, 1) - 0.08 k); cost[T] = 1 + 0.02 T for T = 0..512;
             token budget 512.
  block_logits
             block target logits; the drafter emits bf16 draft logits
             d = bf16(z + N(0, 0.75 * 1.05**k)) and samples x ~ softmax(d / T)
             (float64 from the stored bf16 values), so the draft distribution
             is exactly the softmax of the logits passed on.
  tree       a candidate tree per request (64 nodes: the root, 8 children, 4
             children on each of the first 4, 3 on each of the first 8 of
             those, 1 on each of the first 15 of those); bf16 node rows
             z ~ N(0, 4); a node's children are the top-k tokens of its parent
             row plus N(0, 0.2) noise (k = its number of children), so
             siblings are distinct and the best guess is often the argmax.
  calibration
             N samples of the scheduled confidences and an acceptance length per
             sample: draft k (given the earlier ones) is accepted when a uniform
             falls below c^(1/T*_k), for a known per-position temperature T*
             (the confidences are miscalibrated by T*, which a fit recovers).
  ratio_budgeted
             block logits and the scheduled confidences at B in {4, 16, 64};
             budget ratios (0.25, 0.5, 0.75, 1); the profiled cost of ratio rho
             is the affine stand-in 1 + 0.02 * rho * B * (G + 1) (the scheduled
             cost per target position, at the ratio's share of full depth).

Draft probabilities q = softmax(draft_logits / T) (float32) and
the draft tokens are sampled from q, as a sampling drafter does.  Uniforms are
float32 in [0, 1), laid out [B, G+1].
"""

import numpy as np

BASE_SEED = 1234
_STREAMS = {
    "target": 1,
    "draft_noise": 2,
    "draft_sample": 3,
    "verify_u": 4,
    "confidence": 5,
    "peaks": 6,
    "labels": 7,
}


def rng(seed, stream):
    """Independent Philox stream for (seed, stream name)."""
    return np.random.Generator(np.random.Philox(key=(int(seed) << 8) + _STREAMS[stream]))


def f32_to_bf16_bits(a):
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = ((bits[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


class Workload(dict):
    """Plain dict with attribute access: logits, dtype, draft_probs, draft_tokens, uniforms, ..."""

    __getattr__ = dict.__getitem__

    def logits_f32(self):
        if self["dtype"] == "bf16":
            return bf16_bits_to_f32(self["logits"])
        return self["logits"]


def _drafter(target_f32, G, T, noise_std, seed):
    """Sampling drafter: q = softmax((target + noise) / T) per position, x ~ q."""
    B, G1, V = target_f32.shape
    g_noise = rng(seed, "draft_noise")
    g_samp = rng(seed, "draft_sample")
    q = np.empty((B, G, V), dtype=np.float32)
    x = np.empty((B, G), dtype=np.int32)
    for k in range(G):
        sd = noise_std(k)
        d = target_f32[:, k, :] + np.float32(sd) * g_noise.standard_normal((B, V), dtype=np.float32)
        d = d / np.float32(T)
        d -= d.max(axis=1, keepdims=True)
        e = np.exp(d)
        q[:, k, :] = e / e.sum(axis=1, dtype=np.float64, keepdims=True).astype(np.float32)
        for b in range(B):
            w = q[b, k, :].astype(np.float64)
            x[b, k] = g_samp.choice(V, p=w / w.sum())
    return q, x


def _logit_drafter(target_f32, G, T, noise_std, seed):
    """Logits drafter: d = bf16(target + noise) per position, x ~ softmax(d / T)."""
    B, G1, V = target_f32.shape
    g_noise = rng(seed, "draft_noise")
    g_samp = rng(seed, "draft_sample")
    bits = np.empty((B, G, V), dtype=np.uint16)
    x = np.empty((B, G), dtype=np.int32)
    for k in range(G):
        sd = noise_std(k)
        d = target_f32[:, k, :] + np.float32(sd) * g_noise.standard_normal((B, V), dtype=np.float32)
        bits[:, k, :] = f32_to_bf16_bits(d)
        dd = bf16_bits_to_f32(bits[:, k, :]).astype(np.float64) / float(T)
        dd -= dd.max(axis=1, keepdims=True)
        e = np.exp(dd)
        for b in range(B):
            x[b, k] = g_samp.choice(V, p=e[b] / e[b].sum())
    return bits, x


def _uniforms(B, G, seed):
    return rng(seed, "verify_u").random((B, G + 1), dtype=np.float32)


def page_example():
    """The worked example: p=(0.5,0.3,0.2), q=(0.4,0.5,0.1), one draft (G=1), T=1.

    Target row 1 (the bonus row) is set to the same p.  Tokens/uniforms are
    filled in by the caller.
    """
    p = np.array([0.5, 0.3, 0.2])
    z = np.log(p).astype(np.float32)
    logits = np.stack([z, z])[None, :, :]                     # [1, 2, 3]
    q = np.array([[[0.4, 0.5, 0.1]]], dtype=np.float32)        # [1, 1, 3]
    return Workload(name="page_example", B=1, G=1, V=3, T=1.0, dtype="f32",
                    logits=logits, draft_probs=q,
                    draft_tokens=np.zeros((1, 1), np.int32),
                    uniforms=np.zeros((1, 2), np.float32), verify_len=None, seed=None)


def tiny(seed=BASE_SEED + 1, B=4, G=4, V=1024):
    z = (2.0 * rng(seed, "target").standard_normal((B, G + 1, V))).astype(np.float32)
    q, x = _drafter(z, G, 1.0, lambda k: 0.5, seed)
    return Workload(name="tiny", B=B, G=G, V=V, T=1.0, dtype="f32", logits=z,
                    draft_probs=q, draft_tokens=x, uniforms=_uniforms(B, G, seed),
                    verify_len=None, seed=seed)


def mtp(seed=BASE_SEED + 2, B=16, G=3, V=32000, T=0.7):
    g = rng(seed, "target")
    z = (3.0 * g.standard_normal((B, G + 1, V))).astype(np.float32)
    gp = rng(seed, "peaks")
    peaked = gp.random((B, G + 1)) < 1.0 / 8.0
    where = gp.integers(0, V, size=(B, G + 1))
    for b, k in zip(*np.nonzero(peaked)):
        z[b, k, where[b, k]] += 8.0
    bits = f32_to_bf16_bits(z)
    zf = bf16_bits_to_f32(bits)
    q, x = _drafter(zf, G, T, lambda k: 1.0, seed)
    return Workload(name="mtp", B=B, G=G, V=V, T=T, dtype="bf16", logits=bits,
                    draft_probs=q, draft_tokens=x, uniforms=_uniforms(B, G, seed),
                    verify_len=None, seed=seed)


def zipf_logits(seed, B, G1, V, exponent=1.1):
    """bf16 bits of z = -exponent * ln(rank), ranks a fresh permutation of 1..V per row."""
    table = f32_to_bf16_bits((-exponent * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32))
    perm = np.tile(np.arange(V, dtype=np.int32), (B * G1, 1))
    rng(seed, "target").permuted(perm, axis=1, out=perm)
    return table[perm].reshape(B, G1, V)


def block(seed=BASE_SEED + 3, B=64, G=15, V=129280, T=1.0):
    bits = zipf_logits(seed, B, G + 1, V)
    zf = bf16_bits_to_f32(bits)
    q, x = _drafter(zf, G, T, lambda k: 0.75 * 1.05 ** k, seed)
    return Workload(name="block", B=B, G=G, V=V, T=T, dtype="bf16", logits=bits,
                    draft_probs=q, draft_tokens=x, uniforms=_uniforms(B, G, seed),
                    verify_len=None, seed=seed)


def block_logits(seed=BASE_SEED + 7, B=64, G=15, V=129280, T=1.0):
    bits = zipf_logits(seed, B, G + 1, V)
    zf = bf16_bits_to_f32(bits)
    d, x = _logit_drafter(zf, G, T, lambda k: 0.75 * 1.05 ** k, seed)
    return Workload(name="block_logits", B=B, G=G, V=V, T=T, dtype="bf16", logits=bits,
                    draft_probs=None, draft_logits=d, draft_tokens=x, uniforms=_uniforms(B, G, seed),
                    verify_len=None, seed=seed)


def greedy(seed=BASE_SEED + 4, B=64, G=7, V=152064):
    z = (4.0 * rng(seed, "target").standard_normal((B, G + 1, V))).astype(np.float32)
    bits = f32_to_bf16_bits(z)
    zf = bf16_bits_to_f32(bits)
    gn = rng(seed, "draft_noise")
    x = np.empty((B, G), dtype=np.int32)
    for k in range(G):
        d = bf16_bits_to_f32(f32_to_bf16_bits(zf[:, k, :] + (0.2 * gn.standard_normal((B, V))).astype(np.float32)))
        x[:, k] = d.argmax(axis=1)
    return Workload(name="greedy", B=B, G=G, V=V, T=0.0, dtype="bf16", logits=bits,
                    draft_probs=None, draft_tokens=x, uniforms=None, verify_len=None, seed=seed)


def confidences(seed, B, G, mean=1.5, std=1.0, decay=0.08):
    g = mean + std * rng(seed, "confidence").standard_normal((B, G))
    c = 1.0 / (1.0 + np.exp(-(g - decay * np.arange(G)[None, :])))
    return c.astype(np.float32)


def linear_cost(a=1.0, b=0.02, table_len=513):
    return (a + b * np.arange(table_len, dtype=np.float64)).astype(np.float32)


def scheduled(B, seed=BASE_SEED + 5, G=15, V=129280, T=1.0, budget=512):
    w = block(seed=seed, B=B, G=G, V=V, T=T)
    w["name"] = "scheduled"
    w["confidence"] = confidences(seed, B, G)
    w["cost_table"] = linear_cost(table_len=budget + 1)
    w["budget"] = budget
    return w


RATIOS = (0.25, 0.5, 0.75, 1.0)


def ratio_costs(B, G, ratios=RATIOS, a=1.0, b=0.02):
    """Stand-in profiled step cost of each budget ratio at batch size B (float32)."""
    return [float(v) for v in (a + b * np.asarray(ratios, np.float64) * B * (G + 1)).astype(np.float32)]


def ratio_budgeted(B, seed=BASE_SEED + 6, G=15, V=129280, T=1.0):
    w = block(seed=seed, B=B, G=G, V=V, T=T)
    w["name"] = "ratio_budgeted"
    w["confidence"] = confidences(seed, B, G)
    w["ratios"] = RATIOS
    w["ratio_cost"] = ratio_costs(B, G)
    return w


def calibration(N, G=15, true_temps=None, seed=BASE_SEED + 8):
    """(conf [N, G] float32, acc_len [N] int32, true_temps [G]): synthetic STS fitting data."""
    if true_temps is None:
        true_temps = np.array([1.0, 0.6, 1.5, 0.8, 2.0, 1.2, 0.5, 1.0, 1.8, 0.7, 1.4, 0.9, 1.6, 1.1, 0.8])[:G]
    T = np.asarray(true_temps, np.float64)
    conf = confidences(seed, N, G)
    u = rng(seed, "labels").random((N, G))
    ok = u < np.exp2(np.log2(conf.astype(np.float64)) / T[None, :])
    acc_len = np.where(ok.all(axis=1), G, np.argmin(ok, axis=1)).astype(np.int32)
    return conf, acc_len, T


def tree_topology(levels=((0, 8), (4, 4), (8, 3), (15, 1))):
    """Parents of a layered candidate tree.  Each level (w, k): the first w nodes
    of the previous level (all of them when w == 0) get k children each."""
    parents = [-1]
    prev = [0]
    for w, k in levels:
        take = prev if w == 0 else prev[:w]
        cur = []
        for p in take:
            for _ in range(k):
                parents.append(p)
                cur.append(len(parents) - 1)
        prev = cur
    return np.asarray(parents, np.int64)


def tree(seed=BASE_SEED + 9, B=8, V=152064, parents=None, noise=0.2):
    par = tree_topology() if parents is None else np.asarray(parents, np.int64)
    M = len(par)
    z = (4.0 * rng(seed, "target").standard_normal((B, M, V))).astype(np.float32)
    bits = f32_to_bf16_bits(z)
    zf = bf16_bits_to_f32(bits)
    gn = rng(seed, "draft_noise")
    tok = np.zeros((B, M), np.int64)
    for p in range(M):
        kids = np.nonzero(par == p)[0]
        if len(kids) == 0:
            continue
        d = zf[:, p, :] + (noise * gn.standard_normal((B, V))).astype(np.float32)
        top = np.argsort(-d, axis=1, kind="stable")[:, : len(kids)]
        tok[:, kids] = top
    return Workload(name="tree", B=B, M=M, V=V, T=0.0, dtype="bf16", logits=bits,
                    parents=np.tile(par, (B, 1)).astype(np.int32), node_tokens=tok.astype(np.int32), seed=seed)
