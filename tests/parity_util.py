"""Helpers for GPU-vs-oracle parity tests (imported by the gpu test modules).

Rules (the bar the GPU path must meet):
  * accepted lengths and emitted tokens equal the oracle's exactly, except for
    requests where one of the oracle's draws lies within 1e-6 of its decision
    threshold (min(1, p/q) for an accept test; C(y-1)/R or C(y)/R for the final
    draw, all in the oracle's float64); those are counted, and any mismatch
    among them is reported;
  * p(x_k), q(x_k) and the residual mass agree within 1e-5 absolute; the
    row log-sum-exp within 1e-5 relative;
  * temperature 0 is bit-exact with no allowance.
"""

import numpy as np
import torch

import oracle
import lossless_draft_verification_verify_amd as sv

BAND = 1e-6
PROB_ATOL = 1e-5


def to_device(w, device="cuda"):
    """Upload a workload's inputs; bf16 logits travel as their bit patterns."""
    if w["dtype"] == "bf16":
        z = torch.from_numpy(np.ascontiguousarray(w["logits"]).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        z = torch.from_numpy(np.ascontiguousarray(w["logits"], dtype=np.float32)).to(device)
    q = None if w.get("draft_probs") is None else torch.from_numpy(np.ascontiguousarray(w["draft_probs"])).to(device)
    x = torch.from_numpy(np.ascontiguousarray(w["draft_tokens"], dtype=np.int32)).to(device)
    u = None if w.get("uniforms") is None else torch.from_numpy(np.ascontiguousarray(w["uniforms"], dtype=np.float32)).to(device)
    vl = w.get("verify_len")
    vl = None if vl is None else torch.from_numpy(np.ascontiguousarray(vl, dtype=np.int32)).to(device)
    return z, q, x, u, vl


def run_gpu(w, diag=True, verify_len=None, with_event=False):
    """The HIP path on w.  with_event: pass a row-pass event (recorded between
    the row launch and the request launch)."""
    z, q, x, u, vl = to_device(w)
    if verify_len is not None:
        vl = verify_len
    T = np.float32(w["T"])
    ev = torch.cuda.Event() if with_event else None
    if float(T) == 0.0:
        acc, tok = sv.verify(z, None, x, None, 0.0, vl, row_pass_event=ev)
        dg = None
    elif diag:
        acc, tok, dg = sv.verify(z, q, x, u, float(T), vl, diag=True, row_pass_event=ev)
    else:
        acc, tok = sv.verify(z, q, x, u, float(T), vl, row_pass_event=ev)
        dg = None
    torch.cuda.synchronize()
    out = {"accepted": acc.cpu().numpy().astype(np.int64), "tokens": tok.cpu().numpy().astype(np.int64)}
    if dg is not None:
        out.update({k: v.cpu().numpy().astype(np.float64) for k, v in dg.items()})
        out["lse"] = out.pop("target_lse")
    return out


def run_oracle(w, verify_len=None):
    vl = w.get("verify_len") if verify_len is None else verify_len
    return oracle.verify(w["logits"], w.get("draft_probs"), w["draft_tokens"], w.get("uniforms"),
                         np.float32(w["T"]), vl)


def near_threshold(w, orc, verify_len=None):
    """Per request: does any draw the oracle made lie within BAND of its threshold?"""
    B, G = w["draft_tokens"].shape
    if float(w["T"]) == 0.0:
        return np.zeros(B, bool)
    u = np.asarray(w["uniforms"], np.float64)
    vl = w.get("verify_len") if verify_len is None else verify_len
    n = np.full(B, G) if vl is None else np.asarray(vl)
    flagged = np.zeros(B, bool)
    acc = orc["accepted"]
    T = np.float32(w["T"])
    for b in range(B):
        if acc[b] < 0:
            continue
        j = int(acc[b])
        for k in range(min(j + 1, int(n[b]))):          # tests actually made
            ratio = orc["p_draft"][b, k] / orc["q_draft"][b, k] if orc["q_draft"][b, k] > 0 else np.inf
            thr = min(1.0, ratio)
            if abs(u[b, k] - thr) <= BAND:
                flagged[b] = True
        # final draw
        zb = w["logits"][b]
        zf = oracle.bf16_bits_to_f64(zb) if w["dtype"] == "bf16" else np.asarray(zb, np.float64)
        row = j
        p, _ = oracle.target_probs(zf[row], T)
        if j < n[b]:
            r = oracle.residual(p, np.asarray(w["draft_probs"][b, j], np.float64))
            if not (np.cumsum(r)[-1] > 0):
                r = p
        else:
            r = p
        C = np.cumsum(r)
        R = C[-1]
        y = int(orc["tokens"][b, j])
        lo = C[y - 1] / R if y > 0 else 0.0
        hi = C[y] / R
        if abs(u[b, G] - lo) <= BAND or abs(u[b, G] - hi) <= BAND:
            flagged[b] = True
    return flagged


def compare(w, gpu, orc, verify_len=None, check_diag=True):
    """Assert parity; return a small report dict."""
    B = len(orc["accepted"])
    flagged = near_threshold(w, orc, verify_len)
    same = (gpu["accepted"] == orc["accepted"]) & np.all(gpu["tokens"] == orc["tokens"], axis=1)
    differ_flagged = int((~same & flagged).sum())
    bad = np.nonzero(~same & ~flagged)[0]
    assert bad.size == 0, (
        f"{w['name']}: {bad.size} unflagged mismatches, first b={bad[0]}: "
        f"gpu acc={gpu['accepted'][bad[0]]} tok={gpu['tokens'][bad[0]]} "
        f"oracle acc={orc['accepted'][bad[0]]} tok={orc['tokens'][bad[0]]}")
    rep = {"requests": B, "exact": int(same.sum()), "flagged": int(flagged.sum()),
           "flagged_and_differ": differ_flagged}
    if check_diag and float(w["T"]) > 0 and "p_draft" in gpu:
        ok = orc["accepted"] >= 0
        for key in ("p_draft", "q_draft"):
            g, o = gpu[key][ok], orc[key][ok]
            both = ~np.isnan(o)
            assert np.array_equal(np.isnan(g), np.isnan(o)), key
            err = np.max(np.abs(g[both] - o[both]), initial=0.0)
            assert err <= PROB_ATOL, (key, err)
            rep[key + "_maxerr"] = float(err)
        g, o = gpu["resid_mass"][ok], orc["resid_mass"][ok]
        # resid_mass: compare where the oracle rejected and the GPU took the same path
        sel = (o >= 0) & same[ok]
        err = np.max(np.abs(g[sel] - o[sel]), initial=0.0)
        assert err <= PROB_ATOL, ("resid_mass", err)
        assert np.all(g[(o < 0) & same[ok]] == -1.0)
        rep["resid_mass_maxerr"] = float(err)
        g, o = gpu["lse"][ok], orc["lse"][ok]
        both = ~np.isnan(o)
        assert np.array_equal(np.isnan(g), np.isnan(o)), "lse nan pattern"
        rel = np.max(np.abs(g[both] - o[both]) / np.maximum(1.0, np.abs(o[both])), initial=0.0)
        assert rel <= 1e-5, ("lse", rel)
        rep["lse_maxrel"] = float(rel)
    return rep


def sub_fp32_run_confidences(B=48, A=32):
    """Confidences whose depth-2 survivals s = c0 * c1 all round to one fp32
    value but differ (or tie exactly) in fp64, ordered against the request
    index.  c0 = 1 - a u, c1 = 1 - (2A - a) u with u = 2^-24 and a = b + 1, so
    s = 1 - 2A u + a (2A - a) u^2 exactly; the last term is far below half an
    fp32 ulp.  The exact order within the run is a (2A - a) descending, then
    b ascending on exact ties (a and 2A - a)."""
    u = 2.0 ** -24
    a = np.arange(1, B + 1, dtype=np.float64)
    conf = np.stack([1.0 - a * u, 1.0 - (2 * A - a) * u], axis=1).astype(np.float32)
    assert np.all(conf.astype(np.float64) == np.stack([1.0 - a * u, 1.0 - (2 * A - a) * u], axis=1))
    s1 = conf[:, 0].astype(np.float64) * conf[:, 1].astype(np.float64)
    assert len(set(s1.astype(np.float32).tolist())) == 1 and len(set(s1.tolist())) > B // 2
    return conf

