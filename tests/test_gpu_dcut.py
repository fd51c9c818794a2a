"""GPU parity of ratio-budgeted depth (spec_dcut) and packed verification
(spec_verify_packed) against the float64 oracle, through the C ABI.

Bar: keep depths, row offsets and total rows exact; the estimated progress U
of each ratio within 1e-12 relative; the chosen ratio equal to the oracle's
unless the oracle's best and second-best U / C agree to 1e-12 relative (the
GPU sums U over requests in a tree order), and then the depths must be those
of the ratio the GPU chose.  Packed verification meets the verify bar
(parity_util) against the oracle's packed verification.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import dcut as OD
import workloads as W
import lossless_draft_verification_verify_amd as sv
from parity_util import compare, sub_fp32_run_confidences, to_device

pytestmark = pytest.mark.gpu

RATIOS = (0.25, 0.5, 0.75, 1.0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.load()
    yield


def run_dcut(conf, ratios, costs):
    c = torch.from_numpy(np.ascontiguousarray(conf, dtype=np.float32)).cuda()
    vl, off, r, K, U = sv.dcut(c, ratios, costs)
    torch.cuda.synchronize()
    return {"verify_len": vl.cpu().numpy().astype(np.int64), "row_offsets": off.cpu().numpy().astype(np.int64),
            "ratio_index": int(r.item()), "total_rows": int(K.item()), "utility": U.cpu().numpy()}


def check_dcut(conf, ratios, costs, tag=""):
    g = run_dcut(conf, ratios, costs)
    o = OD.dcut(conf.astype(np.float32), ratios, costs)
    R = len(ratios)
    rel = np.abs(g["utility"][:R] - o["utility"]) / np.maximum(1.0, np.abs(o["utility"]))
    assert rel.max() <= 1e-12, (tag, rel.max())
    theta = o["utility"] / np.asarray(costs, np.float32).astype(np.float64)
    r = g["ratio_index"]
    if r != o["ratio_index"]:
        best = theta[o["ratio_index"]]
        assert abs(theta[r] - best) <= 1e-12 * best, (tag, r, o["ratio_index"], theta)
        say(f"    near tie {tag}: gpu ratio {r}, oracle {o['ratio_index']}")
    n = o["lengths"][r]
    np.testing.assert_array_equal(g["verify_len"], n, err_msg=tag)
    np.testing.assert_array_equal(g["row_offsets"], OD.row_offsets(n), err_msg=tag)
    assert g["total_rows"] == int(o["budgets"][r]) == int((n + 1).sum()), tag
    return g, o


# ------------------------------------------------------------ spec_dcut

def test_dcut_hand_worked_case():
    g = run_dcut(np.array([[1.0, 0.5], [0.5, 0.5]], np.float32), RATIOS, [1.0, 1.2, 1.5, 2.0])
    assert g["verify_len"].tolist() == [2, 1] and g["row_offsets"].tolist() == [0, 3, 5]
    assert g["ratio_index"] == 2 and g["total_rows"] == 5
    np.testing.assert_array_equal(g["utility"], [2.0, 3.0, 4.0, 4.25])


def test_dcut_random_against_oracle():
    g0 = np.random.default_rng(21)
    for trial in range(40):
        B = int(g0.integers(1, 70))
        G = int(g0.integers(0, 17))
        conf = (1 / (1 + np.exp(-(g0.normal(1.5, 1.0, size=(B, G)) - 0.08 * np.arange(G))))).astype(np.float32)
        if trial % 5 == 1:
            conf[g0.random((B, G)) < 0.2] = 0.0
        if trial % 5 == 2:
            conf = (np.round(conf * 4) / 4).astype(np.float32)        # many exact ties
        if trial % 7 == 3:
            conf = (conf * 1.6 - 0.2).astype(np.float32)               # outside [0, 1]: clamped
            conf[g0.random((B, G)) < 0.05] = np.nan
        if trial % 3 == 0:
            ratios = list(RATIOS)
        else:
            R = int(g0.integers(1, 9))
            ratios = [float(np.float32(v)) for v in g0.uniform(0.01, 1.0, size=R)]
        K = np.array([OD.ratio_budget(r, B, G) for r in ratios])
        costs = [float(np.float32(v)) for v in 1.0 + g0.choice([0.0, 0.002, 0.02, 0.2]) * K]
        check_dcut(conf, ratios, costs, tag=f"trial {trial} B={B} G={G}")


@pytest.mark.parametrize("B,G", [(256, 16), (4096, 1), (1, 255), (3, 0), (4096, 0), (64, 15), (1024, 4),
                                 (100, 40)])
def test_dcut_large_and_shapes(B, G):
    say(f"[parity] dcut B={B} G={G}")
    g0 = np.random.default_rng(B * 7 + G)
    conf = (1 / (1 + np.exp(-g0.normal(2.0, 1.0, size=(B, G))))).astype(np.float32)
    K = np.array([OD.ratio_budget(r, B, G) for r in RATIOS])
    for slope in (0.0, 0.0005, 0.02, 5.0):
        check_dcut(conf, RATIOS, [float(v) for v in 1.0 + slope * K], tag=f"B={B} G={G} slope={slope}")


def test_dcut_extremes():
    B, G = 16, 15
    # every score 1: U / C with C proportional to K ties exactly -> the first ratio
    K = np.array([OD.ratio_budget(r, B, G) for r in RATIOS])
    g = run_dcut(np.ones((B, G), np.float32), RATIOS, [float(0.01 * k) for k in K])
    assert g["ratio_index"] == 0 and g["total_rows"] == K[0]
    # every confidence 0: U = B for every ratio; the budget is still filled
    g = run_dcut(np.zeros((B, G), np.float32), RATIOS, [2.0, 1.0, 1.0, 3.0])
    assert g["ratio_index"] == 1 and g["total_rows"] == K[1]
    np.testing.assert_array_equal(g["utility"], [B] * 4)
    # one ratio only
    conf = np.random.default_rng(3).uniform(0, 1, (B, G)).astype(np.float32)
    check_dcut(conf, [0.6], [1.0], tag="one ratio")


def test_dcut_repeated_calls_identical():
    conf = np.random.default_rng(5).uniform(0, 1, (64, 15)).astype(np.float32)
    costs = [1.0, 1.05, 1.1, 1.3]
    a = run_dcut(conf, RATIOS, costs)
    for _ in range(3):
        b = run_dcut(conf, RATIOS, costs)
        for k in a:
            np.testing.assert_array_equal(np.asarray(a[k]), np.asarray(b[k]))


# ------------------------------------------------------------ spec_verify_packed

def _rand(name, B, G, V, T=1.0, dtype="bf16", seed=0):
    g0 = np.random.default_rng(seed)
    z = (2.0 * g0.normal(size=(B, G + 1, V))).astype(np.float32)
    if dtype == "bf16":
        logits = W.f32_to_bf16_bits(z)
        zf = W.bf16_bits_to_f32(logits)
    else:
        logits = zf = z
    d = zf[:, :G].astype(np.float64) + 0.7 * g0.normal(size=(B, G, V))
    q = np.exp(d - d.max(2, keepdims=True))
    q = (q / q.sum(2, keepdims=True)).astype(np.float32)
    if T == 0.0:
        x = np.argmax(zf[:, :G] + 0.3 * g0.normal(size=(B, G, V)), axis=2).astype(np.int32)
    else:
        x = np.array([[g0.choice(V, p=q[b, k] / q[b, k].astype(np.float64).sum()) for k in range(G)]
                      for b in range(B)], np.int32).reshape(B, G)
    u = g0.random((B, G + 1), dtype=np.float32)
    conf = (1 / (1 + np.exp(-(g0.normal(1.5, 1.0, size=(B, G)) - 0.08 * np.arange(G))))).astype(np.float32)
    return W.Workload(name=name, B=B, G=G, V=V, T=T, dtype=dtype, logits=logits, draft_probs=q,
                      draft_tokens=x, uniforms=u, verify_len=None), conf


def pack_device(z, off, spare=0):
    """Gather the kept target rows of z [B, G+1, V] into [K + spare, V] (test-side packing)."""
    B, G1, V = z.shape
    idx = [b * G1 + k for b in range(B) for k in range(int(off[b + 1] - off[b]))]
    rows = z.reshape(B * G1, V)[torch.tensor(idx, dtype=torch.long, device=z.device)]
    if spare:
        rows = torch.cat([rows, torch.zeros(spare, V, dtype=z.dtype, device=z.device)])
    return rows.contiguous()


def run_packed(w, off_np, spare=0, diag=True, off_dev=None):
    z, q, x, u, _ = to_device(w)
    off = off_dev if off_dev is not None else torch.from_numpy(off_np.astype(np.int32)).cuda()
    zp = pack_device(z, off_np, spare)
    T = float(np.float32(w["T"]))
    if T == 0.0:
        acc, tok = sv.verify_packed(zp, off, None, x, None, 0.0)
        dg = None
    else:
        out = sv.verify_packed(zp, off, q, x, u, T, diag=diag)
        acc, tok, dg = out if diag else (*out, None)
    torch.cuda.synchronize()
    res = {"accepted": acc.cpu().numpy().astype(np.int64), "tokens": tok.cpu().numpy().astype(np.int64)}
    if dg is not None:
        res.update({k: v.cpu().numpy().astype(np.float64) for k, v in dg.items()})
        res["lse"] = res.pop("target_lse")
    return res


def packed_oracle(w, off_np, spare=0):
    zp = OD.pack_rows(w["logits"], off_np, rows=int(off_np[-1]) + spare)
    return OD.verify_packed(zp, off_np, w.get("draft_probs"), w["draft_tokens"], w.get("uniforms"),
                            np.float32(w["T"]))


@pytest.mark.parametrize("dtype,T,B,G,V", [
    ("bf16", 1.0, 24, 6, 5000), ("f32", 0.7, 24, 6, 4099), ("bf16", 0.0, 24, 6, 5000),
    ("bf16", 1.0, 300, 3, 2000), ("bf16", 0.0, 300, 3, 2000), ("f32", 1.0, 8, 15, 129281),
])
def test_verify_packed_matches_oracle(dtype, T, B, G, V):
    w, conf = _rand(f"packed_{dtype}_T{T}_B{B}", B, G, V, T=T, dtype=dtype, seed=B + G + V)
    say(f"[parity] {w['name']} G={G} V={V}")
    d = check_dcut(conf, RATIOS, [1.0, 1.1, 1.25, 1.5], tag=w["name"])[1]
    r = d["ratio_index"]
    n = d["lengths"][r]
    off = OD.row_offsets(n)
    spare = 3
    g = run_packed(w, off, spare=spare, diag=T > 0)
    o = packed_oracle(w, off, spare=spare)
    if T == 0.0:
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        np.testing.assert_array_equal(g["tokens"], o["tokens"])
        say("    bit-exact")
    else:
        w["verify_len"] = n
        say("   ", compare(w, g, o, n))


def test_verify_packed_bad_offsets():
    w, _ = _rand("packed_bad", 6, 3, 3000, seed=4)
    n = np.array([1, 3, 0, 2, 3, 1])
    off = OD.row_offsets(n)                          # [0, 2, 6, 7, 10, 14, 16]
    for bad_off, who in (([0, 2, 6, 7, 10, 14, 17], [5]),        # past the buffer
                         ([0, 2, 2, 7, 10, 14, 16], [1, 2]),     # empty request, then 5 rows > G+1
                         ([-1, 2, 6, 7, 10, 14, 16], [0])):      # negative start
        bo = np.array(bad_off)
        for T in (1.0, 0.0):
            w["T"] = T
            z, q, x, u, _ = to_device(w)
            zp = pack_device(z, off)                              # exactly off[B] = 16 rows
            dev_off = torch.from_numpy(bo.astype(np.int32)).cuda()
            if T == 0.0:
                acc, tok = sv.verify_packed(zp, dev_off, None, x, None, 0.0)
            else:
                acc, tok = sv.verify_packed(zp, dev_off, q, x, u, T)
            torch.cuda.synchronize()
            zpo = OD.pack_rows(w["logits"], off)
            o = OD.verify_packed(zpo, bo, w["draft_probs"], w["draft_tokens"], w["uniforms"], np.float32(T))
            acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
            for b in who:
                assert acc[b] == -1 and (tok[b] == -1).all(), (bad_off, T, b)
            np.testing.assert_array_equal(acc, o["accepted"])
            np.testing.assert_array_equal(tok, o["tokens"])


@pytest.mark.parametrize("B", [4, 16, 64])
def test_dcut_packed_end_to_end(B):
    """Ratio budget on the device, rows packed by its offsets, packed verify: the
    scheduled block workload (V = 129280, bf16, T = 1)."""
    w = W.scheduled(B)
    conf = w["confidence"]
    G = w["G"]
    K = np.array([OD.ratio_budget(r, B, G) for r in RATIOS])
    costs = [float(np.float32(v)) for v in 1.0 + 0.02 * K]
    say(f"[parity] dcut + packed verify B={B}")
    c = torch.from_numpy(conf).cuda()
    vl, off, r, Kd, U = sv.dcut(c, RATIOS, costs)
    torch.cuda.synchronize()
    d = OD.dcut(conf, RATIOS, costs)
    assert int(r.item()) == d["ratio_index"]
    np.testing.assert_array_equal(off.cpu().numpy(), d["row_offsets"])
    n = d["verify_len"]
    say(f"    ratio={RATIOS[d['ratio_index']]} K={d['total_rows']} lens={n.tolist()[:16]}")
    g = run_packed(w, d["row_offsets"], off_dev=off)
    o = packed_oracle(w, d["row_offsets"])
    w["verify_len"] = n
    say("   ", compare(w, g, o, n))


def test_packed_equals_unpacked_with_lengths():
    """The same requests through spec_verify (verify_len) and spec_verify_packed give identical outputs."""
    for T in (1.0, 0.0):
        w, conf = _rand(f"packed_vs_vlen_T{T}", 40, 7, 6000, T=T, seed=9)
        d = OD.dcut(conf, RATIOS, [1.0, 1.05, 1.1, 1.2])
        n = d["verify_len"]
        g = run_packed(w, d["row_offsets"], diag=False)
        z, q, x, u, _ = to_device(w)
        vl = torch.from_numpy(n.astype(np.int32)).cuda()
        if T == 0.0:
            acc, tok = sv.verify(z, None, x, None, 0.0, vl)
        else:
            acc, tok = sv.verify(z, q, x, u, T, vl)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g["accepted"], acc.cpu().numpy())
        np.testing.assert_array_equal(g["tokens"], tok.cpu().numpy())


def test_dcut_run_of_equal_fp32_survivals():
    """Ratio budgets whose cut falls inside a run of depth-2 survivals that
    differ only below fp32 precision (the exact order decides who is kept)."""
    conf = sub_fp32_run_confidences()
    B, G = conf.shape
    for rho in (0.70, 0.72, 0.75, 0.8, 0.9):
        keep = OD.ratio_budget(rho, B, G) - B
        assert B < keep < 2 * B, rho                 # inside the depth-2 run
        g, o = check_dcut(conf, [rho], [1.0], tag=f"rho {rho}")
        deep = sorted(np.flatnonzero(o["lengths"][0] == 2).tolist())
        assert deep != list(range(keep - B)), rho     # not the request-index order
