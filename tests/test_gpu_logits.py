"""GPU parity of verification with draft logits (spec_verify_logits) against
the float64 oracle, through the C ABI.

The oracle forms q = softmax(d / T) in float64 from the same stored logits;
the bar is the verify bar (parity_util): tokens and lengths exact except for
draws within 1e-6 of a threshold, p(x), q(x) and R within 1e-5.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import acceptance as A
import workloads as W
import lossless_draft_verification_verify_amd as sv
from parity_util import compare

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.load()
    yield


def dev_logits(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def run_logits(w, diag=True, verify_len=None):
    z = dev_logits(w["logits"], w["dtype"])
    d = dev_logits(w["draft_logits"], w["dtype"])
    x = torch.from_numpy(np.ascontiguousarray(w["draft_tokens"], np.int32)).cuda()
    u = torch.from_numpy(np.ascontiguousarray(w["uniforms"], np.float32)).cuda()
    vl = verify_len if verify_len is not None else w.get("verify_len")
    vl = None if vl is None else torch.from_numpy(np.asarray(vl, np.int32)).cuda()
    T = float(np.float32(w["T"]))
    if T == 0.0:
        acc, tok = sv.verify(z, None, x, None, 0.0, vl, draft_logits=d)
        dg = None
    elif diag:
        acc, tok, dg = sv.verify(z, None, x, u, T, vl, diag=True, draft_logits=d)
    else:
        acc, tok = sv.verify(z, None, x, u, T, vl, draft_logits=d)
        dg = None
    torch.cuda.synchronize()
    out = {"accepted": acc.cpu().numpy().astype(np.int64), "tokens": tok.cpu().numpy().astype(np.int64)}
    if dg is not None:
        out.update({k: v.cpu().numpy().astype(np.float64) for k, v in dg.items()})
        out["lse"] = out.pop("target_lse")
    return out


def check(w, diag=True):
    say(f"[parity] {w['name']} B={w['B']} G={w['G']} V={w['V']} T={w['T']} dtype={w['dtype']}")
    g = run_logits(w, diag)
    o = A.verify_logits(w["logits"], w["draft_logits"], w["draft_tokens"], w["uniforms"], np.float32(w["T"]),
                        w.get("verify_len"))
    if float(w["T"]) == 0.0:
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        np.testing.assert_array_equal(g["tokens"], o["tokens"])
        say("    bit-exact")
        return g, o
    # the oracle's draft distribution, for the near-threshold bands
    w = W.Workload(w)
    w["draft_probs"] = A.draft_probs_from_logits(w["draft_logits"], np.float32(w["T"]))
    rep = compare(w, g, o, w.get("verify_len"), check_diag=diag)
    say("   ", rep)
    return g, o


def _rand(name, B, G, V, T=1.0, dtype="bf16", seed=0, noise=0.8):
    g0 = np.random.default_rng(seed)
    z = (2.0 * g0.normal(size=(B, G + 1, V))).astype(np.float32)
    d = (z[:, :G] + noise * g0.normal(size=(B, G, V))).astype(np.float32)
    if dtype == "bf16":
        zb, db = W.f32_to_bf16_bits(z), W.f32_to_bf16_bits(d)
        df = W.bf16_bits_to_f32(db).astype(np.float64)
    else:
        zb, db, df = z, d, d.astype(np.float64)
    q = np.exp((df - df.max(2, keepdims=True)) / T)
    q = q / q.sum(2, keepdims=True)
    x = np.array([[g0.choice(V, p=q[b, k]) for k in range(G)] for b in range(B)], np.int32).reshape(B, G)
    u = g0.random((B, G + 1), dtype=np.float32)
    return W.Workload(name=name, B=B, G=G, V=V, T=T, dtype=dtype, logits=zb, draft_logits=db, draft_probs=None,
                      draft_tokens=x, uniforms=u, verify_len=None)


@pytest.mark.parametrize("dtype,V,T", [("bf16", 5000, 1.0), ("f32", 4099, 0.7), ("bf16", 1023, 1.0),
                                       ("f32", 7, 1.0), ("bf16", 129281, 1.0), ("bf16", 32000, 0.7)])
def test_random_against_oracle(dtype, V, T):
    w = _rand(f"logits_{dtype}_V{V}", 12, 5, V, T=T, dtype=dtype, seed=V)
    check(w)
    w["verify_len"] = np.random.default_rng(V).integers(0, 6, size=12).astype(np.int32)
    check(w)


def test_greedy_ignores_draft_logits():
    w = _rand("logits_greedy", 16, 4, 3000, seed=5)
    w["T"] = 0.0
    check(w)


def test_bad_draft_rows_are_data_errors():
    w = _rand("logits_bad", 6, 3, 3000, seed=6)
    d = w["draft_logits"].copy()
    d[0, 1, 9] = 0x7FC0                       # bf16 NaN in a verified draft row
    d[2, 0, :] = 0xFF80                       # an all -inf draft row
    d[3, 2, 4] = 0x7F80                       # +inf: maximum +inf
    d[4, 2, :] = 0xFF80                       # row 2 of request 4, not verified at n = 2
    w["draft_logits"] = d
    w["verify_len"] = np.array([3, 3, 3, 3, 2, 3], np.int32)
    g, o = check(w)
    assert g["accepted"][[0, 2, 3]].tolist() == [-1, -1, -1] and g["accepted"][4] >= 0


def test_many_requests_and_ragged():
    w = _rand("logits_many", 300, 3, 2000, seed=7)       # B > 256: the full-grid row kernel
    check(w, diag=False)


def test_block_logits_full_size():
    """bf16 target and draft logits, B=64, gamma=15, V=129280, T=1 (the draft-logits workload)."""
    check(W.block_logits())
