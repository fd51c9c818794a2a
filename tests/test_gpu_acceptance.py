"""GPU parity of the acceptance diagnostics (spec_acceptance) against the
float64 oracle, through the C ABI.

Bar: alpha within 1e-5 absolute of the oracle (1 - alpha is the residual mass
max(p - q, 0) summed, which the verify rule holds to 1e-5), NaN exactly where
the oracle has NaN.  Terms are fp32 against the rounded row reference, sums
fp64; the exponent of each term is rounded relative to its own size, so large
logits at a low temperature keep the bar.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import acceptance as A
import workloads as W
import lossless_draft_verification_verify_amd as sv

pytestmark = pytest.mark.gpu
ATOL = 1e-5


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


def run(z, dtype, draft, T, vlen=None, logits=False):
    zt = dev_logits(z, dtype)
    dt = dev_logits(draft, dtype) if logits else torch.from_numpy(np.ascontiguousarray(draft, np.float32)).cuda()
    vl = None if vlen is None else torch.from_numpy(np.asarray(vlen, np.int32)).cuda()
    out = sv.acceptance(zt, dt, T, vl, draft_is_logits=logits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(z, dtype, draft, T, vlen=None, logits=False, tag=""):
    g = run(z, dtype, draft, T, vlen, logits)
    o = A.acceptance(z, draft, np.float32(T), vlen, draft_is_logits=logits)
    assert np.array_equal(np.isnan(g), np.isnan(o)), (tag, np.argwhere(np.isnan(g) != np.isnan(o))[:4])
    err = np.max(np.abs(g - o)[~np.isnan(o)], initial=0.0)
    assert err <= ATOL, (tag, err)
    say(f"    {tag}: {int((~np.isnan(o)).sum())} positions, max |err| {err:.2e}")
    return g, o


def _rand(B, G, V, dtype, seed, T=1.0):
    g0 = np.random.default_rng(seed)
    z = (2.0 * g0.normal(size=(B, G + 1, V))).astype(np.float32)
    d = (z[:, :G] + 0.8 * g0.normal(size=(B, G, V))).astype(np.float32)
    if dtype == "bf16":
        zb, db = W.f32_to_bf16_bits(z), W.f32_to_bf16_bits(d)
        df = W.bf16_bits_to_f32(db).astype(np.float64)
    else:
        zb, db, df = z, d, d.astype(np.float64)
    q = np.exp((df - df.max(2, keepdims=True)) / T)
    q = (q / q.sum(2, keepdims=True)).astype(np.float32)
    return zb, db, q


def test_page_example():
    w = W.page_example()
    g, _ = check(w["logits"], "f32", w["draft_probs"], 1.0, tag="page example")
    assert abs(g[0, 0] - 0.8) < 1e-6


@pytest.mark.parametrize("dtype,V", [("bf16", 5000), ("f32", 4099), ("bf16", 1023), ("f32", 7), ("bf16", 129281)])
@pytest.mark.parametrize("logits", [False, True])
def test_random_against_oracle(dtype, V, logits):
    B, G = 6, 4
    z, d, q = _rand(B, G, V, dtype, seed=V + logits)
    vlen = np.array([4, 2, 0, 3, 4, 1])
    say(f"[parity] acceptance {dtype} V={V} logits={logits}")
    check(z, dtype, d if logits else q, 1.0, vlen, logits, tag=f"{dtype} V={V}")
    check(z, dtype, d if logits else q, 0.6, None, logits, tag=f"{dtype} V={V} T=0.6")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("logits", [False, True])
def test_large_logits_low_temperature(dtype, logits):
    """Logits near 30 at T = 0.1 (m / T about 300, so fl(m log2(e) / T) is far
    from its neighbours' scale): the exponent of each term must be rounded
    relative to the term, not to the reference."""
    B, G, V = 4, 3, 20000
    g0 = np.random.default_rng(41 + logits)
    z = (30.0 + 0.3 * g0.normal(size=(B, G + 1, V))).astype(np.float32)
    d = (z[:, :G] + 0.1 * g0.normal(size=(B, G, V))).astype(np.float32)
    T = 0.1
    if dtype == "bf16":
        zb, db = W.f32_to_bf16_bits(z), W.f32_to_bf16_bits(d)
        df = W.bf16_bits_to_f32(db).astype(np.float64)
    else:
        zb, db, df = z, d, d.astype(np.float64)
    q = np.exp((df - df.max(2, keepdims=True)) / T)
    q = (q / q.sum(2, keepdims=True)).astype(np.float32)
    say(f"[parity] acceptance large logits T=0.1 {dtype} logits={logits}")
    check(zb, dtype, db if logits else q, T, None, logits, tag=f"shift 30 T=0.1 {dtype}")


def test_bad_rows_and_lengths():
    B, G, V = 5, 3, 3000
    z, d, q = _rand(B, G, V, "f32", seed=3)
    z[0, 1, 17] = np.nan                           # position (0, 1) only
    d[1, 0, :] = -np.inf                           # logits mode: position (1, 0)
    z[2, 2, 5] = np.inf                            # max +inf: position (2, 2)
    z[3, 3, :] = np.nan                            # the bonus row: no position uses it
    vlen = np.array([3, 3, 3, 3, 7])               # request 4: invalid length
    for logits in (False, True):
        g, o = check(z, "f32", d if logits else q, 1.0, vlen, logits, tag=f"bad rows logits={logits}")
        assert np.isnan(g[0, 1]) and np.isnan(g[2, 2]) and np.isnan(g[4]).all()
        assert not np.isnan(g[3]).any()
        assert np.isnan(g[1, 0]) == logits


def test_identical_rows_accept_all():
    B, G, V = 3, 2, 4000
    z, _, _ = _rand(B, G, V, "f32", seed=4)
    g = run(z, "f32", z[:, :G].copy(), 1.0, logits=True)
    assert np.all(np.abs(g - 1.0) <= ATOL)


def test_block_full_size():
    """The block workload (B=64, gamma=15, V=129280): oracle on 8 sampled requests."""
    w = W.block()
    say("[parity] acceptance block full size")
    g = run(w["logits"], "bf16", w["draft_probs"], 1.0)
    sel = np.array([0, 7, 13, 22, 31, 40, 51, 63])
    o = A.acceptance(w["logits"][sel], w["draft_probs"][sel], 1.0)
    err = np.max(np.abs(g[sel] - o))
    assert not np.isnan(g).any() and err <= ATOL, err
    say(f"    mean alpha by position: {np.round(g.mean(0), 3).tolist()}  max |err| {err:.2e}")


def test_block_logits_full_size():
    w = W.block_logits(B=16)
    say("[parity] acceptance block logits B=16")
    g = run(w["logits"], "bf16", w["draft_logits"], 1.0, logits=True)
    sel = np.array([0, 5, 10, 15])
    o = A.acceptance(w["logits"][sel], w["draft_logits"][sel], 1.0, draft_is_logits=True)
    err = np.max(np.abs(g[sel] - o))
    assert not np.isnan(g).any() and err <= ATOL, err
