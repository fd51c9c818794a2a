"""spec_verify_noalloc (static device scratch, no allocation) against
spec_verify (caller's workspace), through the C ABI.

Both run the same kernels, so the outputs (and the diagnostics) must agree bit
for bit.  Two calls in a row on the shared scratch, the second with a smaller
input (the scratch then holds the first call's words beyond the second's
layout), at T > 0 and at T = 0, with and without verify lengths; a shape beyond
the scratch is refused before anything is enqueued.
"""

import sys

import numpy as np
import pytest
import torch

import workloads as W
import lossless_draft_verification_verify_amd as sv
from lossless_draft_verification_verify_amd import _capi

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


def upload(w):
    if w["dtype"] == "bf16":
        z = torch.from_numpy(np.ascontiguousarray(w["logits"]).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        z = torch.from_numpy(np.ascontiguousarray(w["logits"], np.float32)).cuda()
    q = None if w.get("draft_probs") is None else torch.from_numpy(w["draft_probs"]).cuda()
    x = torch.from_numpy(np.ascontiguousarray(w["draft_tokens"], np.int32)).cuda()
    u = None if w.get("uniforms") is None else torch.from_numpy(w["uniforms"]).cuda()
    return z, q, x, u


def noalloc(z, q, x, u, T, vl=None, diag=False):
    """The no-allocation entry point through the C ABI."""
    B, G1, V = z.shape
    G = G1 - 1
    code = _capi.SPEC_DTYPE_BF16 if z.dtype == torch.bfloat16 else _capi.SPEC_DTYPE_F32
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, G1), -7, dtype=torch.int32, device="cuda")
    dg, d = None, None
    if diag:
        dg = {"target_lse": torch.empty(B, G1, device="cuda"), "p_draft": torch.empty(B, G, device="cuda"),
              "q_draft": torch.empty(B, G, device="cuda"), "resid_mass": torch.empty(B, device="cuda")}
        d = _capi.DiagT(*(dg[k].data_ptr() for k in ("target_lse", "p_draft", "q_draft", "resid_mass")), 0)
    ptr = (lambda t: 0 if t is None else t.data_ptr())
    st = _capi.spec_verify_noalloc(z.data_ptr(), code, ptr(q), ptr(x), ptr(u), ptr(vl), B, G, V, float(T),
                                   acc.data_ptr(), tok.data_ptr(), d, torch.cuda.current_stream().cuda_stream)
    return st, acc, tok, dg


def check_pair(w, vl=None, diag=True):
    z, q, x, u = upload(w)
    T = float(w["T"])
    vld = None if vl is None else torch.from_numpy(np.asarray(vl, np.int32)).cuda()
    st, acc, tok, dg = noalloc(z, q, x, u, T, vld, diag=diag and T > 0)
    assert st == 0, _capi.status_string(st)
    if diag and T > 0:
        acc0, tok0, dg0 = sv.verify(z, q, x, u, T, vld, diag=True)
    else:
        acc0, tok0 = sv.verify(z, q, x, u, T, vld)
        dg0 = None
    torch.cuda.synchronize()
    assert torch.equal(acc, acc0), (acc.cpu(), acc0.cpu())
    assert torch.equal(tok, tok0)
    assert int((acc < 0).sum()) == 0
    if dg0 is not None:
        for k in dg0:
            a, b = dg[k].cpu().numpy(), dg0[k].cpu().numpy()
            assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)]), k
    return acc


@pytest.mark.parametrize("greedy", [False, True])
def test_noalloc_matches_verify_twice_then_smaller(greedy):
    big = W.greedy(B=24, G=7, V=60000, seed=501) if greedy else W.block(B=24, G=15, V=60000, seed=501)
    small = W.greedy(B=5, G=3, V=3001, seed=502) if greedy else W.block(B=5, G=3, V=3001, seed=502)
    say(f"[no-alloc] greedy={greedy}: B={big['B']} G={big['G']} V={big['V']}, then the same, then "
        f"B={small['B']} G={small['G']} V={small['V']}")
    a1 = check_pair(big)
    a2 = check_pair(big)
    assert torch.equal(a1, a2)
    check_pair(small)


def test_noalloc_verify_lengths_and_headline_shape():
    w = W.block(B=64, G=15, V=129280, seed=503)
    vl = np.random.default_rng(503).integers(0, 16, size=64)
    say("[no-alloc] B=64 G=15 V=129280 with verify lengths, then full lengths, then B=3 V=999")
    check_pair(w, vl)
    check_pair(w)
    check_pair(W.block(B=3, G=2, V=999, seed=504), diag=True)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    B, G, V = 1000, 15, 129280
    need = _capi.verify_workspace_bytes(B, G, V, _capi.SPEC_DTYPE_BF16)
    assert need > _capi.NOALLOC_SCRATCH_BYTES
    z = torch.empty(1, 1, 1, dtype=torch.bfloat16, device="cuda")   # never read: refused on the host
    st = _capi.spec_verify_noalloc(z.data_ptr(), _capi.SPEC_DTYPE_BF16, z.data_ptr(), z.data_ptr(), z.data_ptr(),
                                   0, B, G, V, 1.0, z.data_ptr(), z.data_ptr(), None,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 9, st
    assert "static scratch" in _capi.status_string(st)
