"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Same seeded inputs on both sides (workloads.py).  Sizes are small enough for
the oracle to finish in seconds while spanning several row chunks, several
final-draw tiles and ragged tails; the full-size workloads run too.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import lossless_draft_verification_verify_amd as sv
from parity_util import compare, run_gpu, run_oracle, sub_fp32_run_confidences, to_device

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


def check(w, verify_len=None, diag=True):
    say(f"[parity] {w['name']} B={w['B']} G={w['G']} V={w['V']} T={w['T']} dtype={w['dtype']}")
    g = run_gpu(w, diag=diag)
    o = run_oracle(w, verify_len)
    rep = compare(w, g, o, verify_len, check_diag=diag)
    say("   ", rep)
    return g, o, rep


# ------------------------------------------------------------ page example

def test_page_example_grid():
    """Worked example p=(0.5,0.3,0.2), q=(0.4,0.5,0.1): every x, a grid of (u0, u1)."""
    base = W.page_example()
    M0, M1 = 50, 20
    u0 = (np.arange(M0) + 0.5) / M0
    u1 = (np.arange(M1) + 0.5) / M1
    xs, us = [], []
    for x in range(3):
        for a in u0:
            for b in u1:
                xs.append([x])
                us.append([a, b])
    N = len(xs)
    w = W.Workload(base)
    w.update(B=N, logits=np.repeat(base["logits"], N, 0), draft_probs=np.repeat(base["draft_probs"], N, 0),
             draft_tokens=np.array(xs, np.int32), uniforms=np.array(us, np.float32))
    g, o, rep = check(w)
    # acceptance mass and first-token law of the page: 0.8 and (0.5, 0.3, 0.2)
    q = base["draft_probs"][0, 0].astype(np.float64)
    acc = g["accepted"].reshape(3, -1)
    first = g["tokens"][:, 0].reshape(3, -1)
    mass = sum(q[x] * np.mean(acc[x] == 1) for x in range(3))
    law = sum(q[x] * np.bincount(first[x], minlength=3) / first.shape[1] for x in range(3))
    assert abs(mass - 0.8) < 1e-6
    np.testing.assert_allclose(law, [0.5, 0.3, 0.2], atol=1e-6)


# ------------------------------------------------------------ configs

def test_tiny_fp32():
    for seed in range(6):
        check(W.tiny(seed=1235 + seed))


def test_mtp_bf16():
    check(W.mtp())


def test_block_reduced_ragged():
    # V not a multiple of the row chunk (16384) or the draw tile (8192)
    check(W.block(B=8, G=15, V=20000))
    check(W.block(B=5, G=6, V=40961, seed=77))


def test_block_full_size():
    g, o, rep = check(W.block())
    assert rep["requests"] == 64


def test_greedy_full_size_bit_exact():
    w = W.greedy()
    say("[parity] greedy full")
    g = run_gpu(w)
    o = run_oracle(w)
    np.testing.assert_array_equal(g["accepted"], o["accepted"])
    np.testing.assert_array_equal(g["tokens"], o["tokens"])
    say("    accepted mean", g["accepted"].mean())


def test_greedy_ties_and_sizes():
    g0 = np.random.default_rng(3)
    for (B, G, V) in [(16, 7, 1024), (9, 3, 1023), (4, 5, 16385), (3, 2, 50001)]:
        z = np.round(g0.normal(0, 1, size=(B, G + 1, V)) * 2) / 2          # many exact ties
        bits = W.f32_to_bf16_bits(z.astype(np.float32))
        zf = W.bf16_bits_to_f32(bits).astype(np.float64)
        a = zf.argmax(2)
        x = np.where(g0.random((B, G)) < 0.8, a[:, :G], g0.integers(0, V, (B, G))).astype(np.int32)
        w = W.Workload(name=f"greedy_ties_{V}", B=B, G=G, V=V, T=0.0, dtype="bf16", logits=bits,
                       draft_probs=None, draft_tokens=x, uniforms=None, verify_len=None)
        say(f"[parity] {w['name']}")
        g = run_gpu(w)
        o = run_oracle(w)
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        np.testing.assert_array_equal(g["tokens"], o["tokens"])
        # fp32 logits, same ties
        w2 = W.Workload(w)
        w2.update(dtype="f32", logits=zf.astype(np.float32), name=f"greedy_ties_f32_{V}")
        g = run_gpu(w2)
        o = run_oracle(w2)
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        np.testing.assert_array_equal(g["tokens"], o["tokens"])


# ------------------------------------------------------------ scheduling

@pytest.mark.parametrize("B", [4, 16, 64])
def test_scheduled_end_to_end(B):
    w = W.scheduled(B)
    say(f"[parity] scheduled B={B}")
    c = torch.from_numpy(w["confidence"]).cuda()
    cost = torch.from_numpy(w["cost_table"]).cuda()
    vl, T, tau = sv.schedule(c, cost, w["budget"])
    torch.cuda.synchronize()
    lens_o, T_o, tau_o = oracle.schedule(w["confidence"], w["cost_table"], w["budget"])
    np.testing.assert_array_equal(vl.cpu().numpy(), lens_o)
    assert int(T.item()) == T_o
    assert abs(float(tau.item()) - tau_o) <= 1e-6 * tau_o
    say(f"    T={T_o} tau={tau_o:.4f} lens={lens_o.tolist()[:16]}")
    # verify with the device-resident lengths
    w["verify_len"] = lens_o
    g = run_gpu(w, verify_len=vl)
    o = run_oracle(w, lens_o)
    say("   ", compare(w, g, o, lens_o))


def test_schedule_random_against_oracle():
    g0 = np.random.default_rng(11)
    for trial in range(30):
        B = int(g0.integers(1, 70))
        G = int(g0.integers(0, 17))
        conf = (1 / (1 + np.exp(-g0.normal(1.0, 1.5, size=(B, G))))).astype(np.float32)
        if trial % 5 == 1:
            conf[g0.random((B, G)) < 0.2] = 0.0
        if trial % 5 == 2:
            conf = np.round(conf * 4) / 4                      # many exact ties
        if trial % 7 == 3:
            conf = (conf * 1.6).astype(np.float32)             # > 1: non-contiguous skips
        L = int(B * (G + 1) + int(g0.integers(1, 40)))
        a, b = 1.0, float(g0.choice([0.0, 0.001, 0.02, 0.2]))
        cost = (a + b * np.arange(L)).astype(np.float32)
        if trial % 4 == 3:
            cost = (a + b * np.arange(L) + 0.3 * np.sqrt(np.arange(L))).astype(np.float32)
        budget = int(g0.integers(B, L))
        eps = float(g0.choice([0.0, 0.01]))
        vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget, eps)
        torch.cuda.synchronize()
        lo, To, tauo = oracle.schedule(conf, cost, budget, eps)
        np.testing.assert_array_equal(vl.cpu().numpy(), lo, err_msg=f"trial {trial}")
        assert int(T.item()) == To, trial
        assert abs(float(tau.item()) - np.float32(tauo)) <= 1e-6 * max(1.0, tauo), trial


@pytest.mark.parametrize("B,G,slope,extra", [
    (256, 16, 0.0, 130),       # 4096 candidates; theta always improves: the budget stops the walk
    (64, 15, 0.001, 400),      # the walk crosses several 64-candidate blocks before theta stops it
    (4096, 1, 0.0005, 3000),   # one draft per request, 4096 requests
    (1, 255, 0.002, 255),      # one request, the deepest block
    (3, 0, 0.02, 2),           # no drafts at all
    (64, 15, 5.0, 50),         # steep cost: nothing is worth verifying
])
def test_schedule_large_and_block_boundaries(B, G, slope, extra):
    g0 = np.random.default_rng(B * 1000 + G)
    conf = (1 / (1 + np.exp(-g0.normal(2.0, 1.0, size=(B, G))))).astype(np.float32)
    budget = min(B + extra, B * (G + 1))
    cost = (1.0 + slope * np.arange(budget + 2)).astype(np.float32)
    vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget)
    torch.cuda.synchronize()
    lo, To, tauo = oracle.schedule(conf, cost, budget)
    np.testing.assert_array_equal(vl.cpu().numpy(), lo)
    assert int(T.item()) == To
    assert abs(float(tau.item()) - np.float32(tauo)) <= 1e-6 * max(1.0, tauo)


def test_schedule_selective_prefix_against_oracle():
    """Schedules whose walk stops before, at and after the first 256 candidates
    of the order (the kernel sorts only a prefix of the order that a histogram
    of survivals picks, and sorts everything when the walk runs past it), with
    exact ties, zero confidences, a negative eps and many requests."""
    g0 = np.random.default_rng(23)
    for trial in range(40):
        B = int(g0.choice([17, 40, 64, 100, 256, 512, 1024]))
        G = int(g0.integers(1, 17))
        while B * G > 4096:
            G -= 1
        conf = (1 / (1 + np.exp(-g0.normal(1.5, 1.2, size=(B, G))))).astype(np.float32)
        if trial % 4 == 1:
            conf = (np.round(conf * 8) / 8).astype(np.float32)        # large runs of equal survival
        if trial % 6 == 2:
            conf[g0.random((B, G)) < 0.3] = 0.0
        L = B * (G + 1) + 2
        slope = float(g0.choice([0.0, 0.0005, 0.002, 0.01, 0.05]))
        cost = (1.0 + slope * np.arange(L)).astype(np.float32)
        budget = int(g0.integers(B, L))
        eps = float(g0.choice([-0.5, 0.0, 0.01]))
        lo, To, tauo = oracle.schedule(conf, cost, budget, eps)
        say(f"[parity] schedule selective trial {trial}: B={B} G={G} slope={slope} budget={budget} eps={eps} "
            f"kept={To - B}")
        vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget, eps)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(vl.cpu().numpy(), lo, err_msg=f"trial {trial}")
        assert int(T.item()) == To, trial
        assert abs(float(tau.item()) - np.float32(tauo)) <= 1e-6 * max(1.0, tauo), trial


def test_schedule_one_survival_bin_holds_every_candidate():
    """512 requests with equal confidence: every candidate falls in one
    survival bin, more than the selective sort takes, so every one is sorted."""
    B, G = 512, 1
    conf = np.full((B, G), 0.75, np.float32)
    cost = np.ones(B * 2 + 1, np.float32)
    for budget in (B, B + 1, B + 300, 2 * B):
        lo, To, tauo = oracle.schedule(conf, cost, budget)
        say(f"[parity] schedule, one bin, budget {budget}")
        vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(vl.cpu().numpy(), lo, err_msg=f"budget {budget}")
        assert int(T.item()) == To == budget
        assert float(tau.item()) == np.float32(tauo), budget


# ------------------------------------------------------------ edge cases

def _rand_workload(name, B, G, V, T=1.0, dtype="bf16", seed=0, zscale=2.0):
    g0 = np.random.default_rng(seed)
    z = (zscale * g0.normal(size=(B, G + 1, V))).astype(np.float32)
    if dtype == "bf16":
        bits = W.f32_to_bf16_bits(z)
        zf = W.bf16_bits_to_f32(bits)
        logits = bits
    else:
        zf = z
        logits = z
    d = zf[:, :G].astype(np.float64) + 0.7 * g0.normal(size=(B, G, V))
    q = np.exp((d - d.max(2, keepdims=True)) / T)
    q = (q / q.sum(2, keepdims=True)).astype(np.float32)
    x = np.array([[g0.choice(V, p=q[b, k] / q[b, k].astype(np.float64).sum()) for k in range(G)]
                  for b in range(B)], np.int32).reshape(B, G)
    u = g0.random((B, G + 1), dtype=np.float32)
    return W.Workload(name=name, B=B, G=G, V=V, T=T, dtype=dtype, logits=logits, draft_probs=q,
                      draft_tokens=x, uniforms=u, verify_len=None)


def test_gamma_zero_plain_sampling():
    w = _rand_workload("gamma0", 50, 0, 3000, seed=1)
    check(w)


def test_verify_len_mixed():
    w = _rand_workload("vlen", 40, 6, 5000, seed=2)
    w["verify_len"] = np.random.default_rng(2).integers(0, 7, size=40).astype(np.int32)
    check(w)


def test_unaligned_vocab_sizes():
    for V, dt in [(1023, "bf16"), (1023, "f32"), (129281, "bf16"), (8193, "f32"), (7, "bf16")]:
        check(_rand_workload(f"V{V}_{dt}", 6, 4, V, dtype=dt, seed=V))


def test_maximum_drafts():
    # G = 255, the most draft positions a request may carry.
    check(_rand_workload("G255_bf16", 2, 255, 700, seed=31))
    check(_rand_workload("G255_f32", 2, 255, 300, dtype="f32", seed=32))


def test_large_vocabulary():
    # V = 2^22 + 7: 2049 chunks per row give 513 partials per row (past the
    # merge that holds a row's partials in registers) and 2049 draw sub-tiles
    # (past the one-block mass scan and selection).
    check(_rand_workload("V4M", 2, 2, (1 << 22) + 7, seed=33, zscale=3.0))


def test_large_vocabulary_greedy():
    # V = 2^22 + 3 at T = 0: 2049 chunk partials per row, past the greedy
    # merge's one-batch path.
    g0 = np.random.default_rng(34)
    B, G, V = 3, 2, (1 << 22) + 3
    bits = W.f32_to_bf16_bits((2.0 * g0.normal(size=(B, G + 1, V))).astype(np.float32))
    a = W.bf16_bits_to_f32(bits).argmax(2)
    x = np.where(g0.random((B, G)) < 0.7, a[:, :G], g0.integers(0, V, (B, G))).astype(np.int32)
    w = W.Workload(name="greedy_V4M", B=B, G=G, V=V, T=0.0, dtype="bf16", logits=bits,
                   draft_probs=None, draft_tokens=x, uniforms=None, verify_len=None)
    say(f"[parity] {w['name']}")
    g = run_gpu(w)
    o = run_oracle(w)
    np.testing.assert_array_equal(g["accepted"], o["accepted"])
    np.testing.assert_array_equal(g["tokens"], o["tokens"])


def test_maximum_batch():
    # B = 65536 requests (the batch limit), a tiny vocabulary.
    check(_rand_workload("B65536", 65536, 1, 16, seed=35))


def test_q_equal_p_accepts_all():
    B, G, V = 12, 5, 4096
    z = np.zeros((B, G + 1, V), np.float32)                  # uniform rows: p = 1/V exactly
    q = np.full((B, G, V), 1.0 / V, np.float32)
    g0 = np.random.default_rng(4)
    w = W.Workload(name="q_eq_p", B=B, G=G, V=V, T=1.0, dtype="f32", logits=z, draft_probs=q,
                   draft_tokens=g0.integers(0, V, (B, G)).astype(np.int32),
                   uniforms=g0.random((B, G + 1), dtype=np.float32), verify_len=None)
    g, o, rep = check(w)
    assert np.all(g["accepted"] == G)


def test_onehot_draft_zero_target_mass_and_masked_vocab():
    B, G, V = 10, 3, 2048
    g0 = np.random.default_rng(5)
    z = g0.normal(0, 2, size=(B, G + 1, V)).astype(np.float32)
    z[:, :, 1000:1500] = -np.inf                             # masked vocabulary
    x = np.full((B, G), 1200, np.int32)                     # draft a masked token
    q = np.zeros((B, G, V), np.float32)
    q[:, :, 1200] = 1.0                                     # one-hot draft
    w = W.Workload(name="onehot_masked", B=B, G=G, V=V, T=1.0, dtype="f32", logits=z, draft_probs=q,
                   draft_tokens=x, uniforms=g0.random((B, G + 1), dtype=np.float32), verify_len=None)
    g, o, rep = check(w)
    assert np.all(g["accepted"] == 0)
    assert np.all((g["tokens"][:, 0] < 1000) | (g["tokens"][:, 0] >= 1500))


def test_extreme_uniforms():
    w = _rand_workload("u_extremes", 32, 4, 3000, seed=6)
    u = w["uniforms"]
    u[:16] = 0.0
    u[16:] = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    check(w)


def test_low_temperature_and_peaked_rows():
    check(_rand_workload("lowT", 16, 4, 6000, T=0.05, seed=7))
    check(_rand_workload("peaked", 16, 4, 6000, T=1.0, seed=8, zscale=12.0))


def test_data_errors():
    w = _rand_workload("errors", 8, 3, 1500, dtype="f32", seed=9)
    z = w["logits"]
    z[1, 2, 7] = np.nan                      # NaN in a read row
    z[2, 0, 3] = np.inf                      # +inf maximum
    z[3, 1, :] = -np.inf                     # all -inf
    w["draft_tokens"][4, 1] = 1500           # out of range
    w["draft_tokens"][5, 0] = -3
    vl = np.array([3, 3, 3, 3, 3, 3, 4, 1], np.int32)   # request 6: verify_len > G
    z[7, 3, :] = np.nan                      # beyond verify_len=1: never read
    w["verify_len"] = vl
    g, o, rep = check(w)
    assert g["accepted"].tolist()[:7] == [g["accepted"][0], -1, -1, -1, -1, -1, -1]
    assert g["accepted"][7] >= 0


@pytest.mark.parametrize("B,lengths", [(16, False), (13, False), (16, True)])
def test_data_error_after_an_early_rejection(B, lengths):
    """Requests certainly rejected at row 0 whose later rows (or ids) are bad
    are still data errors: the decision that rows 0..j settle goes out before
    the request's later rows are in, and the check of every read row decides
    the outputs.  Full lengths (the grid in XCD order, or not) and verify
    lengths; with and without diagnostics."""
    G, V = 4, 2000
    w = _rand_workload("late_errors", B, G, V, dtype="f32", seed=21)
    z, q, x, u = w["logits"], w["draft_probs"], w["draft_tokens"], w["uniforms"]
    for b in range(8):                        # p(x_0) / q(x_0) ~ e^-40: rejected at row 0
        x[b, 0] = 5
        q[b, 0, :] = 0.0
        q[b, 0, 5] = 1.0
        z[b, 0, 5] = -40.0
        u[b, 0] = 0.5
    z[0, 3, 11] = np.nan                      # NaN in a later row
    z[1, G, 0] = np.inf                       # +inf maximum in the bonus row
    x[2, 2] = V + 7                           # a later id out of range
    z[3, 1, :] = -np.inf                      # a later row all -inf
    x[4, 3] = -1
    if lengths:
        w["verify_len"] = np.full(B, G, np.int32)
    for diag in (True, False):
        g, o, rep = check(w, diag=diag)
        assert g["accepted"][:8].tolist() == [-1] * 5 + [0] * 3
        assert (g["tokens"][:5] == -1).all()


def test_random_shapes_one_launch():
    """Seeded sweep over the one-launch verify's shapes: every depth G up to 15
    (rows spread over one to four waves of the decision workgroup), B in and
    out of multiples of 8, full and random verify lengths, three temperatures,
    bf16 and fp32."""
    g = np.random.default_rng(77)
    for trial in range(14):
        B = int(g.choice([1, 7, 8, 13, 24, 64]))
        G = int(g.integers(1, 16))
        V = int(g.choice([257, 1000, 2048, 4099]))
        T = float(g.choice([0.5, 1.0, 2.0]))
        dtype = "bf16" if trial % 2 == 0 else "f32"
        w = _rand_workload(f"sweep{trial}", B, G, V, T=T, dtype=dtype, seed=100 + trial,
                           zscale=float(g.choice([1.0, 2.0, 4.0])))
        if trial % 3 == 1:
            w["verify_len"] = g.integers(0, G + 1, size=B).astype(np.int32)
        check(w, diag=(trial % 4 == 0))


def test_two_streams_at_once():
    """Calls on two streams (each with its own workspace) run at the same time:
    one-launch verifies of different shapes, with and without verify lengths,
    enqueued back to back without synchronising, each against the oracle."""
    ws = [_rand_workload("stream_a", 16, 7, 20000, seed=61),
          _rand_workload("stream_b", 24, 5, 8000, T=0.7, dtype="f32", seed=62)]
    ws[1]["verify_len"] = np.random.default_rng(63).integers(0, 6, size=24).astype(np.int32)
    orc = [run_oracle(w) for w in ws]
    ins = [to_device(w) for w in ws]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rnd in range(3):
        outs = []
        for w, (z, q, x, u, vl), st in zip(ws, ins, streams):
            with torch.cuda.stream(st):
                outs.append(sv.verify(z, q, x, u, float(w["T"]), vl))
        torch.cuda.synchronize()
        for w, o, (acc, tok) in zip(ws, orc, outs):
            g = {"accepted": acc.cpu().numpy().astype(np.int64), "tokens": tok.cpu().numpy().astype(np.int64)}
            say(f"    round {rnd} {w['name']}:", compare(w, g, o, check_diag=False))


def test_many_requests():
    # Many small requests (T > 0): each request's draw workgroups trail its
    # rows by a lag of many requests in the one launch.
    check(_rand_workload("many_small", 700, 1, 300, seed=10))
    check(_rand_workload("many_tiny", 1500, 1, 64, seed=13))
    # T = 0: 700 requests share the row launch, 1500 exceed half the resident
    # capacity and run as a second launch.
    g0 = np.random.default_rng(14)
    for B, V in ((700, 300), (1500, 64)):
        bits = W.f32_to_bf16_bits((2.0 * g0.normal(size=(B, 2, V))).astype(np.float32))
        a = W.bf16_bits_to_f32(bits).argmax(2)
        x = np.where(g0.random((B, 1)) < 0.5, a[:, :1], g0.integers(0, V, (B, 1))).astype(np.int32)
        w = W.Workload(name=f"many_greedy_{B}", B=B, G=1, V=V, T=0.0, dtype="bf16", logits=bits,
                       draft_probs=None, draft_tokens=x, uniforms=None, verify_len=None)
        say(f"[parity] {w['name']}")
        g = run_gpu(w)
        o = run_oracle(w)
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        np.testing.assert_array_equal(g["tokens"], o["tokens"])


def test_row_pass_event_changes_nothing():
    # Asking for the row-pass event (a timing aid) leaves every output and
    # diagnostic bitwise unchanged, and both calls match the oracle.
    cases = [W.block(B=8, G=15, V=20000), W.tiny(seed=1240), _rand_workload("split_fp32", 5, 4, 3000, dtype="f32", seed=4)]
    w = _rand_workload("split_vlen", 6, 5, 5000, seed=21)
    w["verify_len"] = np.array([0, 5, 2, 3, 1, 4], np.int32)
    cases.append(w)
    for w in cases:
        say(f"[parity] with row-pass event: {w['name']} B={w['B']} G={w['G']} V={w['V']}")
        g1 = run_gpu(w)
        g2 = run_gpu(w, with_event=True)
        for k in g1:
            np.testing.assert_array_equal(np.nan_to_num(g1[k], nan=-7.0), np.nan_to_num(g2[k], nan=-7.0), err_msg=k)
        o = run_oracle(w)
        say("   ", compare(w, g2, o, w.get("verify_len")))


def test_launch_plan_query():
    from lossless_draft_verification_verify_amd import _capi
    torch.cuda.init()
    # sampled with draft probabilities and no verify lengths: one launch
    assert _capi.verify_launches(64, 15, 129280, _capi.SPEC_DTYPE_BF16, 1.0) == 1
    assert _capi.verify_launches(64, 7, 152064, _capi.SPEC_DTYPE_BF16, 0.0) == 1
    # far more requests than half the resident workgroups: the greedy call splits
    assert _capi.verify_launches(60000, 1, 64, _capi.SPEC_DTYPE_BF16, 0.0) == 2


def test_workspace_reuse_and_determinism():
    w1 = W.block(B=8, G=15, V=20000, seed=5)
    w2 = _rand_workload("small", 3, 2, 100, seed=12)
    r1 = run_gpu(w1)
    run_gpu(w2)
    r3 = run_gpu(w1)
    for k in ("accepted", "tokens", "p_draft", "lse", "resid_mass"):
        np.testing.assert_array_equal(np.nan_to_num(r1[k], nan=-7.0), np.nan_to_num(r3[k], nan=-7.0))


def test_workspace_left_zero():
    w = W.block(B=4, G=3, V=9000, seed=3)
    z, q, x, u, vl = to_device(w)
    nbytes = sv.verify_workspace_bytes(4, 3, 9000)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sv.verify(z, q, x, u, 1.0, workspace=ws)
    sv.verify(z, None, x, None, 0.0, workspace=ws)
    sv.verify(z, q, x, u, 1.0, workspace=ws, diag=True)
    torch.cuda.synchronize()
    # every word a call uses is zero again afterwards
    assert not ws.cpu().numpy().any()


def test_workspace_shared_across_shapes():
    """One workspace for calls whose shapes (and so data layouts) differ.

    Regression: counters once sat at offsets that moved with B, so a larger
    batch read an earlier call's partial sums as counters.  No workspace word is
    a counter now: every word carries its own written mark and is zeroed by its
    last reader.
    """
    big = W.block(B=64, G=15, V=20000, seed=21)
    wide = _rand_workload("wide", 700, 1, 300, seed=22)
    need = max(sv.verify_workspace_bytes(64, 15, 20000), sv.verify_workspace_bytes(700, 1, 300))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for w in (big, wide, big, wide):
        z, q, x, u, vl = to_device(w)
        say(f"[parity] shared workspace {w['name']} B={w['B']}")
        acc, tok = sv.verify(z, q, x, u, float(w["T"]), workspace=ws)
        torch.cuda.synchronize()
        o = run_oracle(w)
        g = {"accepted": acc.cpu().numpy().astype(np.int64), "tokens": tok.cpu().numpy().astype(np.int64)}
        compare(w, g, o, check_diag=False)
    assert not ws.cpu().numpy().any()


def test_schedule_run_of_equal_fp32_survivals():
    """The budget cuts through a run of depth-2 candidates that differ only
    below fp32 precision: the kept ones must be the exact order's first."""
    conf = sub_fp32_run_confidences()
    B = conf.shape[0]
    L = B * 3 + 2
    cost = np.ones(L, np.float32)                  # theta always improves: the budget stops the walk
    for extra in (1, 2, 5, 7, 13, 20, 31, 47):
        budget = 2 * B + extra
        lo, To, tauo = oracle.schedule(conf, cost, budget)
        assert sorted(np.flatnonzero(lo == 2).tolist()) != list(range(extra))   # not the index order
        say(f"[parity] schedule, equal-fp32 run, budget {budget}")
        vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(vl.cpu().numpy(), lo, err_msg=f"budget {budget}")
        assert int(T.item()) == To == budget
        assert float(tau.item()) == np.float32(tauo), budget      # tau summed in the same order


def _subset(w, n):
    """The first n requests of workload w (requests are independent)."""
    out = dict(w, B=n)
    for key in ("logits", "draft_probs", "draft_tokens", "uniforms", "verify_len"):
        if out.get(key) is not None:
            out[key] = np.ascontiguousarray(w[key][:n])
    return out


@pytest.mark.parametrize("make", [lambda: W.block(B=64, G=5, V=5000, seed=91),
                                  lambda: W.greedy(B=64, G=5, V=5000, seed=92)], ids=["sampled", "greedy"])
def test_batch_independence_across_placements(make):
    """Requests are verified independently: the first n requests give the same
    outputs, bit for bit, whether n is a multiple of 8 (a request's draw
    workgroups grouped on one XCD) or not (workgroups in request order)."""
    w = make()
    say(f"[parity] batch independence T={w['T']}")
    full = run_gpu(w, diag=False)
    for n in (1, 7, 8, 9, 24, 63):
        part = run_gpu(_subset(w, n), diag=False)
        np.testing.assert_array_equal(part["accepted"], full["accepted"][:n], err_msg=f"n={n}")
        np.testing.assert_array_equal(part["tokens"], full["tokens"][:n], err_msg=f"n={n}")
    compare(w, full, run_oracle(w), check_diag=False)


def test_full_lengths_through_the_length_pass_many_jobs():
    """B = 256 (the largest batch that takes the verify-length row pass), every
    length G: each workgroup of that pass runs several row jobs, and the
    outputs must equal the full-grid row pass's bit for bit."""
    B, G, V = 256, 15, 32768
    say(f"[parity] verify-length pass, B={B} G={G} V={V}")
    gen = torch.Generator(device="cuda").manual_seed(1717)
    z = (torch.randn(B, G + 1, V, device="cuda", generator=gen) * 2).to(torch.bfloat16)
    q = torch.softmax(z[:, :G].float() + 0.5 * torch.randn(B, G, V, device="cuda", generator=gen), dim=-1).contiguous()
    x = torch.randint(0, V, (B, G), device="cuda", dtype=torch.int32, generator=gen)
    u = torch.rand(B, G + 1, device="cuda", generator=gen)
    acc0, tok0 = sv.verify(z, q, x, u, 1.0)
    full = torch.full((B,), G, dtype=torch.int32, device="cuda")
    acc1, tok1 = sv.verify(z, q, x, u, 1.0, full)
    torch.cuda.synchronize()
    assert torch.equal(acc0, acc1) and torch.equal(tok0, tok1)
    assert int((acc0 < 0).sum()) == 0


@pytest.mark.parametrize("lengths", ["random", "full"])
def test_verify_length_pass_many_jobs_against_oracle(lengths):
    """B = 256, G = 15, V = 32768 through the verify-length row pass (the
    largest batch that takes it): each workgroup runs two to four row jobs.
    Random lengths in [0, 15] (zeros and full lengths included) and every
    length G, against the oracle: lengths and tokens under the verify rule,
    p(x_k), q(x_k), R and the row log-sum-exp within their tolerances."""
    B, G, V = 256, 15, 32768
    w = W.block(B=B, G=G, V=V, seed=1718)
    if lengths == "random":
        vl = np.random.default_rng(1718).integers(0, G + 1, size=B).astype(np.int32)
        vl[:8] = [0, G, 0, G, 1, G - 1, 7, G]
    else:
        vl = np.full(B, G, np.int32)
    w["verify_len"] = vl
    _, _, rep = check(w, vl)
    assert rep["requests"] == B and rep["exact"] + rep["flagged_and_differ"] == B
