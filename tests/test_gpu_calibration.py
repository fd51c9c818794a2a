"""GPU parity of calibrated and static scheduling against the float64 oracle,
through the C ABI: the STS apply step inside spec_schedule and spec_dcut,
spec_schedule_static, and the spec_sts_fit grid fit.

Bar:
- schedules from calibrated confidences equal the oracle's schedule of the
  oracle's calibrated confidences exactly (lengths, totals, offsets);
- static schedules are exact;
- each fitted temperature equals the oracle's, unless the oracle's ECE at the
  two grid points agrees to 1e-6. The GPU sums the predictions in 2^-40 fixed
  point, the oracle in float64. Each position is checked given the GPU's own
  earlier temperatures.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import calibration as C
from oracle import dcut as OD
import workloads as W
import lossless_draft_verification_verify_amd as sv

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


def grid32():
    return [float(np.float32(t)) for t in C.grid()]


def rand_temps(g0, G):
    return [float(np.float32(t)) for t in g0.choice(C.grid(), size=G)]


def test_calibrated_schedule_against_oracle():
    g0 = np.random.default_rng(31)
    for trial in range(20):
        B = int(g0.integers(1, 70))
        G = int(g0.integers(1, 17))
        conf = W.confidences(100 + trial, B, G)
        temps = rand_temps(g0, G)
        L = B * (G + 1) + 8
        cost = (1.0 + float(g0.choice([0.0, 0.002, 0.02])) * np.arange(L)).astype(np.float32)
        budget = int(g0.integers(B, L))
        vl, T, tau = sv.schedule(torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda(), budget,
                                 calib_temps=temps)
        torch.cuda.synchronize()
        lo, To, _ = oracle.schedule(C.sts_apply(conf, temps), cost, budget)
        np.testing.assert_array_equal(vl.cpu().numpy(), lo, err_msg=f"trial {trial}")
        assert int(T.item()) == To


def test_calibrated_dcut_against_oracle():
    g0 = np.random.default_rng(32)
    for trial in range(20):
        B = int(g0.integers(1, 70))
        G = int(g0.integers(1, 17))
        conf = W.confidences(200 + trial, B, G)
        temps = rand_temps(g0, G)
        costs = W.ratio_costs(B, G)
        vl, off, r, K, U = sv.dcut(torch.from_numpy(conf).cuda(), W.RATIOS, costs, calib_temps=temps)
        torch.cuda.synchronize()
        d = OD.dcut(C.sts_apply(conf, temps), W.RATIOS, costs)
        assert int(r.item()) == d["ratio_index"], trial
        np.testing.assert_array_equal(off.cpu().numpy(), d["row_offsets"], err_msg=f"trial {trial}")


def test_calibration_at_unit_temperature_changes_nothing():
    conf = W.confidences(7, 64, 15)
    cost = W.linear_cost(table_len=513)
    c, t = torch.from_numpy(conf).cuda(), torch.from_numpy(cost).cuda()
    a = sv.schedule(c, t, 512)[0].cpu().numpy()
    b = sv.schedule(c, t, 512, calib_temps=[1.0] * 15)[0].cpu().numpy()
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("B,G", [(64, 15), (5, 3), (1000, 7), (65536, 4), (3, 0), (4096, 255)])
def test_static_modes_against_oracle(B, G):
    g0 = np.random.default_rng(B + G)
    conf = W.confidences(300 + B, B, G) if G > 0 else np.zeros((B, 0), np.float32)
    c = torch.from_numpy(conf).cuda()
    for L in (0, 3, G, G + 5, -2):
        vl, T, off = sv.schedule_static(c, fixed_len=L)
        torch.cuda.synchronize()
        n = C.static_fixed(B, G, L)
        np.testing.assert_array_equal(vl.cpu().numpy(), n)
        assert int(T.item()) == int((n + 1).sum())
        np.testing.assert_array_equal(off.cpu().numpy(), OD.row_offsets(n))
    temps = rand_temps(g0, G) if G > 0 else None
    for tau in (0.0, 0.5, 0.8, 1.0):
        for cal in (None, temps):
            vl, T, off = sv.schedule_static(c, threshold=tau, calib_temps=cal)
            torch.cuda.synchronize()
            n = C.static_threshold(conf if cal is None else C.sts_apply(conf, cal), tau)
            np.testing.assert_array_equal(vl.cpu().numpy(), n, err_msg=f"tau {tau} calib {cal is not None}")
            assert int(T.item()) == int((n + 1).sum())
            np.testing.assert_array_equal(off.cpu().numpy(), OD.row_offsets(n))


def check_fit(conf, L, temps, bins=15, tag=""):
    g = sv.sts_fit(torch.from_numpy(conf).cuda(), torch.from_numpy(L.astype(np.int32)).cuda(), temps, bins)
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    # the oracle's ECE table position by position, given the GPU's earlier choices
    c = np.clip(np.where(np.isnan(conf), 0.0, conf.astype(np.float64)), 0.0, 1.0)
    tt = np.asarray(temps, np.float32).astype(np.float64)
    prefix = np.ones(len(L))
    near = 0
    for k in range(conf.shape[1]):
        y = (L > k).astype(np.float64)
        e = np.array([C.ece(prefix * C.power(c[:, k], T), y, bins) for T in tt])
        best = int(np.argmin(e))
        gi = int(np.argmin(np.abs(tt - g[k])))
        assert tt[gi] == g[k], (tag, k, g[k])
        if gi != best:
            assert abs(e[gi] - e[best]) <= 1e-6, (tag, k, tt[gi], tt[best], e[gi], e[best])
            near += 1
        prefix = prefix * C.power(c[:, k], g[k])
    say(f"    {tag}: fitted {np.round(g, 2).tolist()}, near ties {near}")
    return g


def test_sts_fit_recovers_known_temperatures():
    conf, L, T = W.calibration(60000, G=6)
    g = check_fit(conf, L, grid32(), tag="N=60000 G=6")
    assert np.all(np.abs(g - T) <= 0.25)
    # and the oracle's own fit agrees
    np.testing.assert_array_equal(g, C.sts_fit(conf, L))


@pytest.mark.parametrize("N,G,bins,nt", [(1000, 3, 15, 100), (1025, 15, 15, 100), (300000, 4, 15, 100),
                                         (5000, 5, 32, 40), (777, 2, 1, 7)])
def test_sts_fit_shapes(N, G, bins, nt):
    conf, L, _ = W.calibration(N, G=G, true_temps=np.linspace(0.5, 2.0, G), seed=N)
    temps = [float(np.float32(t)) for t in np.linspace(0.1, 10.0, nt)]
    check_fit(conf, L, temps, bins, tag=f"N={N} G={G} bins={bins} grid={nt}")


def test_fit_then_calibrated_schedule():
    """The fitted temperatures feed the scheduler's apply step."""
    conf, L, _ = W.calibration(40000, G=15)
    fitted = sv.sts_fit(torch.from_numpy(conf).cuda(), torch.from_numpy(L).cuda(), grid32())
    torch.cuda.synchronize()
    temps = fitted.cpu().numpy().tolist()
    c64 = W.confidences(9, 64, 15)
    cost = W.linear_cost(table_len=513)
    vl, T, _ = sv.schedule(torch.from_numpy(c64).cuda(), torch.from_numpy(cost).cuda(), 512, calib_temps=temps)
    torch.cuda.synchronize()
    lo, To, _ = oracle.schedule(C.sts_apply(c64, temps), cost, 512)
    np.testing.assert_array_equal(vl.cpu().numpy(), lo)
    say(f"    calibrated schedule T={To} (uncalibrated {oracle.schedule(c64, cost, 512)[1]})")


@pytest.mark.parametrize("calibrated", [False, True])
def test_static_threshold_then_verify_full_size(calibrated):
    """spec_schedule_static (threshold 0.5) feeding spec_verify on the device at
    the full vocabulary (B = 64, G = 15, V = 129280): the verify-length row
    pass runs about two row jobs per workgroup.  Lengths exact against the
    oracle's static threshold; lengths, tokens and diagnostics of the verify
    against the oracle's verification with those lengths."""
    from parity_util import compare, run_gpu, run_oracle
    w = W.scheduled(64)
    conf = w["confidence"]
    temps = W.calibration(2, G=15)[2].astype(np.float32).tolist() if calibrated else None
    say(f"[parity] static threshold 0.5 then verify, B=64 V=129280 calibrated={calibrated}")
    vl, T, _ = sv.schedule_static(torch.from_numpy(conf).cuda(), threshold=0.5, calib_temps=temps,
                                  row_offsets=False)
    torch.cuda.synchronize()
    n = C.static_threshold(conf if temps is None else C.sts_apply(conf, temps), 0.5)
    np.testing.assert_array_equal(vl.cpu().numpy(), n)
    assert int(T.item()) == int((n + 1).sum())
    g = run_gpu(w, verify_len=vl)
    o = run_oracle(w, n)
    rep = compare(w, g, o, n)
    say("   ", rep, "positions", int(n.sum()))
