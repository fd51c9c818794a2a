"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function include/spec_verify.h declares, sizes
its workspace, and rejects bad arguments with a status before touching the
device (argument errors are caught before any HIP call, so these run on a
machine without a GPU).  Pointers below are fake, never dereferenced.
"""

import os
import re

import pytest

from lossless_draft_verification_verify_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

# Fake, suitably aligned device addresses (never dereferenced by host validation).
P = 0x7F0000000000
Z, Q, X, U, VL, OA, OT, WS = (P + i * 0x100000 for i in range(8))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _capi.load()
    declared = header_functions()
    assert set(declared) == set(_capi.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(10):
        s = _capi.status_string(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert _capi.status_string(99) == "unknown status"


def test_workspace_query():
    w = _capi.verify_workspace_bytes(64, 15, 129280, _capi.SPEC_DTYPE_BF16)
    # a 256-byte zero block + partials 64*16 rows*64 chunks*8 B (sized for the
    # greedy per-chunk count) + draft-row partials 64*15*64*8 B (draft logits)
    # + masses 64*64 sub-tiles*16 B + gathers 64*15*8 B + decision records 64*32 B
    assert w == 256 + 64 * 16 * 64 * 8 + 64 * 15 * 64 * 8 + 65536 + 64 * 15 * 8 + 64 * 32
    # every region is 256-byte aligned, the smallest shape included
    assert _capi.verify_workspace_bytes(1, 0, 1, _capi.SPEC_DTYPE_BF16) == 4 * 256
    assert _capi.verify_workspace_bytes(64, 15, 129280, _capi.SPEC_DTYPE_F32) >= w
    assert _capi.verify_workspace_bytes(0, 15, 100, 1) == 0
    assert _capi.verify_workspace_bytes(1, -1, 100, 1) == 0
    assert _capi.verify_workspace_bytes(1, 1, 100, 7) == 0
    assert _capi.verify_workspace_bytes(1, 256, 100, 1) == 0
    assert _capi.schedule_workspace_bytes(64, 15) == 0


def test_verify_launches_rejects_bad_arguments():
    # Invalid shapes, dtype or temperature give -1 before any device query.
    assert _capi.verify_launches(0, 15, 100, 1, 1.0) == -1
    assert _capi.verify_launches(1, 256, 100, 1, 1.0) == -1
    assert _capi.verify_launches(1, 3, 100, 7, 1.0) == -1
    assert _capi.verify_launches(1, 3, 100, 1, -1.0) == -1
    assert _capi.verify_launches(1, 3, 100, 1, float("nan")) == -1


def _verify(**kw):
    args = dict(logits=Z, dtype_code=1, q=Q, x=X, u=U, vlen=0, B=4, G=3, V=1000, T=1.0, out_acc=OA,
                out_tok=OT, diag=None, ws=WS, ws_bytes=1 << 20, stream=0)
    args.update(kw)
    return _capi.spec_verify(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype_code=5), 4),
    (dict(B=0), 2), (dict(G=-1), 2), (dict(V=0), 2),
    (dict(G=256), 6), (dict(V=(1 << 30) + 1), 6), (dict(B=65537, V=10), 6),
    (dict(T=-0.5), 3), (dict(T=float("nan")), 3), (dict(T=float("inf")), 3), (dict(T=1e-39), 3),
    (dict(logits=0), 1), (dict(out_acc=0), 1), (dict(out_tok=0), 1), (dict(x=0), 1),
    (dict(q=0), 1), (dict(u=0), 1), (dict(ws=0), 1),
    (dict(logits=Z + 1), 8), (dict(q=Q + 2), 8), (dict(x=X + 2), 8), (dict(vlen=VL + 1), 8),
    (dict(ws=WS + 16), 8), (dict(logits=Z + 2, dtype_code=0), 8),
    (dict(ws_bytes=100), 5),
])
def test_verify_rejects_bad_arguments(kw, status):
    assert _verify(**kw) == status


def test_verify_nullable_inputs_follow_the_mode():
    # T == 0: q and u may be NULL; G == 0: q and x may be NULL.  These pass
    # validation, so they must fail later only for lack of a device: check
    # just that they are not reported as NULL pointers.
    assert _verify(T=0.0, q=0, u=0, ws_bytes=100) == 5
    assert _verify(G=0, q=0, x=0, ws_bytes=100) == 5


def test_verify_diag_alignment_checked():
    d = _capi.DiagT(P + 2, 0, 0, 0, 0)
    assert _verify(diag=d) == 8


def _sched(calib=None, **kw):
    args = dict(conf=Q, cost=U, table_len=513, B=4, G=15, budget=512, eps=0.0, out_len=OA, out_T=OT,
                out_tau=X, ws=0, ws_bytes=0, stream=0)
    args.update(kw)
    if calib is None:
        return _capi.spec_schedule(**args)
    return _capi.spec_schedule_calibrated(calib=calib, **args)


def _declaration(name):
    """(type, name) pairs of a function's parameters as include/spec_verify.h declares it."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    out = []
    for p in m.group(1).split(","):
        p = " ".join(p.replace("*", " * ").split())
        typ, _, nm = p.rpartition(" ")
        out.append((typ.replace(" *", "*"), nm))
    return out


# The scheduler's boundary as the hot-path scope fixes it: confidences, cost
# table and budget in, lengths and totals out, then the workspace and stream.
SCHEDULE_PROTOTYPE = [
    ("const float*", "confidence"), ("const float*", "cost_table"), ("int32_t", "table_len"),
    ("int32_t", "B"), ("int32_t", "G"), ("int32_t", "token_budget"), ("float", "eps"),
    ("int32_t*", "out_verify_len"), ("int32_t*", "out_total_tokens"), ("float*", "out_expected_tokens"),
    ("void*", "workspace"), ("size_t", "workspace_bytes"), ("spec_stream_t", "stream"),
]
VERIFY_PROTOTYPE = [
    ("const void*", "target_logits"), ("spec_dtype_t", "target_dtype"), ("const float*", "draft_probs"),
    ("const int32_t*", "draft_tokens"), ("const float*", "uniforms"), ("const int32_t*", "verify_len"),
    ("int32_t", "B"), ("int32_t", "G"), ("int32_t", "V"), ("float", "temperature"),
    ("int32_t*", "out_accepted"), ("int32_t*", "out_tokens"), ("const spec_verify_diag_t*", "diag"),
    ("void*", "workspace"), ("size_t", "workspace_bytes"), ("spec_stream_t", "stream"),
]


def test_boundary_prototypes_are_pinned():
    assert _declaration("spec_schedule") == SCHEDULE_PROTOTYPE
    assert _declaration("spec_verify") == VERIFY_PROTOTYPE
    # the calibrated scheduler is spec_schedule with the host temperatures after the confidences
    cal = _declaration("spec_schedule_calibrated")
    assert cal == SCHEDULE_PROTOTYPE[:1] + [("const float*", "calib_temps")] + SCHEDULE_PROTOTYPE[1:]
    # the binding's ctypes prototype has as many arguments as the declaration
    lib = _capi.load()
    assert len(lib.spec_schedule.argtypes) == len(SCHEDULE_PROTOTYPE)
    assert len(lib.spec_schedule_calibrated.argtypes) == len(cal)
    assert len(lib.spec_verify.argtypes) == len(VERIFY_PROTOTYPE)


def test_calibrated_schedule_validates_like_schedule():
    # every argument error of spec_schedule is reported the same way by the calibrated entry point
    for kw, status in [(dict(B=0), 2), (dict(budget=513), 2), (dict(conf=0), 1), (dict(out_len=0), 1),
                       (dict(conf=Q + 1), 8), (dict(B=300, G=15, budget=400), 6)]:
        assert _sched(calib=[1.0] * kw.get("G", 15), **kw) == status, kw


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=-1), 2), (dict(table_len=0), 2),
    (dict(budget=3), 2), (dict(budget=513), 2), (dict(eps=float("nan")), 2),
    (dict(B=300, G=15, budget=400), 6), (dict(B=5000, G=0, budget=5000, table_len=6000), 6),
    (dict(conf=0), 1), (dict(cost=0), 1), (dict(out_len=0), 1), (dict(out_T=0), 1),
    (dict(conf=Q + 1), 8), (dict(out_tau=X + 2), 8),
])
def test_schedule_rejects_bad_arguments(kw, status):
    assert _sched(**kw) == status


def _packed(**kw):
    args = dict(logits=Z, dtype_code=1, rows=40, roff=VL, q=Q, x=X, u=U, B=4, G=3, V=1000, T=1.0, out_acc=OA,
                out_tok=OT, diag=None, ws=WS, ws_bytes=1 << 20, stream=0)
    args.update(kw)
    return _capi.spec_verify_packed(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(roff=0), 1), (dict(rows=0), 2), (dict(rows=-3), 2),
    (dict(rows=1 << 30, V=1 << 20), 6),
    (dict(roff=VL + 2), 8), (dict(logits=Z + 1), 8),
    (dict(dtype_code=5), 4), (dict(B=0), 2), (dict(T=-1.0), 3), (dict(ws_bytes=100), 5),
    (dict(q=0), 1), (dict(u=0), 1), (dict(x=0), 1),
])
def test_verify_packed_rejects_bad_arguments(kw, status):
    assert _packed(**kw) == status


def test_verify_packed_passes_validation_with_a_small_workspace_only():
    # Valid packed arguments fail only on the workspace size, never as NULL.
    assert _packed(T=0.0, q=0, u=0, ws_bytes=100) == 5
    assert _packed(G=0, q=0, x=0, ws_bytes=100) == 5


def _dcut(**kw):
    args = dict(conf=Q, B=64, G=15, ratios=[0.25, 0.5, 0.75, 1.0], costs=[1.0, 1.1, 1.2, 1.3], out_len=OA,
                out_off=OT, out_ratio=X, out_rows=U, out_util=WS, stream=0)
    args.update(kw)
    return _capi.spec_dcut(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=-1), 2),
    (dict(B=300, G=15), 6), (dict(B=5000, G=0), 6),
    (dict(ratios=[], costs=[]), 2), (dict(ratios=[0.5] * 9, costs=[1.0] * 9), 2),
    (dict(ratios=[0.0, 0.5, 0.75, 1.0]), 2), (dict(ratios=[0.25, 0.5, 0.75, 1.5]), 2),
    (dict(ratios=[0.25, float("nan"), 0.75, 1.0]), 2), (dict(ratios=[-0.25, 0.5, 0.75, 1.0]), 2),
    (dict(costs=[1.0, 0.0, 1.0, 1.0]), 2), (dict(costs=[1.0, float("inf"), 1.0, 1.0]), 2),
    (dict(costs=[1.0, -1.0, 1.0, 1.0]), 2),
    (dict(ratios=None), 1), (dict(costs=None), 1),
    (dict(conf=0), 1), (dict(out_len=0), 1), (dict(out_off=0), 1), (dict(out_ratio=0), 1), (dict(out_rows=0), 1),
    (dict(conf=Q + 2), 8), (dict(out_off=OT + 1), 8), (dict(out_util=WS + 4), 8),
])
def test_dcut_rejects_bad_arguments(kw, status):
    assert _dcut(**kw) == status


def _acc(**kw):
    args = dict(logits=Z, dtype_code=1, draft=Q, draft_kind=1, vlen=0, B=4, G=3, V=1000, T=1.0, out_alpha=OA,
                stream=0)
    args.update(kw)
    return _capi.spec_acceptance(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype_code=5), 4), (dict(draft_kind=2), 4),
    (dict(B=0), 2), (dict(G=-1), 2), (dict(V=0), 2), (dict(G=256), 6),
    (dict(T=0.0), 3), (dict(T=-1.0), 3), (dict(T=float("nan")), 3), (dict(T=float("inf")), 3),
    (dict(logits=0), 1), (dict(draft=0), 1), (dict(out_alpha=0), 1),
    (dict(logits=Z + 1), 8), (dict(draft=Q + 1), 8), (dict(draft=Q + 2, draft_kind=0), 8),
    (dict(vlen=VL + 2), 8), (dict(out_alpha=OA + 2), 8),
])
def test_acceptance_rejects_bad_arguments(kw, status):
    assert _acc(**kw) == status


def test_acceptance_without_drafts_enqueues_nothing():
    # G == 0: nothing to compute, valid without draft or output pointers.
    assert _acc(G=0, draft=0, out_alpha=0) == 0


def _logits(**kw):
    args = dict(logits=Z, dtype_code=1, dl=Q, x=X, u=U, vlen=0, B=4, G=3, V=1000, T=1.0, out_acc=OA, out_tok=OT,
                diag=None, ws=WS, ws_bytes=1 << 20, stream=0)
    args.update(kw)
    return _capi.spec_verify_logits(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dl=0), 1), (dict(dl=Q + 1), 8), (dict(x=0), 1), (dict(u=0), 1), (dict(logits=0), 1),
    (dict(dtype_code=5), 4), (dict(B=0), 2), (dict(T=-1.0), 3), (dict(ws_bytes=100), 5),
    (dict(B=65536, G=255, V=1 << 20), 6),
])
def test_verify_logits_rejects_bad_arguments(kw, status):
    assert _logits(**kw) == status


def test_verify_logits_nullable_draft():
    # T == 0 (greedy) and G == 0 read no draft logits.
    assert _logits(T=0.0, dl=0, u=0, ws_bytes=100) == 5
    assert _logits(G=0, dl=0, x=0, ws_bytes=100) == 5


@pytest.mark.parametrize("calib", [[1.0, 0.0, 1.0], [1.0, -2.0, 1.0], [float("nan"), 1.0, 1.0],
                                   [1.0, float("inf"), 1.0]])
def test_calibration_temperatures_validated(calib):
    assert _sched(G=3, calib=calib) == 2
    assert _dcut(G=3, calib=calib) == 2
    assert _capi.spec_schedule_static(Q, 4, 3, 1, 0, 0.5, calib, OA, OT, 0, 0) == 2


def _static(**kw):
    args = dict(conf=Q, B=4, G=15, mode=1, fixed_len=0, tau=0.5, calib=None, out_len=OA, out_T=OT, out_off=X,
                stream=0)
    args.update(kw)
    return _capi.spec_schedule_static(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=-1), 2), (dict(mode=2), 2), (dict(tau=float("nan")), 2),
    (dict(B=65537), 6), (dict(G=256), 6),
    (dict(out_len=0), 1), (dict(conf=0), 1),
    (dict(conf=Q + 2), 8), (dict(out_off=X + 1), 8),
])
def test_static_rejects_bad_arguments(kw, status):
    assert _static(**kw) == status


def test_static_fixed_needs_no_confidence():
    # passes validation; the launch itself fails only for lack of a device, never as NULL (1)
    assert _static(mode=0, conf=0, fixed_len=3) != 1


def _fit(**kw):
    args = dict(conf=Q, acc_len=X, N=1000, G=4, temps=[0.5, 1.0, 2.0], bins=15, out_temps=OA, ws=WS,
                ws_bytes=1 << 24, stream=0)
    args.update(kw)
    return _capi.spec_sts_fit(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 2), (dict(G=-1), 2), (dict(bins=0), 2), (dict(bins=33), 2), (dict(temps=[]), 2),
    (dict(temps=[1.0] * 129), 2), (dict(temps=[1.0, 0.0]), 2), (dict(temps=[float("nan")]), 2),
    (dict(N=1 << 23), 6), (dict(G=256), 6),
    (dict(conf=0), 1), (dict(acc_len=0), 1), (dict(out_temps=0), 1), (dict(ws=0), 1), (dict(temps=None), 2),
    (dict(ws=WS + 8), 8), (dict(ws_bytes=100), 5),
])
def test_sts_fit_rejects_bad_arguments(kw, status):
    assert _fit(**kw) == status


def test_sts_fit_workspace_query():
    assert _capi.sts_fit_workspace_bytes(1000, 4, 100, 15) == 8192 + 1024 + 1 * 100 * 15 * 2 * 8
    assert _capi.sts_fit_workspace_bytes(1 << 20, 4, 100, 15) == (1 << 23) + 1024 + 256 * 100 * 15 * 2 * 8
    assert _capi.sts_fit_workspace_bytes(0, 4, 100, 15) == 0
    assert _capi.sts_fit_workspace_bytes(10, 4, 128, 32) > 0        # 128 * 32 * 16 B of LDS fits


def _tree(**kw):
    args = dict(logits=Z, dtype_code=1, par=Q, tok=X, B=4, M=8, V=1000, out_acc=OA, out_tok=OT, out_path=U, ws=WS,
                ws_bytes=1 << 20, stream=0)
    args.update(kw)
    return _capi.spec_verify_tree(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype_code=5), 4), (dict(M=0), 2), (dict(B=0), 2), (dict(V=0), 2), (dict(M=257), 6),
    (dict(logits=0), 1), (dict(par=0), 1), (dict(tok=0), 1), (dict(out_acc=0), 1), (dict(out_tok=0), 1),
    (dict(out_path=0), 1), (dict(ws=0), 1),
    (dict(logits=Z + 1), 8), (dict(par=Q + 2), 8), (dict(ws=WS + 8), 8), (dict(ws_bytes=100), 5),
])
def test_verify_tree_rejects_bad_arguments(kw, status):
    assert _tree(**kw) == status


def test_verify_tree_root_only_needs_no_tree():
    assert _tree(M=1, par=0, tok=0, ws_bytes=10) == 5


def _noalloc(**kw):
    args = dict(logits=Z, dtype_code=1, q=Q, x=X, u=U, vlen=0, B=4, G=3, V=1000, T=1.0, out_acc=OA, out_tok=OT,
                diag=None, stream=0)
    args.update(kw)
    return _capi.spec_verify_noalloc(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype_code=5), 4), (dict(B=0), 2), (dict(G=256), 6), (dict(T=-1.0), 3),
    (dict(logits=0), 1), (dict(q=0), 1), (dict(u=0), 1), (dict(out_acc=0), 1),
    (dict(logits=Z + 1), 8), (dict(vlen=VL + 2), 8),
    # beyond the static scratch: refused before any device call
    (dict(B=1000, G=15, V=129280), 9), (dict(B=65536, G=3, V=8192), 9),
])
def test_noalloc_rejects_bad_arguments(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SPEC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _capi.NOALLOC_SCRATCH_BYTES
    # the headline shape fits, with room for several times its batch
    assert _capi.verify_workspace_bytes(64, 15, 129280, _capi.SPEC_DTYPE_BF16) * 7 < _capi.NOALLOC_SCRATCH_BYTES
