"""ctypes prototypes of libspecverify.so (the C ABI declared in include/spec_verify.h).

Argument marshalling only.  Loading fails loudly when the library has not been
built; there is no fallback implementation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK = 0
STATUS_NAMES = {
    0: "SPEC_OK",
    1: "SPEC_ERR_NULL_POINTER",
    2: "SPEC_ERR_BAD_SHAPE",
    3: "SPEC_ERR_BAD_TEMPERATURE",
    4: "SPEC_ERR_BAD_DTYPE",
    5: "SPEC_ERR_WORKSPACE_TOO_SMALL",
    6: "SPEC_ERR_UNSUPPORTED",
    7: "SPEC_ERR_DEVICE",
    8: "SPEC_ERR_MISALIGNED",
    9: "SPEC_ERR_SCRATCH_TOO_SMALL",
}
NOALLOC_SCRATCH_BYTES = 8 << 20
SPEC_DTYPE_F32 = 0
SPEC_DTYPE_BF16 = 1
SPEC_DRAFT_PROBS = 0
SPEC_DRAFT_LOGITS = 1
SPEC_STATIC_FIXED = 0
SPEC_STATIC_THRESHOLD = 1

# Every symbol the header declares.
EXPORTS = (
    "spec_verify_workspace_bytes",
    "spec_verify",
    "spec_verify_launches",
    "spec_verify_noalloc",
    "spec_schedule_workspace_bytes",
    "spec_schedule",
    "spec_schedule_calibrated",
    "spec_verify_packed",
    "spec_verify_logits",
    "spec_verify_tree",
    "spec_dcut",
    "spec_acceptance",
    "spec_schedule_static",
    "spec_sts_fit_workspace_bytes",
    "spec_sts_fit",
    "spec_status_string",
)
MAX_RATIOS = 8


class DiagT(ctypes.Structure):
    _fields_ = [
        ("target_lse", ctypes.c_void_p),
        ("p_draft", ctypes.c_void_p),
        ("q_draft", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p),
        ("row_pass_event", ctypes.c_void_p),
    ]


class SpecError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def load():
    """Load libspecverify.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m lossless_draft_verification_verify_amd.build` "
            "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp,
                                ctypes.POINTER(DiagT), vp, sz, vp]
    lib.spec_verify.restype = ctypes.c_int
    lib.spec_verify_noalloc.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp,
                                        ctypes.POINTER(DiagT), vp]
    lib.spec_verify_noalloc.restype = ctypes.c_int
    lib.spec_verify_launches.argtypes = [i32, i32, i32, ctypes.c_int, f32]
    lib.spec_verify_launches.restype = i32
    lib.spec_schedule_workspace_bytes.argtypes = [i32, i32]
    lib.spec_schedule_workspace_bytes.restype = sz
    fp = ctypes.POINTER(f32)
    lib.spec_schedule.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.spec_schedule.restype = ctypes.c_int
    lib.spec_schedule_calibrated.argtypes = [vp, fp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.spec_schedule_calibrated.restype = ctypes.c_int
    lib.spec_verify_packed.argtypes = [vp, ctypes.c_int, i32, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp,
                                       ctypes.POINTER(DiagT), vp, sz, vp]
    lib.spec_verify_packed.restype = ctypes.c_int
    lib.spec_verify_logits.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp,
                                       ctypes.POINTER(DiagT), vp, sz, vp]
    lib.spec_verify_logits.restype = ctypes.c_int
    lib.spec_verify_tree.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_tree.restype = ctypes.c_int
    lib.spec_dcut.argtypes = [vp, i32, i32, fp, fp, i32, fp, vp, vp, vp, vp, vp, vp]
    lib.spec_dcut.restype = ctypes.c_int
    lib.spec_acceptance.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, i32, i32, i32, f32, vp, vp]
    lib.spec_acceptance.restype = ctypes.c_int
    lib.spec_schedule_static.argtypes = [vp, i32, i32, ctypes.c_int, i32, f32, fp, vp, vp, vp, vp]
    lib.spec_schedule_static.restype = ctypes.c_int
    lib.spec_sts_fit_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_sts_fit_workspace_bytes.restype = sz
    lib.spec_sts_fit.argtypes = [vp, vp, i32, i32, fp, i32, i32, vp, vp, sz, vp]
    lib.spec_sts_fit.restype = ctypes.c_int
    lib.spec_status_string.argtypes = [ctypes.c_int]
    lib.spec_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load().spec_status_string(int(status)).decode()


def verify_workspace_bytes(B, G, V, dtype_code):
    return int(load().spec_verify_workspace_bytes(B, G, V, dtype_code))


def verify_launches(B, G, V, dtype_code, T):
    return int(load().spec_verify_launches(B, G, V, dtype_code, ctypes.c_float(T)))


def schedule_workspace_bytes(B, G):
    return int(load().spec_schedule_workspace_bytes(B, G))


def spec_verify(logits, dtype_code, q, x, u, vlen, B, G, V, T, out_acc, out_tok, diag, ws, ws_bytes, stream):
    """Raw call; pointers are ints (0 = NULL), `diag` a DiagT or None.  Returns the status."""
    d = ctypes.byref(diag) if diag is not None else None
    return int(load().spec_verify(logits or None, dtype_code, q or None, x or None, u or None, vlen or None,
                                  B, G, V, ctypes.c_float(T), out_acc or None, out_tok or None, d,
                                  ws or None, ws_bytes, stream or None))


def spec_verify_noalloc(logits, dtype_code, q, x, u, vlen, B, G, V, T, out_acc, out_tok, diag, stream):
    """Raw call of the no-allocation variant (static scratch); returns the status."""
    d = ctypes.byref(diag) if diag is not None else None
    return int(load().spec_verify_noalloc(logits or None, dtype_code, q or None, x or None, u or None,
                                          vlen or None, B, G, V, ctypes.c_float(T), out_acc or None,
                                          out_tok or None, d, stream or None))


def _floats(v):
    """A host float array for the C ABI (None = NULL)."""
    if v is None:
        return None
    return (ctypes.c_float * max(1, len(v)))(*[float(t) for t in v])


def spec_schedule(conf, cost, table_len, B, G, budget, eps, out_len, out_T, out_tau, ws, ws_bytes, stream):
    return int(load().spec_schedule(conf or None, cost or None, table_len, B, G, budget, ctypes.c_float(eps),
                                    out_len or None, out_T or None, out_tau or None, ws or None,
                                    ws_bytes, stream or None))


def spec_schedule_calibrated(conf, calib, cost, table_len, B, G, budget, eps, out_len, out_T, out_tau, ws, ws_bytes,
                             stream):
    """`calib`: a host sequence of G temperatures (None = NULL)."""
    return int(load().spec_schedule_calibrated(conf or None, _floats(calib), cost or None, table_len, B, G, budget,
                                               ctypes.c_float(eps), out_len or None, out_T or None, out_tau or None,
                                               ws or None, ws_bytes, stream or None))


def spec_verify_packed(logits, dtype_code, rows, roff, q, x, u, B, G, V, T, out_acc, out_tok, diag, ws, ws_bytes,
                       stream):
    """Raw call; pointers are ints (0 = NULL), `diag` a DiagT or None.  Returns the status."""
    d = ctypes.byref(diag) if diag is not None else None
    return int(load().spec_verify_packed(logits or None, dtype_code, rows, roff or None, q or None, x or None,
                                         u or None, B, G, V, ctypes.c_float(T), out_acc or None, out_tok or None, d,
                                         ws or None, ws_bytes, stream or None))


def spec_dcut(conf, B, G, ratios, costs, out_len, out_off, out_ratio, out_rows, out_util, stream, calib=None):
    """Raw call; `ratios`, `costs` and `calib` are host sequences of floats (None = NULL)."""
    n = len(ratios) if ratios is not None else (len(costs) if costs is not None else 0)
    return int(load().spec_dcut(conf or None, B, G, _floats(ratios), _floats(costs), n, _floats(calib),
                                out_len or None, out_off or None, out_ratio or None, out_rows or None,
                                out_util or None, stream or None))


def spec_acceptance(logits, dtype_code, draft, draft_kind, vlen, B, G, V, T, out_alpha, stream):
    return int(load().spec_acceptance(logits or None, dtype_code, draft or None, draft_kind, vlen or None, B, G, V,
                                      ctypes.c_float(T), out_alpha or None, stream or None))


def spec_verify_logits(logits, dtype_code, dl, x, u, vlen, B, G, V, T, out_acc, out_tok, diag, ws, ws_bytes, stream):
    d = ctypes.byref(diag) if diag is not None else None
    return int(load().spec_verify_logits(logits or None, dtype_code, dl or None, x or None, u or None, vlen or None,
                                         B, G, V, ctypes.c_float(T), out_acc or None, out_tok or None, d,
                                         ws or None, ws_bytes, stream or None))


def spec_schedule_static(conf, B, G, mode, fixed_len, tau, calib, out_len, out_T, out_off, stream):
    return int(load().spec_schedule_static(conf or None, B, G, mode, fixed_len, ctypes.c_float(tau), _floats(calib),
                                           out_len or None, out_T or None, out_off or None, stream or None))


def sts_fit_workspace_bytes(N, G, nt, bins):
    return int(load().spec_sts_fit_workspace_bytes(N, G, nt, bins))


def spec_sts_fit(conf, acc_len, N, G, temps, bins, out_temps, ws, ws_bytes, stream):
    n = len(temps) if temps is not None else 0
    return int(load().spec_sts_fit(conf or None, acc_len or None, N, G, _floats(temps), n, bins, out_temps or None,
                                   ws or None, ws_bytes, stream or None))


def spec_verify_tree(logits, dtype_code, par, tok, B, M, V, out_acc, out_tok, out_path, ws, ws_bytes, stream):
    return int(load().spec_verify_tree(logits or None, dtype_code, par or None, tok or None, B, M, V,
                                       out_acc or None, out_tok or None, out_path or None, ws or None, ws_bytes,
                                       stream or None))
