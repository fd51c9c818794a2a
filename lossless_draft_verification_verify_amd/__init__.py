"""Batched lossless draft verification and confidence-scheduled depth on MI355X.

Thin PyTorch-facing binding of libspecverify.so (C ABI in include/spec_verify.h).
It only checks tensor metadata, passes device pointers and the current HIP
stream, and keeps one zero-filled workspace per (device, stream).  Every step of
the computation runs in the library's HIP kernels; there is no fallback.

    acc, tok = verify(target_logits, draft_probs, draft_tokens, uniforms, temperature)
    vlen, T, tau = schedule(confidence, cost_table, token_budget)
    acc, tok = verify(..., verify_len=vlen)
    vlen, offsets, r, K, U = dcut(confidence, (0.25, 0.5, 0.75, 1.0), ratio_cost)
    acc, tok = verify_packed(packed_logits, offsets, draft_probs, draft_tokens, uniforms, temperature)
"""

import torch

from . import _capi
from ._capi import SpecError, SPEC_DTYPE_BF16, SPEC_DTYPE_F32  # noqa: F401

__all__ = ["verify", "verify_packed", "verify_tree", "schedule", "dcut", "acceptance", "schedule_static", "sts_fit",
           "verify_workspace_bytes", "SpecError", "load"]

_workspaces = {}


def load():
    """Load the native library (raises ImportError if it is not built)."""
    return _capi.load()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    raise TypeError(f"target_logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t, dtype, device, name):
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def verify_workspace_bytes(B, G, V, dtype=torch.bfloat16):
    code = SPEC_DTYPE_BF16 if dtype == torch.bfloat16 else SPEC_DTYPE_F32
    return _capi.verify_workspace_bytes(B, G, V, code)


def _workspace(device, stream_handle, nbytes):
    key = (device.index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        # zero-filled once; every completed call leaves it zero-filled
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def verify(target_logits, draft_probs, draft_tokens, uniforms, temperature, verify_len=None, *,
           out_accepted=None, out_tokens=None, diag=False, workspace=None, row_pass_event=None, draft_logits=None):
    """Verify a batch of draft blocks on the current stream of target_logits' device.

    target_logits [B, G+1, V] bf16/fp32; draft_probs [B, G, V] fp32 (None at T=0);
    draft_tokens [B, G] int32; uniforms [B, G+1] fp32 (None at T=0);
    verify_len [B] int32 or None.  Returns (accepted [B], tokens [B, G+1]) int32,
    plus a dict of diagnostics when diag=True.  Asynchronous like any kernel.
    row_pass_event: a torch.cuda.Event, or a raw hipEvent_t handle (int), that
    the library records right after the launch of the row pass (for timing
    that kernel alone).
    draft_logits: [B, G, V] of the target's dtype in place of draft_probs
    (which must then be None): q = softmax(draft_logits / temperature).
    """
    z = target_logits
    if not isinstance(z, torch.Tensor) or z.dim() != 3:
        raise ValueError("target_logits must be a [B, G+1, V] tensor")
    dev = z.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be on a GPU")
    B, G1, V = z.shape
    G = G1 - 1
    code = _dtype_code(z)
    T = float(temperature)
    i32, f32 = torch.int32, torch.float32
    if out_accepted is None:
        out_accepted = torch.empty(B, dtype=i32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(B, G1, dtype=i32, device=dev)
    if draft_logits is not None and draft_probs is not None:
        raise ValueError("pass draft_probs or draft_logits, not both")
    for t, shape, name in ((draft_probs, (B, G, V), "draft_probs"), (draft_logits, (B, G, V), "draft_logits"),
                           (draft_tokens, (B, G), "draft_tokens"),
                           (uniforms, (B, G1), "uniforms"), (verify_len, (B,), "verify_len"),
                           (out_accepted, (B,), "out_accepted"), (out_tokens, (B, G1), "out_tokens")):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    stream = torch.cuda.current_stream(dev).cuda_stream
    d = None
    dg = None
    ev = 0
    if isinstance(row_pass_event, int):
        ev = row_pass_event
    elif row_pass_event is not None:
        if row_pass_event.cuda_event == 0:          # torch creates the event on its first record
            row_pass_event.record(torch.cuda.current_stream(dev))
        ev = row_pass_event.cuda_event
    if diag:
        dg = {"target_lse": torch.empty(B, G1, dtype=f32, device=dev),
              "p_draft": torch.empty(B, G, dtype=f32, device=dev),
              "q_draft": torch.empty(B, G, dtype=f32, device=dev),
              "resid_mass": torch.empty(B, dtype=f32, device=dev)}
        d = _capi.DiagT(*(dg[k].data_ptr() for k in ("target_lse", "p_draft", "q_draft", "resid_mass")), ev)
    elif ev:
        d = _capi.DiagT(0, 0, 0, 0, ev)
    nbytes = _capi.verify_workspace_bytes(B, G, V, code)
    ws = workspace if workspace is not None else _workspace(dev, stream, nbytes)
    if draft_logits is not None:
        st = _capi.spec_verify_logits(
            z.data_ptr(), code, _ptr(draft_logits, z.dtype, dev, "draft_logits"),
            _ptr(draft_tokens, i32, dev, "draft_tokens"), _ptr(uniforms, f32, dev, "uniforms"),
            _ptr(verify_len, i32, dev, "verify_len"), B, G, V, T,
            _ptr(out_accepted, i32, dev, "out_accepted"), _ptr(out_tokens, i32, dev, "out_tokens"), d,
            ws.data_ptr(), ws.numel() * ws.element_size(), stream)
        where = "spec_verify_logits"
    else:
        st = _capi.spec_verify(
            z.data_ptr(), code, _ptr(draft_probs, f32, dev, "draft_probs"),
            _ptr(draft_tokens, i32, dev, "draft_tokens"), _ptr(uniforms, f32, dev, "uniforms"),
            _ptr(verify_len, i32, dev, "verify_len"), B, G, V, T,
            _ptr(out_accepted, i32, dev, "out_accepted"), _ptr(out_tokens, i32, dev, "out_tokens"), d,
            ws.data_ptr(), ws.numel() * ws.element_size(), stream)
        where = "spec_verify"
    if st != _capi.SPEC_OK:
        raise SpecError(st, where)
    if diag:
        return out_accepted, out_tokens, dg
    return out_accepted, out_tokens


def schedule(confidence, cost_table, token_budget, eps=0.0, *, out_verify_len=None, out_total=None,
             out_expected=None, calib_temps=None):
    """Choose per-request verify lengths.  Returns (verify_len [B], T [1], tau [1]) device tensors.
    calib_temps: a host sequence of G temperatures (spec_schedule_calibrated), or None (spec_schedule)."""
    c = confidence
    if not isinstance(c, torch.Tensor) or c.dim() != 2:
        raise ValueError("confidence must be a [B, G] tensor")
    dev = c.device
    B, G = c.shape
    i32, f32 = torch.int32, torch.float32
    if cost_table.dim() != 1:
        raise ValueError("cost_table must be 1-D")
    L = cost_table.shape[0]
    if out_verify_len is None:
        out_verify_len = torch.empty(B, dtype=i32, device=dev)
    if out_total is None:
        out_total = torch.empty(1, dtype=i32, device=dev)
    if out_expected is None:
        out_expected = torch.empty(1, dtype=f32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(cost_table, f32, dev, "cost_table"), L, B, G, int(token_budget), float(eps),
            _ptr(out_verify_len, i32, dev, "out_verify_len"), _ptr(out_total, i32, dev, "out_total"),
            _ptr(out_expected, f32, dev, "out_expected"), 0, 0, stream)
    if calib_temps is None:
        st, where = _capi.spec_schedule(_ptr(c, f32, dev, "confidence"), *args), "spec_schedule"
    else:
        st = _capi.spec_schedule_calibrated(_ptr(c, f32, dev, "confidence"), calib_temps, *args)
        where = "spec_schedule_calibrated"
    if st != _capi.SPEC_OK:
        raise SpecError(st, where)
    return out_verify_len, out_total, out_expected


def verify_packed(packed_logits, row_offsets, draft_probs, draft_tokens, uniforms, temperature, *,
                  out_accepted=None, out_tokens=None, diag=False, workspace=None, row_pass_event=None):
    """Verify over packed target rows: request b's rows are packed_logits[off[b]:off[b+1]].

    packed_logits [rows, V] bf16/fp32; row_offsets [B+1] int32 (device);
    draft_probs [B, G, V]; draft_tokens [B, G]; uniforms [B, G+1] as for verify().
    Returns what verify() returns.
    """
    z = packed_logits
    if not isinstance(z, torch.Tensor) or z.dim() != 2:
        raise ValueError("packed_logits must be a [rows, V] tensor")
    dev = z.device
    if dev.type != "cuda":
        raise ValueError("packed_logits must be on a GPU")
    rows, V = z.shape
    if not isinstance(draft_tokens, torch.Tensor) or draft_tokens.dim() != 2:
        raise ValueError("draft_tokens must be a [B, G] tensor")
    B, G = draft_tokens.shape
    G1 = G + 1
    code = _dtype_code(z)
    T = float(temperature)
    i32, f32 = torch.int32, torch.float32
    if out_accepted is None:
        out_accepted = torch.empty(B, dtype=i32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(B, G1, dtype=i32, device=dev)
    for t, shape, name in ((draft_probs, (B, G, V), "draft_probs"), (uniforms, (B, G1), "uniforms"),
                           (row_offsets, (B + 1,), "row_offsets"), (out_accepted, (B,), "out_accepted"),
                           (out_tokens, (B, G1), "out_tokens")):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    stream = torch.cuda.current_stream(dev).cuda_stream
    d, dg, ev = None, None, 0
    if isinstance(row_pass_event, int):
        ev = row_pass_event
    elif row_pass_event is not None:
        if row_pass_event.cuda_event == 0:
            row_pass_event.record(torch.cuda.current_stream(dev))
        ev = row_pass_event.cuda_event
    if diag:
        dg = {"target_lse": torch.empty(B, G1, dtype=f32, device=dev),
              "p_draft": torch.empty(B, G, dtype=f32, device=dev),
              "q_draft": torch.empty(B, G, dtype=f32, device=dev),
              "resid_mass": torch.empty(B, dtype=f32, device=dev)}
        d = _capi.DiagT(*(dg[k].data_ptr() for k in ("target_lse", "p_draft", "q_draft", "resid_mass")), ev)
    elif ev:
        d = _capi.DiagT(0, 0, 0, 0, ev)
    nbytes = _capi.verify_workspace_bytes(B, G, V, code)
    ws = workspace if workspace is not None else _workspace(dev, stream, nbytes)
    st = _capi.spec_verify_packed(
        z.data_ptr(), code, rows, _ptr(row_offsets, i32, dev, "row_offsets"),
        _ptr(draft_probs, f32, dev, "draft_probs"), _ptr(draft_tokens, i32, dev, "draft_tokens"),
        _ptr(uniforms, f32, dev, "uniforms"), B, G, V, T,
        _ptr(out_accepted, i32, dev, "out_accepted"), _ptr(out_tokens, i32, dev, "out_tokens"), d,
        ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_verify_packed")
    if diag:
        return out_accepted, out_tokens, dg
    return out_accepted, out_tokens


def dcut(confidence, ratios, ratio_cost, *, out_verify_len=None, out_row_offsets=None, out_ratio=None,
         out_rows=None, out_utility=None, utility=True, calib_temps=None):
    """Ratio-budgeted depth.  ratios, ratio_cost: host sequences of floats (the
    profiled cost of each ratio at this batch size).  Returns device tensors
    (verify_len [B], row_offsets [B+1], ratio_index [1], total_rows [1],
    utility [R] float64 or None).
    """
    c = confidence
    if not isinstance(c, torch.Tensor) or c.dim() != 2:
        raise ValueError("confidence must be a [B, G] tensor")
    dev = c.device
    B, G = c.shape
    ratios = [float(r) for r in ratios]
    ratio_cost = [float(v) for v in ratio_cost]
    if len(ratios) != len(ratio_cost):
        raise ValueError("ratios and ratio_cost differ in length")
    R = len(ratios)
    i32 = torch.int32
    if out_verify_len is None:
        out_verify_len = torch.empty(B, dtype=i32, device=dev)
    if out_row_offsets is None:
        out_row_offsets = torch.empty(B + 1, dtype=i32, device=dev)
    if out_ratio is None:
        out_ratio = torch.empty(1, dtype=i32, device=dev)
    if out_rows is None:
        out_rows = torch.empty(1, dtype=i32, device=dev)
    if out_utility is None and utility:
        out_utility = torch.empty(max(R, 1), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _capi.spec_dcut(_ptr(c, torch.float32, dev, "confidence"), B, G, ratios, ratio_cost,
                         _ptr(out_verify_len, i32, dev, "out_verify_len"),
                         _ptr(out_row_offsets, i32, dev, "out_row_offsets"), _ptr(out_ratio, i32, dev, "out_ratio"),
                         _ptr(out_rows, i32, dev, "out_rows"),
                         _ptr(out_utility, torch.float64, dev, "out_utility") if out_utility is not None else 0,
                         stream, calib=calib_temps)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_dcut")
    return out_verify_len, out_row_offsets, out_ratio, out_rows, out_utility


def acceptance(target_logits, draft, temperature, verify_len=None, *, draft_is_logits=False, out_alpha=None):
    """Per-position acceptance overlap alpha[b, k] = sum_v min(p_k, q_k) (NaN where untested).

    target_logits [B, G+1, V] bf16/fp32; draft [B, G, V]: fp32 probabilities, or
    logits of the target's dtype when draft_is_logits (softmax at temperature).
    """
    z = target_logits
    if not isinstance(z, torch.Tensor) or z.dim() != 3:
        raise ValueError("target_logits must be a [B, G+1, V] tensor")
    dev = z.device
    B, G1, V = z.shape
    G = G1 - 1
    code = _dtype_code(z)
    ddt = z.dtype if draft_is_logits else torch.float32
    if tuple(draft.shape) != (B, G, V):
        raise ValueError(f"draft has shape {tuple(draft.shape)}, expected {(B, G, V)}")
    if out_alpha is None:
        out_alpha = torch.empty(B, G, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _capi.spec_acceptance(z.data_ptr(), code, _ptr(draft, ddt, dev, "draft"),
                               _capi.SPEC_DRAFT_LOGITS if draft_is_logits else _capi.SPEC_DRAFT_PROBS,
                               _ptr(verify_len, torch.int32, dev, "verify_len"), B, G, V, float(temperature),
                               _ptr(out_alpha, torch.float32, dev, "out_alpha"), stream)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_acceptance")
    return out_alpha


def schedule_static(confidence, B=None, G=None, *, fixed_len=None, threshold=None, calib_temps=None,
                    row_offsets=True, out_verify_len=None, out_total=None, out_row_offsets=None):
    """Static scheduler: fixed_len (every request min(L, G) drafts) or threshold
    (leading drafts whose confidence exceeds it).  Returns device tensors
    (verify_len [B], total [1], row_offsets [B+1] or None)."""
    if (fixed_len is None) == (threshold is None):
        raise ValueError("give exactly one of fixed_len and threshold")
    if confidence is not None:
        dev = confidence.device
        B, G = confidence.shape
    else:
        dev = torch.device("cuda", torch.cuda.current_device())
    i32 = torch.int32
    out_len = out_verify_len if out_verify_len is not None else torch.empty(B, dtype=i32, device=dev)
    out_T = out_total if out_total is not None else torch.empty(1, dtype=i32, device=dev)
    out_off = out_row_offsets
    if out_off is None and row_offsets:
        out_off = torch.empty(B + 1, dtype=i32, device=dev)
    mode = _capi.SPEC_STATIC_FIXED if fixed_len is not None else _capi.SPEC_STATIC_THRESHOLD
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _capi.spec_schedule_static(_ptr(confidence, torch.float32, dev, "confidence"), B, G, mode,
                                    int(fixed_len or 0), float(threshold or 0.0), calib_temps,
                                    out_len.data_ptr(), out_T.data_ptr(),
                                    out_off.data_ptr() if out_off is not None else 0, stream)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_schedule_static")
    return out_len, out_T, out_off


def sts_fit(confidence, acc_len, temps, bins=15):
    """Sequential Temperature Scaling fit.  confidence [N, G] fp32, acc_len [N]
    int32 (device); temps: host sequence (the grid).  Returns out_temps [G] fp32."""
    dev = confidence.device
    N, G = confidence.shape
    temps = [float(t) for t in temps]
    nbytes = _capi.sts_fit_workspace_bytes(N, G, len(temps), bins)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(G, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _capi.spec_sts_fit(_ptr(confidence, torch.float32, dev, "confidence"),
                            _ptr(acc_len, torch.int32, dev, "acc_len"), N, G, temps, bins, out.data_ptr(),
                            ws.data_ptr(), ws.numel(), stream)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_sts_fit")
    return out


def verify_tree(target_logits, parents, node_tokens, *, workspace=None):
    """Greedy verification of a candidate tree per request.

    target_logits [B, M, V] bf16/fp32 (row i: the target after the path to node i);
    parents, node_tokens [B, M] int32 (entry 0 is the root).  Returns device
    tensors (accepted [B], tokens [B, M], path [B, M]).
    """
    z = target_logits
    if not isinstance(z, torch.Tensor) or z.dim() != 3:
        raise ValueError("target_logits must be a [B, M, V] tensor")
    dev = z.device
    B, M, V = z.shape
    code = _dtype_code(z)
    i32 = torch.int32
    for t, name in ((parents, "parents"), (node_tokens, "node_tokens")):
        if t is not None and tuple(t.shape) != (B, M):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, M)}")
    acc = torch.empty(B, dtype=i32, device=dev)
    tok = torch.empty(B, M, dtype=i32, device=dev)
    path = torch.empty(B, M, dtype=i32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = _capi.verify_workspace_bytes(B, M - 1, V, code)
    ws = workspace if workspace is not None else _workspace(dev, stream, nbytes)
    st = _capi.spec_verify_tree(z.data_ptr(), code, _ptr(parents, i32, dev, "parents"),
                                _ptr(node_tokens, i32, dev, "node_tokens"), B, M, V, acc.data_ptr(), tok.data_ptr(),
                                path.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if st != _capi.SPEC_OK:
        raise SpecError(st, "spec_verify_tree")
    return acc, tok, path
