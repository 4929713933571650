"""Python binding of libbdr: the block-draft readout hot path on MI355X (gfx950).

Each function marshals torch device tensors into the C ABI of ``include/bdr.h``
(``data_ptr()`` and the current HIP stream) and raises ``BdrError`` on a non-zero
return.  Every step of the path runs in the HIP kernels of libbdr; there is no
other implementation behind these names.  Output tensors and workspaces that are
not supplied are allocated with torch on the input's device; a workspace passed
in must have been zero-filled once (``torch.zeros``) and may be reused.
"""
from __future__ import annotations

import ctypes as C
import math
from typing import Dict, Optional, Sequence

import torch

from . import _abi
from ._abi import BdrError, BDR_BF16, BDR_BF16_PACKED, BDR_F32  # noqa: F401

__all__ = [
    "dflash_fuse_fc", "dspark_lm_head", "dspark_markov_argmax", "dspark_draft_block",
    "dspark_draft_block_noalloc", "dflash_fuse_fc_lm_head",
    "spec_verify_greedy", "dspark_gumbel_noise", "dspark_markov_sample", "spec_verify_sample",
    "spec_commit", "dflash_fuse_fc_rows", "dflash_fuse_fc_fp8", "dspark_lm_head_fp8",
    "dflash_hc_average", "dflash_fuse_fc_rows_fp8", "PackedWeight", "pack_weight",
    "workspace_bytes", "lib", "BdrError", "set_markov_poll_timeout_us",
    "set_markov_forced_time_out", "MARKOV_TIMED_OUT",
]


def lib():
    """The loaded libbdr (raises ImportError when it has not been built)."""
    return _abi.load()


class PackedWeight:
    """A bf16 weight [rows, cols] in the packed layout of bdr_pack_weight (the
    bytes in ``data``).  dflash_fuse_fc, dflash_fuse_fc_rows, dspark_lm_head,
    dflash_fuse_fc_lm_head, dspark_draft_block and dspark_draft_block_noalloc
    take it in place of the bf16 tensor; their results are those of the
    row-major weight."""

    dtype = torch.bfloat16
    is_cuda = True

    def __init__(self, data: torch.Tensor, rows: int, cols: int):
        self.data = data
        self.shape = torch.Size((rows, cols))
        self.device = data.device

    def is_contiguous(self) -> bool:
        return True

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def pack_weight(w: torch.Tensor) -> PackedWeight:
    """The packed copy of a bf16 weight [rows, cols] (cols % 8 == 0), written on
    w's device and current stream."""
    L = lib()
    _dev(w, "w")
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("pack_weight takes a bf16 [rows, cols] tensor")
    rows, cols = w.shape
    n = L.bdr_packed_weight_bytes(rows, cols)
    if n == 0:
        raise BdrError("bdr_pack_weight", _abi.BDR_EUNSUPPORTED,
                       f"weight [{rows}, {cols}] cannot be packed (cols % 8 == 0 and a packed "
                       "copy under 2^31 bytes are required)")
    data = torch.empty(n, dtype=torch.uint8, device=w.device)
    _abi.check("bdr_pack_weight", L.bdr_pack_weight(_ptr(w), rows, cols, _ptr(data),
                                                    _stream(w.device)))
    return PackedWeight(data, rows, cols)


def _dt(t) -> int:
    if isinstance(t, PackedWeight):
        return BDR_BF16_PACKED
    if t.dtype == torch.bfloat16:
        return BDR_BF16
    if t.dtype == torch.float32:
        return BDR_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    # zero-filled: the library's counters start at zero and are left at zero
    return torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    al = (p + 255) & ~255
    return C.c_void_p(al), ws.numel() * ws.element_size() - (al - p)


def workspace_bytes(kind: str, **kw) -> int:
    """Workspace size the library needs for ``kind`` in {fc, markov, draft, verify}."""
    L = lib()
    if kind == "fc":
        return L.dflash_fuse_fc_workspace_bytes(kw["rows"], kw["hidden"], kw["n_taps"], kw["dtype"])
    if kind == "fc_fp8":
        return L.dflash_fuse_fc_fp8_workspace_bytes(kw["rows"], kw["hidden"], kw["n_taps"])
    if kind == "markov":
        return L.dspark_markov_workspace_bytes(kw["batch"], kw["k"])
    if kind == "draft":
        return L.dspark_draft_workspace_bytes(kw["batch"], kw["k"], kw["vocab"],
                                              int(kw.get("logits_in_workspace", True)))
    if kind == "verify":
        return L.spec_verify_workspace_bytes(kw["batch"], kw["k"], kw["vocab"])
    if kind == "markov_sample":
        return L.dspark_markov_sample_workspace_bytes(kw["batch"], kw["k"], kw["vocab"])
    if kind == "verify_sample":
        return L.spec_verify_sample_workspace_bytes(kw["batch"], kw["k"], kw["vocab"])
    raise ValueError(kind)


# ----------------------------------------------------------------------------- S1
def dflash_fuse_fc(taps: Sequence[torch.Tensor], fc_w: torch.Tensor,
                   out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[rows, H] = concat(taps) @ fc_w^T  (taps: T tensors [rows, H]; fc_w [H, T*H])."""
    L = lib()
    T = len(taps)
    rows, H = taps[0].shape
    for i, t in enumerate(taps):
        _dev(t, f"taps[{i}]")
        if t.shape != (rows, H) or t.dtype != fc_w.dtype:
            raise ValueError("taps must all be [rows, H] with fc_w's dtype")
    _dev(fc_w, "fc_w")
    if tuple(fc_w.shape) != (H, T * H):
        raise ValueError(f"fc_w must be [{H}, {T * H}]")
    dt = _dt(fc_w)
    if out is None:
        out = torch.empty((rows, H), dtype=fc_w.dtype, device=fc_w.device)
    _dev(out, "out")
    need = L.dflash_fuse_fc_workspace_bytes(rows, H, T, dt)
    ws = _workspace(need, fc_w.device, workspace)
    wp, wn = _ws_ptr(ws)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    _abi.check("dflash_fuse_fc", L.dflash_fuse_fc(arr, T, rows, H, dt, _ptr(fc_w), _ptr(out), wp,
                                                  wn, _stream(fc_w.device)))
    return out


# ----------------------------------------------------------------------------- S2
def dspark_lm_head(hidden: torch.Tensor, lm_head_w: torch.Tensor,
                   logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 logits [..., V] = hidden[..., H] @ lm_head_w[V, H]^T."""
    L = lib()
    _dev(hidden, "hidden")
    _dev(lm_head_w, "lm_head_w")
    V, H = lm_head_w.shape
    if hidden.shape[-1] != H or hidden.dtype != lm_head_w.dtype:
        raise ValueError("hidden must be [..., H] with lm_head_w's dtype")
    rows = hidden.numel() // H
    if logits is None:
        logits = torch.empty((*hidden.shape[:-1], V), dtype=torch.float32, device=hidden.device)
    _dev(logits, "logits")
    _abi.check("dspark_lm_head", L.dspark_lm_head(_ptr(hidden), rows, H, V, _dt(lm_head_w),
                                                  _ptr(lm_head_w), _ptr(logits),
                                                  _stream(hidden.device)))
    return logits


# ----------------------------------------------------------------------------- S1 input: hc average
def dflash_hc_average(captured: Sequence[torch.Tensor],
                      out: Optional[Sequence[torch.Tensor]] = None):
    """taps[t][rows, H] = mean over s of captured[t][s, rows, H] (hyper-connection
    streams).  Each captured tensor is a [hc, rows, H] view with a unit last
    stride (any stream/row strides, the same for every tap)."""
    L = lib()
    T = len(captured)
    c0 = captured[0]
    if c0.dim() != 3:
        raise ValueError("captured tensors must be [hc, rows, H]")
    hc, rows, H = c0.shape
    ss, rs, es = c0.stride()
    for i, c in enumerate(captured):
        if not c.is_cuda:
            raise ValueError(f"captured[{i}] must be a device tensor")
        if c.shape != c0.shape or c.stride() != c0.stride() or c.dtype != c0.dtype:
            raise ValueError("captured tensors must share shape, strides and dtype")
    if es != 1:
        raise ValueError("captured tensors need a unit stride along H")
    dt = _dt(c0)
    if out is None:
        out = [torch.empty((rows, H), dtype=c0.dtype, device=c0.device) for _ in range(T)]
    for i, o in enumerate(out):
        _dev(o, f"out[{i}]")
    src = (C.c_void_p * T)(*[c.data_ptr() for c in captured])
    dst = (C.c_void_p * T)(*[o.data_ptr() for o in out])
    _abi.check("dflash_hc_average", L.dflash_hc_average(src, T, hc, rows, H, ss, rs, dt, dst,
                                                        _stream(c0.device)))
    return list(out)


# ----------------------------------------------------------------------------- S1/S2, fp8 weights
def _fp8_weight(q: torch.Tensor, scale: torch.Tensor, qname: str, sname: str):
    _dev(q, qname)
    _dev(scale, sname)
    if q.dtype != torch.uint8 or q.dim() != 2:
        raise ValueError(f"{qname} must be a 2-D uint8 tensor of E4M3 codes")
    if scale.dtype != torch.float32 or tuple(scale.shape) != (q.shape[0],):
        raise ValueError(f"{sname} must be fp32 [{q.shape[0]}]")


def dflash_fuse_fc_fp8(taps: Sequence[torch.Tensor], fc_q: torch.Tensor, fc_scale: torch.Tensor,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 out[rows, H] = fc_scale * (concat(taps) @ e4m3(fc_q)^T)  (taps bf16 [rows, H])."""
    L = lib()
    T = len(taps)
    rows, H = taps[0].shape
    for i, t in enumerate(taps):
        _dev(t, f"taps[{i}]")
        if t.shape != (rows, H) or t.dtype != torch.bfloat16:
            raise ValueError("taps must all be bf16 [rows, H]")
    _fp8_weight(fc_q, fc_scale, "fc_q", "fc_scale")
    if tuple(fc_q.shape) != (H, T * H):
        raise ValueError(f"fc_q must be [{H}, {T * H}]")
    if out is None:
        out = torch.empty((rows, H), dtype=torch.bfloat16, device=fc_q.device)
    _dev(out, "out")
    need = L.dflash_fuse_fc_fp8_workspace_bytes(rows, H, T)
    ws = _workspace(need, fc_q.device, workspace)
    wp, wn = _ws_ptr(ws)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    _abi.check("dflash_fuse_fc_fp8", L.dflash_fuse_fc_fp8(arr, T, rows, H, _ptr(fc_q),
                                                          _ptr(fc_scale), _ptr(out), wp, wn,
                                                          _stream(fc_q.device)))
    return out


def dspark_lm_head_fp8(hidden: torch.Tensor, lm_head_q: torch.Tensor, lm_head_scale: torch.Tensor,
                       logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 logits [..., V] = lm_head_scale * (hidden[..., H] @ e4m3(lm_head_q)[V, H]^T)."""
    L = lib()
    _dev(hidden, "hidden")
    _fp8_weight(lm_head_q, lm_head_scale, "lm_head_q", "lm_head_scale")
    V, H = lm_head_q.shape
    if hidden.shape[-1] != H or hidden.dtype != torch.bfloat16:
        raise ValueError("hidden must be bf16 [..., H]")
    rows = hidden.numel() // H
    if logits is None:
        logits = torch.empty((*hidden.shape[:-1], V), dtype=torch.float32, device=hidden.device)
    _dev(logits, "logits")
    _abi.check("dspark_lm_head_fp8", L.dspark_lm_head_fp8(_ptr(hidden), rows, H, V,
                                                          _ptr(lm_head_q), _ptr(lm_head_scale),
                                                          _ptr(logits), _stream(hidden.device)))
    return logits


# ----------------------------------------------------------------------------- S1 + S2
def dflash_fuse_fc_lm_head(taps: Sequence[torch.Tensor], fc_w: torch.Tensor,
                           lm_hidden: torch.Tensor, lm_head_w: torch.Tensor,
                           fc_out: Optional[torch.Tensor] = None,
                           logits: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None):
    """(fc_out [rows, H], logits [..., V] fp32): the drafter fc over the taps and the
    LM head over lm_hidden [..., H] in one call (one launch when both take the
    row-split kernel)."""
    L = lib()
    T = len(taps)
    rows, H = taps[0].shape
    for i, t in enumerate(taps):
        _dev(t, f"taps[{i}]")
        if t.shape != (rows, H) or t.dtype != fc_w.dtype:
            raise ValueError("taps must all be [rows, H] with fc_w's dtype")
    _dev(fc_w, "fc_w")
    _dev(lm_hidden, "lm_hidden")
    _dev(lm_head_w, "lm_head_w")
    if tuple(fc_w.shape) != (H, T * H):
        raise ValueError(f"fc_w must be [{H}, {T * H}]")
    V = lm_head_w.shape[0]
    if lm_head_w.shape[1] != H or lm_hidden.shape[-1] != H:
        raise ValueError("lm_head_w must be [V, H] and lm_hidden [..., H]")
    if lm_hidden.dtype != fc_w.dtype or lm_head_w.dtype != fc_w.dtype:
        raise ValueError("all weights and activations must share one dtype")
    if isinstance(fc_w, PackedWeight) != isinstance(lm_head_w, PackedWeight):
        raise ValueError("fc_w and lm_head_w must both be packed or both be tensors")
    dt = _dt(fc_w)
    lm_rows = lm_hidden.numel() // H
    dev = fc_w.device
    if fc_out is None:
        fc_out = torch.empty((rows, H), dtype=fc_w.dtype, device=dev)
    if logits is None:
        logits = torch.empty((*lm_hidden.shape[:-1], V), dtype=torch.float32, device=dev)
    _dev(fc_out, "fc_out")
    _dev(logits, "logits")
    need = L.dflash_fuse_fc_lm_head_workspace_bytes(rows, H, T, lm_rows, V, dt)
    ws = _workspace(need, dev, workspace)
    wp, wn = _ws_ptr(ws)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    _abi.check("dflash_fuse_fc_lm_head",
               L.dflash_fuse_fc_lm_head(arr, T, rows, H, dt, _ptr(fc_w), _ptr(fc_out),
                                        _ptr(lm_hidden), lm_rows, V, _ptr(lm_head_w),
                                        _ptr(logits), wp, wn, _stream(dev)))
    return fc_out, logits


# ----------------------------------------------------------------------------- S3
# BdrError code of a Markov call whose status word reports a wait that gave up
MARKOV_TIMED_OUT = -5


def _status_in(status: Optional[torch.Tensor], check: bool, device) -> Optional[torch.Tensor]:
    if status is not None:
        _dev(status, "status")
        if status.dtype != torch.int32 or status.numel() < 1:
            raise ValueError("status must be an int32 device tensor")
        return status
    return torch.empty(1, dtype=torch.int32, device=device) if check else None


def _status_out(fn: str, status: Optional[torch.Tensor], check: bool) -> None:
    """With check: wait for the call and raise if one of its bounded waits gave up."""
    if check and status is not None and int(status.view(-1)[0].item()) != 0:
        raise BdrError(fn, MARKOV_TIMED_OUT,
                       "a bounded wait of the persistent Markov chain gave up (its workgroups "
                       "were not all resident, e.g. beside another chain launch); the draft "
                       "is invalid")


def set_markov_poll_timeout_us(us: float) -> None:
    """Process-wide limit of the Markov chain's bounded waits for later launches
    (negative: the default)."""
    lib().bdr_set_markov_poll_timeout_us(float(us))


def set_markov_forced_time_out(on: bool) -> None:
    """Process-wide error-path hook for later launches: every bounded wait of
    the chain disregards what it reads and gives up once its limit passes."""
    lib().bdr_set_markov_forced_time_out(1 if on else 0)


def set_row_split_override(ring: int = 0, workgroups: int = 0, ksplit: int = 0) -> None:
    """Process-wide plan override of the row-split GEMM (0 = the planner's
    choice): the bf16 ring depth, the row ranges and the K splits."""
    _abi.check("bdr_set_row_split_override",
               lib().bdr_set_row_split_override(int(ring), int(workgroups), int(ksplit)))


def _markov_args(w1, w2, dt_ref):
    if w1 is None and w2 is None:
        return None, None, 0
    _dev(w1, "markov_w1")
    _dev(w2, "markov_w2")
    if w1.shape != w2.shape or w1.dtype != w2.dtype:
        raise ValueError("markov_w1 and markov_w2 must both be [V, r] of one dtype")
    return w1, w2, int(w1.shape[1])


def dspark_markov_argmax(logits: torch.Tensor, markov_w1: Optional[torch.Tensor],
                         markov_w2: Optional[torch.Tensor], prev_token: torch.Tensor,
                         draft_tokens: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None,
                         check: bool = True) -> torch.Tensor:
    """Draft tokens [B, k] (int32) from fp32 logits [B, k, V] and the Markov head.

    ``status`` (int32 device tensor) receives the call's status word; with
    ``check`` (default) the call is waited for and BdrError is raised when one
    of the chain's bounded waits gave up."""
    L = lib()
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 3:
        raise ValueError("logits must be fp32 [B, k, V]")
    B, k, V = logits.shape
    w1, w2, r = _markov_args(markov_w1, markov_w2, logits)
    wdt = _dt(w1) if w1 is not None else BDR_F32
    _dev(prev_token, "prev_token")
    if prev_token.dtype != torch.int32 or prev_token.numel() != B:
        raise ValueError("prev_token must be int32 [B]")
    if draft_tokens is None:
        draft_tokens = torch.empty((B, k), dtype=torch.int32, device=logits.device)
    _dev(draft_tokens, "draft_tokens")
    ws = _workspace(L.dspark_markov_workspace_bytes(B, k), logits.device, workspace)
    wp, wn = _ws_ptr(ws)
    st = _status_in(status, check, logits.device)
    _abi.check("dspark_markov_argmax",
               L.dspark_markov_argmax(_ptr(logits), B, k, V, wdt, _ptr(w1), _ptr(w2), r,
                                      _ptr(prev_token), _ptr(draft_tokens), _ptr(st), wp, wn,
                                      _stream(logits.device)))
    _status_out("dspark_markov_argmax", st, check and B > 0)
    return draft_tokens


# ----------------------------------------------------------------------------- S2+S3
def dspark_draft_block(draft_hidden: torch.Tensor, lm_head_w: torch.Tensor,
                       markov_w1: Optional[torch.Tensor], markov_w2: Optional[torch.Tensor],
                       prev_token: torch.Tensor, draft_tokens: Optional[torch.Tensor] = None,
                       logits_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None,
                       check: bool = True) -> torch.Tensor:
    """Draft one block: LM head over draft_hidden [B, k, H], then the Markov argmax chain
    (``status`` / ``check`` as in dspark_markov_argmax)."""
    L = lib()
    _dev(draft_hidden, "draft_hidden")
    _dev(lm_head_w, "lm_head_w")
    B, k, H = draft_hidden.shape
    V = lm_head_w.shape[0]
    if lm_head_w.shape[1] != H or draft_hidden.dtype != lm_head_w.dtype:
        raise ValueError("lm_head_w must be [V, H] with draft_hidden's dtype")
    w1, w2, r = _markov_args(markov_w1, markov_w2, lm_head_w)
    if w1 is not None and w1.dtype != lm_head_w.dtype:
        raise ValueError("Markov weights must share the LM head's dtype")
    _dev(prev_token, "prev_token")
    if prev_token.dtype != torch.int32 or prev_token.numel() != B:
        raise ValueError("prev_token must be int32 [B]")
    if draft_tokens is None:
        draft_tokens = torch.empty((B, k), dtype=torch.int32, device=draft_hidden.device)
    _dev(draft_tokens, "draft_tokens")
    if logits_out is not None:
        _dev(logits_out, "logits_out")
    need = L.dspark_draft_workspace_bytes(B, k, V, int(logits_out is None))
    ws = _workspace(need, draft_hidden.device, workspace)
    wp, wn = _ws_ptr(ws)
    st = _status_in(status, check, draft_hidden.device)
    _abi.check("dspark_draft_block",
               L.dspark_draft_block(_ptr(draft_hidden), B, k, H, V, _dt(lm_head_w),
                                    _ptr(lm_head_w), _ptr(w1), _ptr(w2), r, _ptr(prev_token),
                                    _ptr(draft_tokens), _ptr(logits_out), _ptr(st), wp, wn,
                                    _stream(draft_hidden.device)))
    _status_out("dspark_draft_block", st, check and B > 0)
    return draft_tokens


def dspark_draft_block_noalloc(draft_hidden: torch.Tensor, lm_head_w: torch.Tensor,
                               markov_w1: Optional[torch.Tensor], markov_w2: Optional[torch.Tensor],
                               prev_token: torch.Tensor, draft_tokens: Optional[torch.Tensor] = None,
                               logits_out: Optional[torch.Tensor] = None,
                               status: Optional[torch.Tensor] = None,
                               check: bool = True) -> torch.Tensor:
    """dspark_draft_block with no workspace (the library's static per-device
    scratch; batch * k <= 256): for callers that cannot allocate inside the
    call.  Outputs not supplied are allocated here, before the call."""
    L = lib()
    _dev(draft_hidden, "draft_hidden")
    _dev(lm_head_w, "lm_head_w")
    B, k, H = draft_hidden.shape
    V = lm_head_w.shape[0]
    if lm_head_w.shape[1] != H or draft_hidden.dtype != lm_head_w.dtype:
        raise ValueError("lm_head_w must be [V, H] with draft_hidden's dtype")
    w1, w2, r = _markov_args(markov_w1, markov_w2, lm_head_w)
    if w1 is not None and w1.dtype != lm_head_w.dtype:
        raise ValueError("Markov weights must share the LM head's dtype")
    _dev(prev_token, "prev_token")
    if prev_token.dtype != torch.int32 or prev_token.numel() != B:
        raise ValueError("prev_token must be int32 [B]")
    dev = draft_hidden.device
    if draft_tokens is None:
        draft_tokens = torch.empty((B, k), dtype=torch.int32, device=dev)
    if logits_out is None:
        logits_out = torch.empty((B, k, V), dtype=torch.float32, device=dev)
    _dev(draft_tokens, "draft_tokens")
    _dev(logits_out, "logits_out")
    if logits_out.dtype != torch.float32 or tuple(logits_out.shape) != (B, k, V):
        raise ValueError("logits_out must be fp32 [B, k, V]")
    st = _status_in(status, check, dev)
    _abi.check("dspark_draft_block_noalloc",
               L.dspark_draft_block_noalloc(_ptr(draft_hidden), B, k, H, V, _dt(lm_head_w),
                                            _ptr(lm_head_w), _ptr(w1), _ptr(w2), r,
                                            _ptr(prev_token), _ptr(draft_tokens),
                                            _ptr(logits_out), _ptr(st), _stream(dev)))
    _status_out("dspark_draft_block_noalloc", st, check and B > 0)
    return draft_tokens


# ----------------------------------------------------------------------------- S4
def spec_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor,
                       confidence: Optional[torch.Tensor] = None,
                       threshold: float = math.nan,
                       accept_counts: Optional[torch.Tensor] = None,
                       proposed_counts: Optional[torch.Tensor] = None,
                       target_argmax: bool = True,
                       out: Optional[Dict[str, torch.Tensor]] = None,
                       workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Greedy verification of draft_tokens [B, k] against target_logits [B, k+1, V].

    Returns block_len, accepted, bonus ([B] int32) and, if requested,
    target_argmax ([B, k+1] int32, -1 past the block).  accept_counts /
    proposed_counts ([k] int64) are accumulated in place when given.
    """
    L = lib()
    _dev(target_logits, "target_logits")
    B, k1, V = target_logits.shape
    k = k1 - 1
    _dev(draft_tokens, "draft_tokens")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, k):
        raise ValueError("draft_tokens must be int32 [B, k]")
    if confidence is not None:
        _dev(confidence, "confidence")
        if confidence.dtype != torch.float32 or tuple(confidence.shape) != (B, k):
            raise ValueError("confidence must be fp32 [B, k]")
    for name, t in (("accept_counts", accept_counts), ("proposed_counts", proposed_counts)):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.int64 or t.numel() != k:
                raise ValueError(f"{name} must be int64 [k]")
    dev = target_logits.device
    res = dict(out) if out is not None else {}
    for name in ("block_len", "accepted", "bonus"):
        if name not in res:
            res[name] = torch.empty(B, dtype=torch.int32, device=dev)
    if target_argmax and "target_argmax" not in res:
        res["target_argmax"] = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    ws = _workspace(L.spec_verify_workspace_bytes(B, k, V), dev, workspace)
    wp, wn = _ws_ptr(ws)
    _abi.check("spec_verify_greedy",
               L.spec_verify_greedy(_ptr(target_logits), _dt(target_logits), B, k, V,
                                    _ptr(draft_tokens), _ptr(confidence), float(threshold),
                                    _ptr(res["block_len"]), _ptr(res["accepted"]),
                                    _ptr(res["bonus"]), _ptr(res.get("target_argmax")),
                                    _ptr(accept_counts), _ptr(proposed_counts), wp, wn,
                                    _stream(dev)))
    return res


# ----------------------------------------------------------------------------- sampling
def dspark_gumbel_noise(batch: int, k: int, vocab: int, seed: int, stream_id: int = 0,
                        out: Optional[torch.Tensor] = None, device="cuda") -> torch.Tensor:
    """Gumbel noise [B, k, V] fp32 of a stream of the sampling path's generator."""
    L = lib()
    if out is None:
        out = torch.empty((batch, k, vocab), dtype=torch.float32, device=device)
    _dev(out, "out")
    if out.dtype != torch.float32 or tuple(out.shape) != (batch, k, vocab):
        raise ValueError("out must be fp32 [B, k, V]")
    _abi.check("dspark_gumbel_noise",
               L.dspark_gumbel_noise(batch, k, vocab, int(seed), int(stream_id), _ptr(out),
                                     _stream(out.device)))
    return out


def dspark_markov_sample(logits: torch.Tensor, markov_w1: Optional[torch.Tensor],
                         markov_w2: Optional[torch.Tensor], prev_token: torch.Tensor,
                         temperature: float, seed: int,
                         draft_tokens: Optional[torch.Tensor] = None,
                         draft_logits: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None,
                         check: bool = True,
                         confidence: Optional[torch.Tensor] = None,
                         threshold: Optional[float] = None):
    """Probabilistic drafting: (draft_tokens [B, k] int32, draft_logits [B, k, V] fp32)
    (``status`` / ``check`` as in dspark_markov_argmax).

    Each position's token is drawn from softmax((logits + Markov bias) / T) and
    becomes the next position's Markov context; draft_logits holds the biased
    logits the tokens were drawn from (the q of rejection sampling).  With
    ``confidence`` [B, k] and ``threshold``, draft_logits is written only at the
    positions j < L_b that spec_verify_sample reads (the rest keep their values).
    """
    L = lib()
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 3:
        raise ValueError("logits must be fp32 [B, k, V]")
    B, k, V = logits.shape
    w1, w2, r = _markov_args(markov_w1, markov_w2, logits)
    wdt = _dt(w1) if w1 is not None else BDR_F32
    _dev(prev_token, "prev_token")
    if prev_token.dtype != torch.int32 or prev_token.numel() != B:
        raise ValueError("prev_token must be int32 [B]")
    if draft_tokens is None:
        draft_tokens = torch.empty((B, k), dtype=torch.int32, device=logits.device)
    if draft_logits is None:
        draft_logits = torch.empty((B, k, V), dtype=torch.float32, device=logits.device)
    _dev(draft_tokens, "draft_tokens")
    _dev(draft_logits, "draft_logits")
    if confidence is not None:
        _dev(confidence, "confidence")
        if confidence.dtype != torch.float32 or confidence.numel() != B * k:
            raise ValueError("confidence must be fp32 [B, k]")
    th = float("nan") if threshold is None else float(threshold)
    ws = _workspace(L.dspark_markov_sample_workspace_bytes(B, k, V), logits.device, workspace)
    wp, wn = _ws_ptr(ws)
    st = _status_in(status, check, logits.device)
    _abi.check("dspark_markov_sample",
               L.dspark_markov_sample(_ptr(logits), B, k, V, wdt, _ptr(w1), _ptr(w2), r,
                                      _ptr(prev_token), float(temperature), int(seed),
                                      _ptr(draft_tokens), _ptr(draft_logits), _ptr(confidence),
                                      th, _ptr(st), wp, wn, _stream(logits.device)))
    _status_out("dspark_markov_sample", st, check and B > 0)
    return draft_tokens, draft_logits


def spec_verify_sample(target_logits: torch.Tensor, draft_tokens: torch.Tensor,
                       draft_logits: torch.Tensor, temperature: float, seed: int,
                       confidence: Optional[torch.Tensor] = None,
                       threshold: float = math.nan,
                       accept_counts: Optional[torch.Tensor] = None,
                       proposed_counts: Optional[torch.Tensor] = None,
                       out: Optional[Dict[str, torch.Tensor]] = None,
                       workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Rejection-sampling verification of draft_tokens [B, k] drawn from
    draft_logits [B, k, V] against target_logits [B, k+1, V].

    Returns block_len, accepted, bonus ([B] int32); accept_counts /
    proposed_counts ([k] int64) are accumulated in place when given.
    """
    L = lib()
    _dev(target_logits, "target_logits")
    B, k1, V = target_logits.shape
    k = k1 - 1
    _dev(draft_tokens, "draft_tokens")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, k):
        raise ValueError("draft_tokens must be int32 [B, k]")
    _dev(draft_logits, "draft_logits")
    if draft_logits.dtype != torch.float32 or tuple(draft_logits.shape) != (B, k, V):
        raise ValueError("draft_logits must be fp32 [B, k, V]")
    if confidence is not None:
        _dev(confidence, "confidence")
        if confidence.dtype != torch.float32 or tuple(confidence.shape) != (B, k):
            raise ValueError("confidence must be fp32 [B, k]")
    for name, t in (("accept_counts", accept_counts), ("proposed_counts", proposed_counts)):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.int64 or t.numel() != k:
                raise ValueError(f"{name} must be int64 [k]")
    dev = target_logits.device
    res = dict(out) if out is not None else {}
    for name in ("block_len", "accepted", "bonus"):
        if name not in res:
            res[name] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(L.spec_verify_sample_workspace_bytes(B, k, V), dev, workspace)
    wp, wn = _ws_ptr(ws)
    _abi.check("spec_verify_sample",
               L.spec_verify_sample(_ptr(target_logits), _dt(target_logits), B, k, V,
                                    _ptr(draft_tokens), _ptr(draft_logits), _ptr(confidence),
                                    float(threshold), float(temperature), int(seed),
                                    _ptr(res["block_len"]), _ptr(res["accepted"]),
                                    _ptr(res["bonus"]), _ptr(accept_counts),
                                    _ptr(proposed_counts), wp, wn, _stream(dev)))
    return res


# ----------------------------------------------------------------------------- loop
def spec_commit(draft_tokens: torch.Tensor, accepted: torch.Tensor, bonus: torch.Tensor,
                block_len: Optional[torch.Tensor] = None,
                out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Commit a verified block: next_prev [B], emitted [B, k+1] (-1 padded),
    draft_list [B, k] (-1 padded), row_index [B*(k+1)] (first row_count valid),
    row_count [1], row_offsets [B+1] -- all int32 on the device."""
    L = lib()
    _dev(draft_tokens, "draft_tokens")
    B, k = draft_tokens.shape
    for name, t in (("accepted", accepted), ("bonus", bonus), ("block_len", block_len)):
        if t is not None:
            _dev(t, name)
            if t.dtype != torch.int32 or t.numel() != B:
                raise ValueError(f"{name} must be int32 [B]")
    dev = draft_tokens.device
    res = dict(out) if out is not None else {}
    shapes = {"next_prev": (B,), "emitted": (B, k + 1), "draft_list": (B, k),
              "row_index": (B * (k + 1),), "row_count": (1,), "row_offsets": (B + 1,)}
    for name, shp in shapes.items():
        if name not in res:
            res[name] = torch.empty(shp, dtype=torch.int32, device=dev)
    _abi.check("spec_commit",
               L.spec_commit(_ptr(draft_tokens), _ptr(accepted), _ptr(bonus), _ptr(block_len), B, k,
                             _ptr(res["next_prev"]), _ptr(res["emitted"]), _ptr(res["draft_list"]),
                             _ptr(res["row_index"]), _ptr(res["row_count"]),
                             _ptr(res["row_offsets"]), _stream(dev)))
    return res


def dflash_fuse_fc_rows(taps: Sequence[torch.Tensor], fc_w: torch.Tensor, row_index: torch.Tensor,
                        row_count: torch.Tensor, max_rows: Optional[int] = None,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[r] = fc(concat(taps)[row_index[r]]) for r < row_count[0], zeros after (out [max_rows, H])."""
    L = lib()
    T = len(taps)
    rows, H = taps[0].shape
    for i, t in enumerate(taps):
        _dev(t, f"taps[{i}]")
        if t.shape != (rows, H) or t.dtype != fc_w.dtype:
            raise ValueError("taps must all be [rows, H] with fc_w's dtype")
    _dev(fc_w, "fc_w")
    _dev(row_index, "row_index")
    _dev(row_count, "row_count")
    if max_rows is None:
        max_rows = row_index.numel()
    dt = _dt(fc_w)
    if out is None:
        out = torch.empty((max_rows, H), dtype=fc_w.dtype, device=fc_w.device)
    _dev(out, "out")
    ws = _workspace(L.dflash_fuse_fc_rows_workspace_bytes(max_rows, H, T, dt), fc_w.device, workspace)
    wp, wn = _ws_ptr(ws)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    _abi.check("dflash_fuse_fc_rows",
               L.dflash_fuse_fc_rows(arr, T, rows, H, dt, _ptr(row_index), _ptr(row_count), max_rows,
                                     _ptr(fc_w), _ptr(out), wp, wn, _stream(fc_w.device)))
    return out


def dflash_fuse_fc_rows_fp8(taps: Sequence[torch.Tensor], fc_q: torch.Tensor, fc_scale: torch.Tensor,
                            row_index: torch.Tensor, row_count: torch.Tensor,
                            max_rows: Optional[int] = None, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dflash_fuse_fc_rows with fp8 weights (E4M3 fc_q [H, T*H] + fp32 fc_scale [H]); bf16 taps/out."""
    L = lib()
    T = len(taps)
    rows, H = taps[0].shape
    for i, t in enumerate(taps):
        _dev(t, f"taps[{i}]")
        if t.shape != (rows, H) or t.dtype != torch.bfloat16:
            raise ValueError("taps must all be bf16 [rows, H]")
    _fp8_weight(fc_q, fc_scale, "fc_q", "fc_scale")
    _dev(row_index, "row_index")
    _dev(row_count, "row_count")
    if max_rows is None:
        max_rows = row_index.numel()
    if out is None:
        out = torch.empty((max_rows, H), dtype=torch.bfloat16, device=fc_q.device)
    _dev(out, "out")
    ws = _workspace(L.dflash_fuse_fc_rows_fp8_workspace_bytes(max_rows, H, T), fc_q.device, workspace)
    wp, wn = _ws_ptr(ws)
    arr = (C.c_void_p * T)(*[t.data_ptr() for t in taps])
    _abi.check("dflash_fuse_fc_rows_fp8",
               L.dflash_fuse_fc_rows_fp8(arr, T, rows, H, _ptr(row_index), _ptr(row_count), max_rows,
                                         _ptr(fc_q), _ptr(fc_scale), _ptr(out), wp, wn,
                                         _stream(fc_q.device)))
    return out

