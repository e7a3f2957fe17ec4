"""Python binding of libdspark, the MI355X verify hot path (argument marshalling only).

Every function here has the name of a C entry point declared in
``include/dspark.h`` and does nothing but check that tensors are on the GPU
with the expected dtype and layout, allocate missing outputs with torch, and
pass raw device pointers plus torch's current HIP stream to the library. All
computation happens in the HIP kernels of ``libdspark.so``; there is no CPU
fallback, and every entry point raises ImportError when the library is not
built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

DSPARK_CUT_THRESHOLD = 0
DSPARK_CUT_BUDGET = 1
DSPARK_CUT_STATIC = 2
DSPARK_CUT_COMBINED = 3
MODES = {"threshold": DSPARK_CUT_THRESHOLD, "budget": DSPARK_CUT_BUDGET,
         "static": DSPARK_CUT_STATIC, "combined": DSPARK_CUT_COMBINED}

_lib = None


class DsparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().dspark_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdspark.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m confidence_scheduled_ragged_amd.build` "
                "or `python -c 'import __graft_entry__; __graft_entry__.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, LL, S = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong,
                          ctypes.c_size_t)
        L.dspark_confidence.argtypes = [P, P, F, P, I, I, I, P, P, P]
        L.dspark_schedule.argtypes = [P, I, I, I, P, LL, P, P]
        L.dspark_compact.argtypes = [P, P, I, I, P, P, P, P, I, P, P]
        L.dspark_accept.argtypes = [P, P, P, P, I, I, I, P, P, P, P, S, P]
        L.dspark_step.argtypes = [P, P, F, P, P, P, I, I, I, I, I, P, LL, P, P, P, P, P, P, P, P,
                                  P, P, S, P]
        L.dspark_cap_accept.argtypes = [P, P, P, I, I, P, P, P, P, P]
        L.dspark_gather_rows.argtypes = [P, P, P, I, I, LL, P, P]
        L.dspark_tier_select.argtypes = [P, I, I, P, I, ctypes.c_int32, P, P, P, P, P]
        L.dspark_cost_cutoff.argtypes = [P, I, P, I, P, P]
        L.dspark_step_ex.argtypes = L.dspark_step.argtypes + [P, P, I, ctypes.c_ulonglong]
        L.dspark_step_status.argtypes = [P, P, P]
        L.dspark_step_noalloc.argtypes = L.dspark_step.argtypes[:22] + [P, P]
        L.dspark_workspace_bytes.argtypes = [I, I, I]
        L.dspark_workspace_bytes.restype = S
        L.dspark_workspace_init.argtypes = [P, S, P]
        L.dspark_status_string.argtypes = [I]
        L.dspark_status_string.restype = ctypes.c_char_p
        for f in (L.dspark_confidence, L.dspark_schedule, L.dspark_compact, L.dspark_accept,
                  L.dspark_step, L.dspark_workspace_init, L.dspark_cap_accept,
                  L.dspark_gather_rows, L.dspark_tier_select, L.dspark_cost_cutoff,
                  L.dspark_step_ex, L.dspark_step_status, L.dspark_step_noalloc):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ok(fn: str, status: int):
    if status != 0:
        raise DsparkError(fn, status)


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def dspark_status_string(status: int) -> str:
    return lib().dspark_status_string(int(status)).decode()


# --------------------------------------------------------------- workspace

def dspark_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return int(lib().dspark_workspace_bytes(B, gamma, V))


def dspark_workspace_init(ws: torch.Tensor) -> None:
    _need(ws, "ws", torch.uint8)
    _ok("dspark_workspace_init",
        lib().dspark_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)))


_WS: Dict[tuple, torch.Tensor] = {}


def _ws_key(device) -> tuple:
    device = torch.device(device)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return (device.type, idx)


def workspace(B: int, gamma: int, V: int, device) -> torch.Tensor:
    """A zero-initialised workspace of the required size, cached per device.
    Calls sharing it must not overlap in time (one stream, or ordered)."""
    device = torch.device(device)
    need = dspark_workspace_bytes(B, gamma, V)
    if need == 0:
        raise ValueError(f"invalid sizes B={B} gamma={gamma} V={V}")
    key = _ws_key(device)
    ws = _WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        dspark_workspace_init(ws)
        _WS[key] = ws
    return ws


# ------------------------------------------------------------- entry points

def dspark_confidence(hidden, w, bias, temps, conf=None, survival=None):
    """Steps 1-2: conf[b,i] and survival[b,i] ([B, gamma] fp32)."""
    B, g, d = hidden.shape
    _need(hidden, "hidden", torch.bfloat16)
    _need(w, "w", torch.bfloat16, (d,))
    _need(temps, "temps", torch.float32, (g,))
    dev = hidden.device
    conf = torch.empty((B, g), dtype=torch.float32, device=dev) if conf is None else conf
    survival = torch.empty((B, g), dtype=torch.float32, device=dev) if survival is None else survival
    _need(conf, "conf", torch.float32, (B, g))
    _need(survival, "survival", torch.float32, (B, g))
    _ok("dspark_confidence", lib().dspark_confidence(
        _ptr(hidden), _ptr(w), float(bias), _ptr(temps), B, g, d, _ptr(conf), _ptr(survival),
        _stream(dev)))
    return conf, survival


def dspark_schedule(survival, mode, cutoff=None, budget=0, lengths=None):
    """Step 3: lengths[B] int32 from the survival curves."""
    B, g = survival.shape
    _need(survival, "survival", torch.float32)
    m = _mode(mode)
    if cutoff is not None:
        _need(cutoff, "cutoff", torch.float32, (B,))
    dev = survival.device
    lengths = torch.empty(B, dtype=torch.int32, device=dev) if lengths is None else lengths
    _need(lengths, "lengths", torch.int32, (B,))
    _ok("dspark_schedule", lib().dspark_schedule(
        _ptr(survival), B, g, m, _ptr(cutoff), int(budget), _ptr(lengths), _stream(dev)))
    return lengths


def dspark_compact(lengths, tokens, logits=None, out=None):
    """Step 4: (cu_seqlens, packed_tokens, packed_src_row, packed_logits or None)."""
    B, g1 = tokens.shape
    g = g1 - 1
    _need(lengths, "lengths", torch.int32, (B,))
    _need(tokens, "tokens", torch.int32)
    dev = tokens.device
    cap = B * g1
    out = out or {}
    cu = out.get("cu_seqlens")
    ptok = out.get("packed_tokens")
    psrc = out.get("packed_src_row")
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev) if cu is None else cu
    ptok = torch.full((cap,), -1, dtype=torch.int32, device=dev) if ptok is None else ptok
    psrc = torch.full((cap,), -1, dtype=torch.int32, device=dev) if psrc is None else psrc
    _need(cu, "cu_seqlens", torch.int32, (B + 1,))
    _need(ptok, "packed_tokens", torch.int32, (cap,))
    _need(psrc, "packed_src_row", torch.int32, (cap,))
    plog = None
    V = 0
    if logits is not None:
        _need(logits, "logits", torch.bfloat16)
        V = logits.shape[-1]
        if logits.numel() != cap * V:
            raise ValueError("logits must hold B*(gamma+1) rows")
        plog = out.get("packed_logits")
        plog = torch.zeros((cap, V), dtype=torch.bfloat16, device=dev) if plog is None else plog
        _need(plog, "packed_logits", torch.bfloat16, (cap, V))
    _ok("dspark_compact", lib().dspark_compact(
        _ptr(lengths), _ptr(tokens), B, g, _ptr(cu), _ptr(ptok), _ptr(psrc), _ptr(logits), V,
        _ptr(plog), _stream(dev)))
    return cu, ptok, psrc, plog


def dspark_accept(logits, packed_src_row, cu_seqlens, tokens, out=None, ws=None):
    """Steps 5-6: (packed_argmax, accepted, bonus). packed_src_row None means
    `logits` is already packed ([B*(gamma+1), V], rows past cu_seqlens[B] unused)."""
    B, g1 = tokens.shape
    g = g1 - 1
    _need(logits, "logits", torch.bfloat16)
    V = logits.shape[-1]
    _need(cu_seqlens, "cu_seqlens", torch.int32, (B + 1,))
    _need(tokens, "tokens", torch.int32)
    cap = B * g1
    # dense [B*(gamma+1), V] with source rows, or packed rows with capacity
    # B*(gamma+1) (the packed total is a device value, so the full capacity is
    # required for the reads to stay inside the buffer)
    if logits.numel() != cap * V:
        raise ValueError("logits must hold B*(gamma+1) rows of V entries")
    if packed_src_row is not None:
        _need(packed_src_row, "packed_src_row", torch.int32, (cap,))
    dev = tokens.device
    out = out or {}
    pam = out.get("packed_argmax")
    acc = out.get("accepted")
    bon = out.get("bonus")
    pam = torch.full((cap,), -1, dtype=torch.int32, device=dev) if pam is None else pam
    acc = torch.empty(B, dtype=torch.int32, device=dev) if acc is None else acc
    bon = torch.empty(B, dtype=torch.int32, device=dev) if bon is None else bon
    _need(pam, "packed_argmax", torch.int32, (cap,))
    _need(acc, "accepted", torch.int32, (B,))
    _need(bon, "bonus", torch.int32, (B,))
    ws = workspace(B, g, V, dev) if ws is None else _need(ws, "ws", torch.uint8)
    _ok("dspark_accept", lib().dspark_accept(
        _ptr(logits), _ptr(packed_src_row), _ptr(cu_seqlens), _ptr(tokens), B, g, V, _ptr(pam),
        _ptr(acc), _ptr(bon), _ptr(ws), ws.numel(), _stream(dev)))
    return pam, acc, bon


STEP_OUTPUTS = ("conf", "survival", "lengths", "cu_seqlens", "packed_tokens", "packed_src_row",
                "packed_argmax", "accepted", "bonus")


def dspark_gather_rows(src, packed_src_row, cu_seqlens, out=None):
    """Packed row gather: out[r] = src[packed_src_row[r]] for r < cu_seqlens[B].
    src is [B*(gamma+1), ...] (or [B, gamma+1, ...]) of any dtype; out has the
    same row shape and B*(gamma+1) rows (allocated when None)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    B = cu_seqlens.numel() - 1
    _need(packed_src_row, "packed_src_row", torch.int32)
    cap = packed_src_row.numel()
    if cap % B != 0:
        raise ValueError("packed_src_row must have B*(gamma+1) entries")
    g = cap // B - 1
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if src.numel() % cap != 0:
        raise ValueError("src must hold B*(gamma+1) rows")
    if src.shape[0] == cap:
        row_shape = (cap,) + tuple(src.shape[1:])
    elif src.dim() >= 2 and tuple(src.shape[:2]) == (B, g + 1):
        row_shape = (cap,) + tuple(src.shape[2:])
    else:
        raise ValueError("src must be [B*(gamma+1), ...] or [B, gamma+1, ...]")
    row_bytes = src.numel() // cap * src.element_size()
    if out is None:
        out = torch.empty(row_shape, dtype=src.dtype, device=src.device)
    if (out.dtype != src.dtype or not out.is_contiguous() or out.device != src.device
            or out.numel() * out.element_size() != cap * row_bytes):
        raise ValueError("out must be a contiguous GPU tensor of B*(gamma+1) rows like src")
    _ok("dspark_gather_rows", lib().dspark_gather_rows(
        _ptr(src), _ptr(packed_src_row), _ptr(cu_seqlens), B, g, row_bytes, _ptr(out),
        _stream(src.device)))
    return out


def dspark_cost_cutoff(table, load, B, cutoff=None):
    """Every request's cutoff from the cost table at the step's load level:
    table fp32 [n] and load int32 [1] on the device; returns cutoff fp32 [B]."""
    _need(table, "table", torch.float32)
    _need(load, "load", torch.int32, (1,))
    dev = table.device
    cutoff = torch.empty(B, dtype=torch.float32, device=dev) if cutoff is None else cutoff
    _need(cutoff, "cutoff", torch.float32, (B,))
    _ok("dspark_cost_cutoff", lib().dspark_cost_cutoff(
        _ptr(table), table.numel(), _ptr(load), int(B), _ptr(cutoff), _stream(dev)))
    return cutoff


def dspark_tier_select(cu_seqlens, gamma, tiers, pad_token=0, packed_tokens=None,
                       packed_src_row=None, out=None):
    """Graph tier of a packed batch: (padded_total [1], tier_index [1]) int32 on
    the device; pads packed_tokens / packed_src_row (when given) up to the
    tier. tiers: int32 device tensor, strictly ascending."""
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    B = cu_seqlens.numel() - 1
    _need(tiers, "tiers", torch.int32)
    dev = cu_seqlens.device
    cap = B * (gamma + 1)
    for t, n in ((packed_tokens, "packed_tokens"), (packed_src_row, "packed_src_row")):
        if t is not None:
            _need(t, n, torch.int32, (cap,))
    out = out or {}
    padded = out.get("padded_total")
    idx = out.get("tier_index")
    padded = torch.empty(1, dtype=torch.int32, device=dev) if padded is None else padded
    idx = torch.empty(1, dtype=torch.int32, device=dev) if idx is None else idx
    _need(padded, "padded_total", torch.int32, (1,))
    _need(idx, "tier_index", torch.int32, (1,))
    _ok("dspark_tier_select", lib().dspark_tier_select(
        _ptr(cu_seqlens), B, int(gamma), _ptr(tiers), tiers.numel(), int(pad_token), _ptr(padded),
        _ptr(idx), _ptr(packed_tokens), _ptr(packed_src_row), _stream(dev)))
    return padded, idx


def dspark_cap_accept(packed_argmax_full, tokens, lengths, out=None, sums=None):
    """Cap-accept audit arm over a static verify: (accepted, bonus,
    accepted_full, sums). packed_argmax_full holds the argmax of every row of
    the full block (static packing, [B*(gamma+1)]); lengths is the cut's
    window. sums, when given (int64 [2]), receives (sum accepted, sum
    accepted_full)."""
    B, g1 = tokens.shape
    _need(tokens, "tokens", torch.int32)
    _need(packed_argmax_full, "packed_argmax_full", torch.int32, (B * g1,))
    _need(lengths, "lengths", torch.int32, (B,))
    dev = tokens.device
    out = out or {}
    acc = out.get("accepted")
    bon = out.get("bonus")
    full = out.get("accepted_full")
    acc = torch.empty(B, dtype=torch.int32, device=dev) if acc is None else acc
    bon = torch.empty(B, dtype=torch.int32, device=dev) if bon is None else bon
    full = torch.empty(B, dtype=torch.int32, device=dev) if full is None else full
    for t, n in ((acc, "accepted"), (bon, "bonus"), (full, "accepted_full")):
        _need(t, n, torch.int32, (B,))
    if sums is not None:
        _need(sums, "sums", torch.int64, (2,))
    _ok("dspark_cap_accept", lib().dspark_cap_accept(
        _ptr(packed_argmax_full), _ptr(tokens), _ptr(lengths), B, g1 - 1, _ptr(acc), _ptr(bon),
        _ptr(full), _ptr(sums), _stream(dev)))
    return acc, bon, full, sums


def alloc_step_outputs(B: int, gamma: int, device, with_conf: bool = True) -> Dict[str, torch.Tensor]:
    cap = B * (gamma + 1)
    i32 = dict(dtype=torch.int32, device=device)
    out = dict(lengths=torch.empty(B, **i32), cu_seqlens=torch.empty(B + 1, **i32),
               packed_tokens=torch.full((cap,), -1, **i32),
               packed_src_row=torch.full((cap,), -1, **i32),
               packed_argmax=torch.full((cap,), -1, **i32),
               accepted=torch.empty(B, **i32), bonus=torch.empty(B, **i32))
    if with_conf:
        out["conf"] = torch.empty((B, gamma), dtype=torch.float32, device=device)
        out["survival"] = torch.empty((B, gamma), dtype=torch.float32, device=device)
    return out


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (created on first use) or a handle."""
    if ev is None:
        return None
    if isinstance(ev, torch.cuda.Event):
        if not ev.cuda_event:
            ev.record()                  # torch creates the event lazily
        return ctypes.c_void_p(ev.cuda_event)
    return ctypes.c_void_p(int(ev))


def dspark_step(hidden, w, bias, temps, tokens, logits, mode, cutoff=None, budget=0, out=None,
                ws=None, events=None, launches=0, wait_ticks=0):
    """Steps 1-6 in one call; returns the dict of output tensors. With any of
    `events` (a pair of timing events, recorded around the step's dominant
    kernel), `launches` (0 by size, 1 one launch where the cut allows it, 2 two
    launches) or `wait_ticks` (bound of the one-launch wait, 100 MHz ticks; 0 is
    the default) the call goes through dspark_step_ex."""
    args, out, ws = _step_args(hidden, w, bias, temps, tokens, logits, mode, cutoff, budget, out,
                               ws, None)
    if events is None and not launches and not wait_ticks:
        _ok("dspark_step", lib().dspark_step(*args))
    else:
        ev = events if events is not None else (None, None)
        _ok("dspark_step_ex", lib().dspark_step_ex(
            *args, _event_handle(ev[0]), _event_handle(ev[1]), int(launches), int(wait_ticks)))
    return out


def _step_args(hidden, w, bias, temps, tokens, logits, mode, cutoff, budget, out, ws, stream):
    """Checked, marshalled arguments of dspark_step (and the outputs)."""
    B, g, d = hidden.shape
    V = logits.shape[-1]
    _need(hidden, "hidden", torch.bfloat16)
    _need(w, "w", torch.bfloat16, (d,))
    _need(temps, "temps", torch.float32, (g,))
    _need(tokens, "tokens", torch.int32, (B, g + 1))
    _need(logits, "logits", torch.bfloat16, (B, g + 1, V))
    m = _mode(mode)
    if cutoff is not None:
        _need(cutoff, "cutoff", torch.float32, (B,))
    dev = hidden.device
    out = alloc_step_outputs(B, g, dev) if out is None else out
    cap = B * (g + 1)
    shapes = dict(conf=(B, g), survival=(B, g), lengths=(B,), cu_seqlens=(B + 1,),
                  packed_tokens=(cap,), packed_src_row=(cap,), packed_argmax=(cap,),
                  accepted=(B,), bonus=(B,))
    for k, shp in shapes.items():
        if out.get(k) is not None:
            _need(out[k], k, torch.float32 if k in ("conf", "survival") else torch.int32, shp)
    ws = workspace(B, g, V, dev) if ws is None else _need(ws, "ws", torch.uint8)
    st = _stream(dev) if stream is None else ctypes.c_void_p(int(stream))
    args = (
        _ptr(hidden), _ptr(w), float(bias), _ptr(temps), _ptr(tokens), _ptr(logits), B, g, d, V,
        m, _ptr(cutoff), int(budget), _ptr(out.get("conf")), _ptr(out.get("survival")),
        _ptr(out["lengths"]), _ptr(out["cu_seqlens"]), _ptr(out["packed_tokens"]),
        _ptr(out["packed_src_row"]), _ptr(out["packed_argmax"]), _ptr(out["accepted"]),
        _ptr(out["bonus"]), _ptr(ws), ws.numel(), st)
    return args, out, ws


class BoundStep:
    """dspark_step on fixed buffers: the arguments are checked and marshalled
    once, and each call is one C call (for serving loops that refill the same
    input buffers every step, where the per-call checks of dspark_step cost
    more host time than a small step takes on the GPU). The tensors must stay
    alive, in place and unresized while the object is used; calls run on the
    stream given at binding (the current stream by default)."""

    def __init__(self, hidden, w, bias, temps, tokens, logits, mode, cutoff=None, budget=0,
                 out=None, ws=None, launches=0, wait_ticks=0, stream=None):
        args, self.out, self.ws = _step_args(hidden, w, bias, temps, tokens, logits, mode, cutoff,
                                             budget, out, ws, stream)
        # the tensors the raw pointers point into
        self._keep = (hidden, w, temps, tokens, logits, cutoff, self.out, self.ws)
        self._fn = lib().dspark_step_ex
        self._args = args + (None, None, int(launches), int(wait_ticks))

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            raise DsparkError("dspark_step_ex", status)
        return self.out


def bind_step(hidden, w, bias, temps, tokens, logits, mode, cutoff=None, budget=0, out=None,
              ws=None, launches=0, wait_ticks=0, stream=None) -> BoundStep:
    """A BoundStep: dspark_step's arguments checked once, launched by calling it."""
    return BoundStep(hidden, w, bias, temps, tokens, logits, mode, cutoff=cutoff, budget=budget,
                     out=out, ws=ws, launches=launches, wait_ticks=wait_ticks, stream=stream)


def dspark_step_ex(hidden, w, bias, temps, tokens, logits, mode, cutoff=None, budget=0,
                   out=None, ws=None, events=None, launches=0, wait_ticks=0):
    """dspark_step with explicit controls: timing events around its dominant
    kernel, the form (launches) and the bound of the one-launch wait."""
    return dspark_step(hidden, w, bias, temps, tokens, logits, mode, cutoff=cutoff,
                       budget=budget, out=out, ws=ws, events=events, launches=launches,
                       wait_ticks=wait_ticks)


def dspark_step_noalloc(hidden, w, bias, temps, tokens, logits, mode, cutoff=None, budget=0,
                        out=None, status=None):
    """dspark_step without a workspace argument: the library's own per-device
    scratch array serves as the workspace, so the call allocates nothing on the
    device side (torch allocates the outputs here only when `out` is None).
    `status` (int32 [1], optional) receives the give-up flag of this call.
    Calls on one device share that scratch and must not overlap in time."""
    B, g, d = hidden.shape
    V = logits.shape[-1]
    _need(hidden, "hidden", torch.bfloat16)
    _need(w, "w", torch.bfloat16, (d,))
    _need(temps, "temps", torch.float32, (g,))
    _need(tokens, "tokens", torch.int32, (B, g + 1))
    _need(logits, "logits", torch.bfloat16, (B, g + 1, V))
    m = _mode(mode)
    if cutoff is not None:
        _need(cutoff, "cutoff", torch.float32, (B,))
    dev = hidden.device
    out = alloc_step_outputs(B, g, dev) if out is None else out
    if status is not None:
        _need(status, "status", torch.int32, (1,))
    _ok("dspark_step_noalloc", lib().dspark_step_noalloc(
        _ptr(hidden), _ptr(w), float(bias), _ptr(temps), _ptr(tokens), _ptr(logits), B, g, d, V,
        m, _ptr(cutoff), int(budget), _ptr(out.get("conf")), _ptr(out.get("survival")),
        _ptr(out["lengths"]), _ptr(out["cu_seqlens"]), _ptr(out["packed_tokens"]),
        _ptr(out["packed_src_row"]), _ptr(out["packed_argmax"]), _ptr(out["accepted"]),
        _ptr(out["bonus"]), _ptr(status), _stream(dev)))
    return out


def dspark_step_status(ws=None, status=None, device=None):
    """The fused step's give-up flag of a workspace, read and cleared on the
    device: an int32 [1] tensor, 0 when no call since the last read gave up its
    bounded wait. ws defaults to the binding's cached workspace of `device`."""
    if ws is None:
        ws = _WS.get(_ws_key(device if device is not None else "cuda"))
        if ws is None:
            raise ValueError("no workspace has been used on this device")
    _need(ws, "ws", torch.uint8)
    status = torch.empty(1, dtype=torch.int32, device=ws.device) if status is None else status
    _need(status, "status", torch.int32, (1,))
    _ok("dspark_step_status", lib().dspark_step_status(_ptr(ws), _ptr(status), _stream(ws.device)))
    return status


__all__ = ["DsparkError", "lib", "LIB_PATH", "dspark_status_string", "dspark_confidence", "dspark_schedule",
           "dspark_compact", "dspark_accept", "dspark_step", "dspark_cap_accept",
           "dspark_gather_rows", "dspark_tier_select", "dspark_cost_cutoff",
           "dspark_step_ex", "dspark_step_status", "dspark_step_noalloc", "BoundStep", "bind_step",
           "dspark_workspace_bytes",
           "dspark_workspace_init", "workspace", "alloc_step_outputs", "STEP_OUTPUTS",
           "DSPARK_CUT_THRESHOLD", "DSPARK_CUT_BUDGET", "DSPARK_CUT_STATIC",
           "DSPARK_CUT_COMBINED"]
