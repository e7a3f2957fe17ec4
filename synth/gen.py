"""Seeded input generator for the verify hot path.

Recipe (one step of one workload):

* Parameters, drawn once per workload: the confidence-head weight
  ``w ~ N(0, 1/d)`` (fp64 draw, rounded to fp32 then to bf16, both
  round-to-nearest-even), the scalar bias, and the STS temperatures
  ``T_i = 1 + slope * i`` for i = 0..gamma-1.
* Host draws per step (numpy PCG64, one SeedSequence stream per purpose):
  the per-request confidence-logit shift ``s_b``, an optional per-position
  latent ``zeta[b,i] ~ N(0,1)``, the per-request cutoffs, the planting flags,
  the draft ids and the root ids. ``lam = s_b + zeta`` is the latent
  confidence logit.
* Device draws per step (torch's seeded generator on the target device):
  the hidden noise ``n ~ N(0,1)`` of shape [B, gamma, d] and the target logits
  ``~ N(0, var)`` of shape [B, gamma+1, V]. The hidden state is
  ``bf16(n + lam * w / |w|^2)``, which moves the head's logit ``w.h`` by
  ``lam`` without this module ever forming ``w.h``.
* Planting: draft position i of request b is predicted by logit row i. When
  its flag is set, the logit at the draft id becomes ``bf16(rowmax + 4)``,
  so that id is the unique maximum of the row. Row gamma is never planted.

The values of the two device-drawn arrays depend on the device type (torch's
CPU and GPU generators differ); every consumer copies one generated step to
wherever it needs it, so both sides always see the same bytes.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

from .configs import Config

_PARAM_STEP = 1 << 30  # step id reserved for the per-workload parameter streams


# --------------------------------------------------------------------------- bf16

def rne_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    return rne_bf16(x)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------------ streams

def _ss(cfg: Config, step: int, purpose: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(0, spawn_key=(cfg.index, step, purpose))


def _rng(cfg: Config, step: int, purpose: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_ss(cfg, step, purpose)))


def _torch_seed(cfg: Config, step: int, purpose: int) -> int:
    s = _ss(cfg, step, purpose).generate_state(2, np.uint32)
    return (int(s[0]) | (int(s[1]) << 32)) & ((1 << 63) - 1)


# ----------------------------------------------------------------------- params

@dataclass
class Params:
    w_bits: np.ndarray      # [d] uint16 (bf16 bits)
    bias: float             # exactly representable in fp32
    temps: np.ndarray       # [gamma] float32


def make_params(cfg: Config) -> Params:
    rng = _rng(cfg, _PARAM_STEP, 0)
    w64 = rng.standard_normal(cfg.d) * np.sqrt(1.0 / cfg.d)
    w_bits = rne_bf16(w64.astype(np.float32))
    temps = (1.0 + cfg.temp_slope * np.arange(cfg.gamma, dtype=np.float64)).astype(np.float32)
    bias = float(np.float32(cfg.bias))
    return Params(w_bits=w_bits, bias=bias, temps=temps)


# ------------------------------------------------------------------------- step

@dataclass
class StepInputs:
    cfg: Config
    step: int
    device: torch.device
    hidden: torch.Tensor        # [B, gamma, d] bfloat16
    w: torch.Tensor             # [d] bfloat16
    bias: float
    temps: torch.Tensor         # [gamma] float32
    cutoff: torch.Tensor        # [B] float32 (threshold mode; zeros in budget mode)
    budget: int                 # batch-wide budget T (budget mode; 0 otherwise)
    tokens: torch.Tensor        # [B, gamma+1] int32; column 0 is the root token
    logits: torch.Tensor        # [B, gamma+1, V] bfloat16
    plant: np.ndarray           # [B, gamma] bool: logit row i was planted with draft i
    lam: np.ndarray             # [B, gamma] float64 latent confidence logit
    match_prob: np.ndarray      # [B, gamma] float64 planting probability
    _host: Dict[str, np.ndarray] = field(default_factory=dict, repr=False)

    @property
    def mode(self) -> str:
        return self.cfg.mode

    # Host copies for the oracle. These are copies of generated data only.
    def host(self, name: str) -> np.ndarray:
        if name not in self._host:
            t = getattr(self, name)
            if t.dtype == torch.bfloat16:
                a = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            else:
                a = t.detach().contiguous().cpu().numpy()
            self._host[name] = a
        return self._host[name]

    def host_rows(self, dense_rows: np.ndarray) -> np.ndarray:
        """Copy only the listed dense logit rows ([n, V] uint16) to the host."""
        idx = torch.as_tensor(np.asarray(dense_rows, dtype=np.int64), device=self.device)
        flat = self.logits.view(-1, self.cfg.V)
        rows = flat.index_select(0, idx)
        return rows.view(torch.int16).cpu().numpy().view(np.uint16)

    def digest(self) -> str:
        h = hashlib.sha256()
        for name in ("hidden", "w", "temps", "cutoff", "tokens", "logits"):
            h.update(self.host(name).tobytes())
        h.update(np.float32(self.bias).tobytes())
        h.update(np.int64(self.budget).tobytes())
        return h.hexdigest()


def _match_prob(cfg: Config, lam: np.ndarray) -> np.ndarray:
    B, g = cfg.B, cfg.gamma
    if cfg.match == "const":
        return np.full((B, g), cfg.match_p)
    if cfg.match == "decay":
        return np.broadcast_to(cfg.match_p * 0.97 ** np.arange(g), (B, g)).copy()
    if cfg.match == "sigmoid":
        return 1.0 / (1.0 + np.exp(-lam))
    if cfg.match == "bimodal":
        p = np.where(np.arange(B) % 2 == 0, 0.95, 0.45)
        return np.broadcast_to(p[:, None], (B, g)).copy()
    raise ValueError(cfg.match)


def _shift(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.shift == "none":
        return np.zeros(cfg.B)
    if cfg.shift == "normal":
        return rng.standard_normal(cfg.B)
    if cfg.shift == "bimodal":
        return np.where(np.arange(cfg.B) % 2 == 0, 3.0, -1.0)
    raise ValueError(cfg.shift)


def make_step(cfg: Config, step: int, device="cpu", params: Optional[Params] = None) -> StepInputs:
    device = torch.device(device)
    if params is None:
        params = make_params(cfg)
    B, g, d, V = cfg.B, cfg.gamma, cfg.d, cfg.V

    # host draws, one stream per purpose so that changing one leaves the rest alone
    s = _shift(cfg, _rng(cfg, step, 1))
    zeta = _rng(cfg, step, 2).standard_normal((B, g)) if cfg.latent else np.zeros((B, g))
    lam = s[:, None] + zeta
    if cfg.mode in ("threshold", "combined"):
        if cfg.cutoff_range is not None:
            lo, hi = cfg.cutoff_range
            cutoff = _rng(cfg, step, 3).uniform(lo, hi, B).astype(np.float32)
        else:
            cutoff = np.full(B, cfg.cutoff, dtype=np.float32)
    else:
        cutoff = np.zeros(B, dtype=np.float32)
    match_prob = _match_prob(cfg, lam)
    plant = _rng(cfg, step, 4).random((B, g)) < match_prob
    drafts = _rng(cfg, step, 5).integers(0, V, size=(B, g), dtype=np.int64)
    roots = _rng(cfg, step, 6).integers(0, V, size=B, dtype=np.int64)
    tokens = np.concatenate([roots[:, None], drafts], axis=1).astype(np.int32)

    # device draws
    gen_h = torch.Generator(device=device)
    gen_h.manual_seed(_torch_seed(cfg, step, 7))
    n = torch.randn((B, g, d), generator=gen_h, device=device, dtype=torch.float32)
    w_f32 = bf16_bits_to_f32(params.w_bits)
    if np.any(lam != 0.0):
        w64 = w_f32.astype(np.float64)
        u = torch.as_tensor((w64 / float(np.sum(w64 * w64))).astype(np.float32), device=device)
        lam_t = torch.as_tensor(lam.astype(np.float32), device=device)
        n.add_(lam_t[:, :, None] * u[None, None, :])
    hidden = n.to(torch.bfloat16)
    del n

    gen_l = torch.Generator(device=device)
    gen_l.manual_seed(_torch_seed(cfg, step, 8))
    logits = torch.empty((B, g + 1, V), dtype=torch.bfloat16, device=device)
    scale = float(np.float32(np.sqrt(cfg.logit_var)))
    # draw per request to bound the fp32 temporary
    for b in range(B):
        x = torch.randn((g + 1, V), generator=gen_l, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        logits[b].copy_(x.to(torch.bfloat16))
    del x
    if plant.any():
        rowmax = logits[:, :g, :].amax(dim=-1)                        # [B, g] bf16, exact
        planted_val = (rowmax.float() + 4.0).to(torch.bfloat16)       # RNE
        bi, ii = np.nonzero(plant)
        bi_t = torch.as_tensor(bi, device=device)
        ii_t = torch.as_tensor(ii, device=device)
        ti_t = torch.as_tensor(drafts[bi, ii], device=device)
        logits[bi_t, ii_t, ti_t] = planted_val[bi_t, ii_t]

    w = torch.as_tensor(params.w_bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return StepInputs(
        cfg=cfg, step=step, device=device, hidden=hidden, w=w, bias=params.bias,
        temps=torch.as_tensor(params.temps).to(device),
        cutoff=torch.as_tensor(cutoff).to(device), budget=cfg.budget,
        tokens=torch.as_tensor(tokens).to(device), logits=logits,
        plant=plant, lam=lam, match_prob=match_prob)
