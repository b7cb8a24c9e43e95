"""Seeded synthetic inputs for the MoE layer workloads.

This module draws inputs only.  It holds none of the layer's arithmetic: no
softmax, no gate, no dispatch, no expert FFN.  Two input-conditioning steps
that the workload recipe itself states need a plain fp64 matrix product and a
partial sort of its rows, and are done here:

* the near-tie redraw: a token whose k-th and (k+1)-th largest router logits
  (bias included) differ by less than ``cfg.margin`` is redrawn, so that the
  selected expert set is the same whatever the precision of the logits;
* the Zipf-shaped router biases of the skewed workload, calibrated on the
  drawn tokens so that expert popularity follows target loads.

Random streams: numpy PCG64 under SeedSequence(0) with one spawn key per
(workload, tensor, expert).  Expert weights are drawn with a torch generator
on the target device (so a 22 GB weight set is drawn in seconds on a GPU),
seeded from the same substream; host and device therefore give different
but equally seeded values, and a check always hands both sides the same
tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerConfig, ShareConfig

ROOT_SEED = 0
# substream ids
S_WR, S_WGATE, S_WUP, S_WDOWN, S_WSGATE, S_WSUP, S_WSDOWN, S_X, S_DY, S_COUNTS = range(10)


def _ss(cid: int, tensor: int, expert: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence(ROOT_SEED, spawn_key=(cid, tensor, expert))


def np_rng(cid: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_ss(cid, tensor, expert)))


def torch_gen(cid: int, tensor: int, expert: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(_ss(cid, tensor, expert).generate_state(1, np.uint64)[0] & ((1 << 63) - 1)))
    return g


def torch_dtype(name: str) -> torch.dtype:
    # MXFP8 weights and activations are drawn in bf16 and quantised afterwards.
    return torch.float32 if name == "f32" else torch.bfloat16


def _round_as(x32: np.ndarray, dtype: str) -> np.ndarray:
    """The fp32 draws as the layer will see them (bf16 round-to-nearest-even), in fp64."""
    t = torch.from_numpy(np.ascontiguousarray(x32))
    if dtype != "f32":
        t = t.to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest value of each row (inf when k == E)."""
    E = logits.shape[1]
    if k >= E:
        return np.full(logits.shape[0], np.inf)
    part = -np.partition(-logits, k, axis=1)[:, : k + 1]
    part.sort(axis=1)
    return part[:, 1] - part[:, 0]


def zipf_targets(n: int, E: int, s: float, hot: float) -> np.ndarray:
    """Target loads proportional to (r + q)^-s, r = 1..E, with q chosen so that the
    hottest expert receives ``hot`` times the mean load (rank r is expert r-1)."""
    r = np.arange(1, E + 1, dtype=np.float64)

    def ratio(q):
        w = (r + q) ** -s
        return E * w[0] / w.sum()

    lo, hi = 0.0, 1.0
    while ratio(hi) > hot:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if ratio(mid) > hot:
            lo = mid
        else:
            hi = mid
    q = 0.5 * (lo + hi)
    w = (r + q) ** -s
    return n * w / w.sum()


def calibrate_bias(l0: np.ndarray, k: int, target: np.ndarray, iters: int = 60) -> np.ndarray:
    """Damped fixed point b <- b + 0.5 ln(target / max(count, 1/2)) on the drawn tokens."""
    E = l0.shape[1]
    b = np.zeros(E)
    for _ in range(iters):
        sel = np.argpartition(-(l0 + b), k - 1, axis=1)[:, :k]
        cnt = np.bincount(sel.ravel(), minlength=E).astype(np.float64)
        b = b + 0.5 * np.log(target / np.maximum(cnt, 0.5))
    return b


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor                   # [T, d] f32 or bf16
    w_router: torch.Tensor            # [E, d] f32
    b_router: Optional[torch.Tensor]  # [E] f32 or None
    w_gate: torch.Tensor              # [E, f, d]
    w_up: torch.Tensor                # [E, f, d]
    w_down: torch.Tensor              # [E, d, f]
    ws_gate: Optional[torch.Tensor] = None   # [fs, d]
    ws_up: Optional[torch.Tensor] = None     # [fs, d]
    ws_down: Optional[torch.Tensor] = None   # [d, fs]
    dy: Optional[torch.Tensor] = None        # [T, d] bf16
    redrawn: int = 0


def draw_router_and_tokens(cfg: LayerConfig):
    """Router weight, bias (skewed workload only), and tokens after the near-tie redraw.
    Returns numpy fp32 arrays (w_r [E,d], b [E] or None, x [T,d]) and the redraw count."""
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    w_r = (np_rng(cfg.cid, S_WR).standard_normal((E, d), dtype=np.float32)
           * np.float32(1.0 / math.sqrt(d)))
    gx = np_rng(cfg.cid, S_X)
    x = gx.standard_normal((T, d), dtype=np.float32)
    w64 = w_r.astype(np.float64)
    b = None
    if cfg.zipf_s > 0:
        l0 = _round_as(x, cfg.dtype) @ w64.T
        b = calibrate_bias(l0, k, zipf_targets(T * k, E, cfg.zipf_s, cfg.hot_ratio)).astype(np.float32)
    b64 = np.zeros(E) if b is None else b.astype(np.float64)
    redrawn = 0
    rows = np.arange(T)
    logits = np.empty((T, E))
    while True:
        logits[rows] = _round_as(x[rows], cfg.dtype) @ w64.T + b64
        bad = np.nonzero(topk_gap(logits[rows], k) < cfg.margin)[0]
        if bad.size == 0:
            break
        rows = rows[bad]
        for t in rows:               # ascending token order, same continuing stream
            x[t] = gx.standard_normal(d, dtype=np.float32)
        redrawn += rows.size
    return w_r, b, x, redrawn


def _expert_stack(cfg, tensor, E, rows, cols, std, device, dtype):
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    s = torch.tensor(std, dtype=torch.float32).item()
    for e in range(E):
        g = torch_gen(cfg.cid, tensor, e, device)
        w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
        out[e].copy_((w * s).to(dtype))
    return out


def make_layer(cfg: LayerConfig, device="cpu", reuse: Optional[LayerInputs] = None) -> LayerInputs:
    """Draw every input of one workload onto ``device``.  With ``reuse``, expert weights
    drawn for another batch of the same workload (same seed substream and shapes) are
    shared instead of drawn again."""
    device = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    w_r, b, x, redrawn = draw_router_and_tokens(cfg)
    sd = float(np.float32(1.0 / math.sqrt(cfg.d)))
    sf = float(np.float32(1.0 / math.sqrt(cfg.f)))
    same = (reuse is not None and reuse.cfg.cid == cfg.cid and reuse.cfg.d == cfg.d
            and reuse.cfg.E == cfg.E and reuse.cfg.f == cfg.f and reuse.cfg.fs == cfg.fs
            and reuse.cfg.dtype == cfg.dtype and reuse.w_gate.device.type == device.type)
    inp = LayerInputs(
        cfg=cfg,
        x=torch.from_numpy(x).to(dt).to(device),
        w_router=torch.from_numpy(w_r).to(device),
        b_router=None if b is None else torch.from_numpy(b).to(device),
        w_gate=reuse.w_gate if same else _expert_stack(cfg, S_WGATE, cfg.E, cfg.f, cfg.d, sd, device, dt),
        w_up=reuse.w_up if same else _expert_stack(cfg, S_WUP, cfg.E, cfg.f, cfg.d, sd, device, dt),
        w_down=reuse.w_down if same else _expert_stack(cfg, S_WDOWN, cfg.E, cfg.d, cfg.f, sf, device, dt),
        redrawn=redrawn,
    )
    if same and cfg.fs:
        inp.ws_gate, inp.ws_up, inp.ws_down = reuse.ws_gate, reuse.ws_up, reuse.ws_down
    elif cfg.fs:
        sfs = float(np.float32(1.0 / math.sqrt(cfg.fs)))
        inp.ws_gate = _expert_stack(cfg, S_WSGATE, 1, cfg.fs, cfg.d, sd, device, dt)[0]
        inp.ws_up = _expert_stack(cfg, S_WSUP, 1, cfg.fs, cfg.d, sd, device, dt)[0]
        inp.ws_down = _expert_stack(cfg, S_WSDOWN, 1, cfg.d, cfg.fs, sfs, device, dt)[0]
    if cfg.backward:
        dy = np_rng(cfg.cid, S_DY).standard_normal((cfg.T, cfg.d), dtype=np.float32)
        inp.dy = torch.from_numpy(dy).to(torch.bfloat16).to(device)
    return inp


@dataclass
class ShareInputs:
    cfg: ShareConfig
    counts: np.ndarray        # [E] int64, multinomial
    ring_x: torch.Tensor      # [C, d] bf16, rows 0..rows-1 filled (ring head 0)
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor


def make_share(cfg: ShareConfig, device="cpu") -> ShareInputs:
    """The expert-FFN operands of one GPU's expert-parallel share: received rows already
    expert-contiguous from ring slot 0, counts ~ Multinomial(rows, uniform)."""
    device = torch.device(device)
    counts = np_rng(cfg.cid, S_COUNTS).multinomial(cfg.rows, np.full(cfg.E, 1.0 / cfg.E))
    ring = torch.zeros((cfg.C, cfg.d), dtype=torch.bfloat16, device=device)
    g = torch_gen(cfg.cid, S_X, 0, device)
    ring[: cfg.rows] = torch.randn((cfg.rows, cfg.d), generator=g, device=device,
                                   dtype=torch.float32).to(torch.bfloat16)
    sd = float(np.float32(1.0 / math.sqrt(cfg.d)))
    sf = float(np.float32(1.0 / math.sqrt(cfg.f)))
    lc = LayerConfig(cfg.name, T=cfg.rows, d=cfg.d, E=cfg.E, k=1, f=cfg.f, cid=cfg.cid)
    return ShareInputs(
        cfg=cfg, counts=counts.astype(np.int64), ring_x=ring,
        w_gate=_expert_stack(lc, S_WGATE, cfg.E, cfg.f, cfg.d, sd, device, torch.bfloat16),
        w_up=_expert_stack(lc, S_WUP, cfg.E, cfg.f, cfg.d, sd, device, torch.bfloat16),
        w_down=_expert_stack(lc, S_WDOWN, cfg.E, cfg.d, cfg.f, sf, device, torch.bfloat16),
    )


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)
