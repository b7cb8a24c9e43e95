"""GPU parity of the backward (reverse ring traversal) against the fp64 oracle.

dx, dW_gate, dW_up, dW_down (bf16) and dW_r (fp32) within max-abs-rel 2e-2;
experts with no rows get exactly zero weight gradients; repeated runs are
bitwise identical."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_33_amd as moe
import oracle
from gen import SKEW_BWD, LayerConfig, make_layer
from layer_util import LazyWeights, rel, to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2

MEDIUM = [
    LayerConfig("bwd_small", T=300, d=256, E=16, k=4, f=128, backward=True, cid=50),
    LayerConfig("bwd_skew", T=512, d=384, E=32, k=4, f=256, zipf_s=1.1, hot_ratio=8.0,
                backward=True, cid=51),
    # 400 copies over 64 experts with a strong skew: several experts receive nothing
    LayerConfig("bwd_sparse", T=200, d=128, E=64, k=2, f=128, zipf_s=1.1, hot_ratio=12.0,
                backward=True, cid=52),
    # 142-163 rows per expert: every expert spans a full and a ragged 128-row tile
    LayerConfig("bwd_tall", T=600, d=256, E=8, k=2, f=128, backward=True, cid=53),
    # skewed loads from 87 to 767 rows: the hottest expert spans six tiles, the last ragged
    LayerConfig("bwd_tall_skew", T=1024, d=256, E=8, k=2, f=128, zipf_s=1.1, hot_ratio=3.0,
                backward=True, cid=54),
]


def run(layer, inp, head):
    layer.forward(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                  head=head, save_au=True)
    out = layer.backward(inp.dy, inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, head=head)
    torch.cuda.synchronize()
    return [t.clone() for t in out]


@pytest.mark.parametrize("cfg", MEDIUM, ids=lambda c: c.name)
def test_backward_parity(cfg):
    print(f"\n[case] backward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}", flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    W = oracle.weights_from_arrays(*(to_oracle(w) for w in (inp.w_gate, inp.w_up, inp.w_down)))
    r = oracle.route(x, w_r, b, cfg.k)
    ref = oracle.backward(x, w_r, r, W, to_oracle(inp.dy))
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    for head in (0, cfg.C - cfg.n // 2):
        dx, dwg, dwu, dwd, dwr = run(layer, inp, head)
        np.testing.assert_array_equal(layer.bufs["topk_idx"].cpu().numpy(), r.idx)
        errs = {"dx": rel(to_oracle(dx), ref.dx), "dw_gate": rel(to_oracle(dwg), ref.dw_gate),
                "dw_up": rel(to_oracle(dwu), ref.dw_up), "dw_down": rel(to_oracle(dwd), ref.dw_down),
                "dw_router": rel(dwr.cpu().numpy(), ref.dw_router)}
        print(f"  head={head}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        for name, v in errs.items():
            assert v <= TOL, name
        empty = np.nonzero(r.count == 0)[0]
        for t in (dwg, dwu, dwd, dwr):
            assert not t[torch.from_numpy(empty).to(DEV)].any()
    if cfg.name == "bwd_sparse":
        assert (r.count == 0).sum() > 0
    first = run(layer, inp, 0)
    for _ in range(2):
        for a, b2 in zip(first, run(layer, inp, 0)):
            assert torch.equal(a, b2)


def test_backward_full_size_sampled():
    cfg = SKEW_BWD
    print(f"\n[case] backward full size {cfg.name}", flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = to_oracle(inp.b_router)
    dy = to_oracle(inp.dy)
    r = oracle.route(x, w_r, b, cfg.k)
    hot_ratio = r.count.max() / r.count.mean()
    print(f"  hottest expert {hot_ratio:.2f}x the mean load", flush=True)
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    head = cfg.C - cfg.n // 2
    dx, dwg, dwu, dwd, dwr = run(layer, inp, head)
    np.testing.assert_array_equal(layer.bufs["topk_idx"].cpu().numpy(), r.idx)
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down)
    order = np.argsort(r.count)
    cold = [int(e) for e in order if r.count[e] > 0][:2]
    experts = sorted({int(order[-1]), *cold, 7})
    for e in experts:
        eg = oracle.expert_backward(e, x, dy, r, lw)
        errs = [rel(to_oracle(t[e]), ref) for t, ref in ((dwg, eg.dw_gate), (dwu, eg.dw_up), (dwd, eg.dw_down))]
        print(f"  expert {e} ({r.count[e]} rows): dW rel {errs}", flush=True)
        assert max(errs) <= TOL
    rows = oracle.router_weight_grad_rows(cold, x, w_r, r, lw, dy)
    err = rel(dwr[torch.tensor(cold, device=DEV)].cpu().numpy(), rows)
    print(f"  dW_r rows {cold}: rel {err:.2e}", flush=True)
    assert err <= TOL
    toks = [0, 4095, 8191]
    dxr, _, _ = oracle.backward_tokens(toks, x, w_r, r, lw, dy)
    err = rel(to_oracle(dx[torch.tensor(toks, device=DEV)]), dxr)
    print(f"  dx tokens {toks}: rel {err:.2e}", flush=True)
    assert err <= TOL
    again = run(layer, inp, head)
    for a, b2 in zip((dx, dwg, dwu, dwd, dwr), again):
        assert torch.equal(a, b2)
