"""GPU parity of the MXFP8 backward (moe_backward_mx) against the fp64 oracle's backward_mx.

The transposed weight codes and scales are bit-exact against the oracle's encoder along
the other axis; the saved A|U of the MXFP8 forward match the oracle's A, U; dx, dW_gate,
dW_up, dW_down and dW_r are within max-abs-rel 6e-2 (the MXFP8 tolerance); experts with
no rows get exactly zero weight gradients; repeated runs are bitwise identical."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_33_amd as moe
import oracle
from gen import SKEW_BWD, LayerConfig, make_layer
from layer_util import LazyWeights, mx_scale_rows, rel, to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 6e-2

MEDIUM = [
    LayerConfig("bwdmx_small", T=300, d=256, E=16, k=4, f=128, dtype="mxfp8", backward=True, cid=80),
    LayerConfig("bwdmx_skew", T=512, d=384, E=32, k=4, f=256, dtype="mxfp8", zipf_s=1.1,
                hot_ratio=8.0, backward=True, cid=81),
    # several experts receive nothing
    LayerConfig("bwdmx_sparse", T=200, d=128, E=64, k=2, f=128, dtype="mxfp8", zipf_s=1.1,
                hot_ratio=12.0, backward=True, cid=82),
    # 87 to 767 rows per expert: several 128-row tiles and 32-row token blocks, ragged
    LayerConfig("bwdmx_tall_skew", T=1024, d=256, E=8, k=2, f=128, dtype="mxfp8", zipf_s=1.1,
                hot_ratio=3.0, backward=True, cid=83),
]


class MxLayer:
    """Forward (MXFP8, saving A|U) and backward_mx of one workload on one Layer."""

    def __init__(self, cfg, inp):
        self.cfg, self.inp = cfg, inp
        q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
        self.wq = tuple(c for c, _ in q)
        self.scales = tuple(s for _, s in q)
        self.bw = moe.quantize_mx_t_backward_weights(inp.w_gate, inp.w_up, inp.w_down)
        self.layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype="mxfp8")

    def run(self, head):
        i = self.inp
        self.layer.forward(i.x, i.w_router, i.b_router, *self.wq, scales=self.scales, head=head,
                           save_au=True)
        out = self.layer.backward_mx(i.dy, i.x, i.w_router, *self.bw, head=head)
        torch.cuda.synchronize()
        return [t.clone() for t in out]


def check_backward_weights(ml, experts):
    """Transposed MX weights: bit-exact against the oracle's encoder along the other axis."""
    gu, gus, dn, dns = ml.bw
    f = ml.cfg.f
    gus_r = mx_scale_rows(gus).reshape(ml.cfg.E, ml.cfg.d, 2 * f // 32)
    dns_r = mx_scale_rows(dns).reshape(ml.cfg.E, f, ml.cfg.d // 32)
    for e in experts:
        wg, wu, wd = (to_oracle(w[e]) for w in (ml.inp.w_gate, ml.inp.w_up, ml.inp.w_down))
        cg, sg = oracle.mx.quantize(wg, axis=0)     # [f, d], blocks along f
        cu, su = oracle.mx.quantize(wu, axis=0)
        cd, sd = oracle.mx.quantize(wd, axis=0)     # [d, f], blocks along d
        np.testing.assert_array_equal(gu[e].cpu().numpy(), np.concatenate([cg.T, cu.T], axis=1))
        np.testing.assert_array_equal(gus_r[e].cpu().numpy(), np.concatenate([sg.T, su.T], axis=1))
        np.testing.assert_array_equal(dn[e].cpu().numpy(), cd.T)
        np.testing.assert_array_equal(dns_r[e].cpu().numpy(), sd.T)


def check_saved_au(ml, x, disp, experts):
    """The MXFP8 forward's saved A|U against A = Q_d(x) Q_d(W_gate)^T, U likewise."""
    au = ml.layer.bufs["saved_au"]
    f = ml.cfg.f
    for e in experts:
        slots = oracle.segment_slots(disp, e)
        if slots.size == 0:
            continue
        ts = disp.slot_copy[slots] // ml.cfg.k
        xq = oracle.mx.fake_quant(x[ts], axis=1)
        wg, wu = (oracle.mx.fake_quant(to_oracle(w[e]), axis=1) for w in (ml.inp.w_gate, ml.inp.w_up))
        got = to_oracle(au[torch.from_numpy(slots).to(DEV)])
        assert rel(got[:, :f], xq @ wg.T) <= 1e-2 and rel(got[:, f:], xq @ wu.T) <= 1e-2


@pytest.mark.parametrize("cfg", MEDIUM, ids=lambda c: c.name)
def test_backward_mx_parity(cfg):
    print(f"\n[case] MXFP8 backward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}",
          flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    W = oracle.weights_from_arrays(*(to_oracle(w) for w in (inp.w_gate, inp.w_up, inp.w_down)))
    r = oracle.route(x, w_r, b, cfg.k)
    ml = MxLayer(cfg, inp)
    check_backward_weights(ml, sorted({0, cfg.E // 2, cfg.E - 1}))
    for head in (0, cfg.C - cfg.n // 2):
        disp = oracle.dispatch(r.idx, cfg.E, cfg.C, head)
        dx, dwg, dwu, dwd, dwr = ml.run(head)
        np.testing.assert_array_equal(ml.layer.bufs["topk_idx"].cpu().numpy(), r.idx)
        check_saved_au(ml, x, disp, [int(np.argmax(r.count)), cfg.E - 1])
        ref = oracle.backward_mx(x, w_r, r, W, to_oracle(inp.dy), disp)
        errs = {"dx": rel(to_oracle(dx), ref.dx), "dw_gate": rel(to_oracle(dwg), ref.dw_gate),
                "dw_up": rel(to_oracle(dwu), ref.dw_up), "dw_down": rel(to_oracle(dwd), ref.dw_down),
                "dw_router": rel(dwr.cpu().numpy(), ref.dw_router)}
        print(f"  head={head}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        for name, v in errs.items():
            assert v <= TOL, name
        empty = np.nonzero(r.count == 0)[0]
        for t in (dwg, dwu, dwd, dwr):
            assert not t[torch.from_numpy(empty).to(DEV)].any()
    if cfg.name == "bwdmx_sparse":
        assert (r.count == 0).sum() > 0
    first = ml.run(0)
    for _ in range(2):
        for a, b2 in zip(first, ml.run(0)):
            assert torch.equal(a, b2)


def test_backward_mx_full_size_sampled():
    """The skewed 8,192-token workload in MXFP8 (d 4096, 512 experts, k 10, f 1024): weight
    gradients of the hottest, the coldest and two more experts, dW_r rows and dx of three
    tokens against the oracle; a second run bitwise equal."""
    cfg = SKEW_BWD.with_(name="skew_bwd_mx_t8192", dtype="mxfp8")
    print(f"\n[case] MXFP8 backward full size {cfg.name}", flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = to_oracle(inp.b_router)
    dy = to_oracle(inp.dy)
    r = oracle.route(x, w_r, b, cfg.k)
    ml = MxLayer(cfg, inp)
    head = cfg.C - cfg.n // 2
    disp = oracle.dispatch(r.idx, cfg.E, cfg.C, head)
    dx, dwg, dwu, dwd, dwr = ml.run(head)
    np.testing.assert_array_equal(ml.layer.bufs["topk_idx"].cpu().numpy(), r.idx)
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down)
    order = np.argsort(r.count)
    cold = [int(e) for e in order if r.count[e] > 0][:2]
    experts = sorted({int(order[-1]), *cold, 7})
    check_backward_weights(ml, experts[:2])
    grads = {}
    for e in experts:
        eg = oracle.expert_backward_mx(e, x, dy, r, lw, disp)
        grads[e] = eg
        errs = [rel(to_oracle(t[e]), ref) for t, ref in ((dwg, eg.dw_gate), (dwu, eg.dw_up), (dwd, eg.dw_down))]
        print(f"  expert {e} ({r.count[e]} rows): dW rel {errs}", flush=True)
        assert max(errs) <= TOL
    # dx and dl of three tokens: their k experts' copies (dg) and the router term
    toks = [0, 4095, 8191]
    need = sorted({int(e) for t in toks for e in r.idx[t]} - set(grads))
    for e in need:
        grads[e] = oracle.expert_backward_mx(e, x, dy, r, lw, disp)
    dxr = np.zeros((len(toks), cfg.d))
    for i, t in enumerate(toks):
        dg = np.zeros(cfg.k)
        for j, e in enumerate(r.idx[t]):
            eg = grads[int(e)]
            c = int(np.nonzero((eg.tokens == t) & (eg.js == j))[0][0])
            dg[j] = eg.dg[c]
            dxr[i] += eg.dx[c]
        dl = oracle.router_logit_grad(r.gate[t][None], dg[None])[0]
        for j, e in enumerate(r.idx[t]):
            dxr[i] += dl[j] * w_r[e]
    err = rel(to_oracle(dx[torch.tensor(toks, device=DEV)]), dxr)
    print(f"  dx tokens {toks}: rel {err:.2e}", flush=True)
    assert err <= TOL
    again = ml.run(head)
    for a, b2 in zip((dx, dwg, dwu, dwd, dwr), again):
        assert torch.equal(a, b2)
    del ml, inp
    torch.cuda.empty_cache()
