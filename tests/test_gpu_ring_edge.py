"""GPU parity at the largest ring the boundary accepts.

The grouped GEMMs address ring rows with 32-bit byte offsets and the boundary rejects
any ring array of 4 GiB or more.  These cases take the largest accepted capacity and a
head that wraps the copies' segment around the ring's end, so that the rows the kernels
read and write sit at the top of a ring just under 4 GiB, and compare the forward (bf16
and MXFP8, chained and single-launch) and the backward (bf16 and MXFP8) with the fp64
oracle as the medium-size tests do."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_33_amd as moe
import oracle
from gen import LayerConfig, make_layer
from layer_util import LazyWeights, rel, to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": 2e-2, "mxfp8": 6e-2}
D = 7168


def largest_ring(row_bytes):
    return ((1 << 32) - 1) // row_bytes


def test_bf16_forward_backward_at_the_largest_ring():
    cfg = LayerConfig("ring_edge_bf16", T=48, d=D, E=8, k=2, f=256, backward=True, cid=88)
    C = largest_ring(D * 2)                       # ring_x and ring_y just under 4 GiB
    n = cfg.n
    head = C - n // 2                              # the segment wraps past the last row
    print(f"\n[case] bf16 ring edge T={cfg.T} d={D} E={cfg.E} k={cfg.k} f={cfg.f} C={C} head={head}",
          flush=True)
    assert moe.make_shape(cfg.T, D, cfg.E, cfg.k, cfg.f, C).capacity * D * 2 < 1 << 32
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down)
    layer = moe.Layer.create(cfg.T, D, cfg.E, cfg.k, cfg.f, C)
    y = layer.forward(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                      head=head, save_au=True)
    torch.cuda.synchronize()
    r = oracle.route(x, w_r, b, cfg.k)
    np.testing.assert_array_equal(layer.bufs["topk_idx"].cpu().numpy(), r.idx)
    disp = oracle.dispatch(r.idx, cfg.E, C, head)
    np.testing.assert_array_equal(layer.bufs["copy_slot"].cpu().numpy(), disp.copy_slot)
    assert disp.copy_slot.max() == C - 1          # a copy sits in the ring's last row
    ref_y = oracle.forward_tokens(range(cfg.T), x, r, lw)   # per token: no ring of C rows
    err = rel(to_oracle(y), ref_y)
    print(f"  forward: y max-abs-rel {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    dx, dwg, dwu, dwd, dwr = layer.backward(inp.dy, inp.x, inp.w_router, inp.w_gate, inp.w_up,
                                            inp.w_down, head=head)
    torch.cuda.synchronize()
    W = oracle.weights_from_arrays(*(to_oracle(w) for w in (inp.w_gate, inp.w_up, inp.w_down)))
    ref = oracle.backward(x, w_r, r, W, to_oracle(inp.dy))
    errs = {"dx": rel(to_oracle(dx), ref.dx), "dw_gate": rel(to_oracle(dwg), ref.dw_gate),
            "dw_up": rel(to_oracle(dwu), ref.dw_up), "dw_down": rel(to_oracle(dwd), ref.dw_down),
            "dw_router": rel(dwr.cpu().numpy(), ref.dw_router)}
    print("  backward: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for name, v in errs.items():
        assert v <= TOL["bf16"], name
    del layer, inp
    torch.cuda.empty_cache()


def test_mxfp8_forward_at_the_largest_ring():
    cfg = LayerConfig("ring_edge_mx", T=48, d=D, E=8, k=2, f=256, dtype="mxfp8", cid=89)
    C = largest_ring(D)                           # one byte per code: ring_x just under 4 GiB
    n = cfg.n
    head = C - n // 2
    print(f"\n[case] MXFP8 ring edge T={cfg.T} d={D} E={cfg.E} k={cfg.k} f={cfg.f} C={C} head={head}",
          flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down, mx_codes=tuple(q))
    layer = moe.Layer.create(cfg.T, D, cfg.E, cfg.k, cfg.f, C, dtype="mxfp8")
    y = layer.forward(inp.x, inp.w_router, inp.b_router, *[c for c, _ in q],
                      scales=tuple(s for _, s in q), head=head)
    torch.cuda.synchronize()
    r = oracle.route(x, w_r, b, cfg.k)
    np.testing.assert_array_equal(layer.bufs["topk_idx"].cpu().numpy(), r.idx)
    disp = oracle.dispatch(r.idx, cfg.E, C, head)
    assert disp.copy_slot.max() == C - 1
    ref_y = oracle.forward_tokens(range(cfg.T), x, r, lw, mx_path=True)
    err = rel(to_oracle(y), ref_y)
    print(f"  forward: y max-abs-rel {err:.3e}", flush=True)
    assert err <= TOL["mxfp8"]
    del layer, inp
    torch.cuda.empty_cache()


def test_fused_forward_at_the_largest_ring():
    """The single-launch forward at the largest bf16 ring: bitwise the chained calls' y and
    ring rows, and the oracle's y."""
    cfg = LayerConfig("ring_edge_fused", T=48, d=D, E=8, k=2, f=256, cid=88)
    C = largest_ring(D * 2)
    head = C - cfg.n // 2
    print(f"\n[case] fused ring edge T={cfg.T} d={D} E={cfg.E} k={cfg.k} f={cfg.f} C={C} head={head}",
          flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    args = (inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down)
    chained = moe.Layer.create(cfg.T, D, cfg.E, cfg.k, cfg.f, C)
    y_c = chained.forward(*args, head=head).clone()
    fused = moe.Layer.create(cfg.T, D, cfg.E, cfg.k, cfg.f, C)
    y_f = fused.forward_fused(*args, head=head)
    torch.cuda.synchronize()
    assert fused.forward_status() == 0
    assert torch.equal(y_c, y_f)
    r = oracle.route(x, w_r, b, cfg.k)
    disp = oracle.dispatch(r.idx, cfg.E, C, head)
    used = torch.from_numpy(np.nonzero(disp.slot_copy >= 0)[0]).to(DEV)
    assert int(used.max()) == C - 1
    for name in ("ring_x", "ring_y"):
        assert torch.equal(chained.bufs[name][used], fused.bufs[name][used]), name
    err = rel(to_oracle(y_f), oracle.forward_tokens(range(cfg.T), x, r, LazyWeights(inp.w_gate, inp.w_up, inp.w_down)))
    print(f"  bitwise equal to the chained calls; y max-abs-rel {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    del chained, fused, inp
    torch.cuda.empty_cache()


def test_mxfp8_backward_at_the_largest_ring():
    """The MXFP8 backward at the largest MX ring (codes just under 4 GiB; its bf16 ring-order
    work arrays are twice that): gradients against the oracle's backward_mx."""
    cfg = LayerConfig("ring_edge_bwd_mx", T=48, d=D, E=8, k=2, f=256, dtype="mxfp8",
                      backward=True, cid=89)
    C = largest_ring(D)
    head = C - cfg.n // 2
    print(f"\n[case] MXFP8 backward ring edge T={cfg.T} d={D} E={cfg.E} k={cfg.k} f={cfg.f} C={C} "
          f"head={head}", flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    bw = moe.quantize_mx_t_backward_weights(inp.w_gate, inp.w_up, inp.w_down)
    layer = moe.Layer.create(cfg.T, D, cfg.E, cfg.k, cfg.f, C, dtype="mxfp8")
    layer.forward(inp.x, inp.w_router, inp.b_router, *[c for c, _ in q],
                  scales=tuple(s for _, s in q), head=head, save_au=True)
    dx, dwg, dwu, dwd, dwr = layer.backward_mx(inp.dy, inp.x, inp.w_router, *bw, head=head)
    torch.cuda.synchronize()
    r = oracle.route(x, w_r, b, cfg.k)
    np.testing.assert_array_equal(layer.bufs["topk_idx"].cpu().numpy(), r.idx)
    disp = oracle.dispatch(r.idx, cfg.E, C, head)
    assert disp.copy_slot.max() == C - 1
    W = oracle.weights_from_arrays(*(to_oracle(w) for w in (inp.w_gate, inp.w_up, inp.w_down)))
    ref = oracle.backward_mx(x, w_r, r, W, to_oracle(inp.dy), disp)
    errs = {"dx": rel(to_oracle(dx), ref.dx), "dw_gate": rel(to_oracle(dwg), ref.dw_gate),
            "dw_up": rel(to_oracle(dwu), ref.dw_up), "dw_down": rel(to_oracle(dwd), ref.dw_down),
            "dw_router": rel(dwr.cpu().numpy(), ref.dw_router)}
    print("  backward: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for name, v in errs.items():
        assert v <= TOL["mxfp8"], name
    del layer, inp
    torch.cuda.empty_cache()
