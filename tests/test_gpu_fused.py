"""GPU parity of the single-launch forward (moe_forward): every output bitwise equal to the
chained calls (route, dispatch, expert FFN, combine) where those run the same 128-row GEMM
tile, the fp64 oracle's tolerances everywhere, repeated calls bitwise identical, and the
barrier's give-up path forced from the host (a spin limit of one poll)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_33_amd as moe
import oracle
from gen import FWD_BF16, SKEW_BWD, LayerConfig, make_layer
from layer_util import LazyWeights, rel, to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"

OUTS = ["topk_idx", "topk_gate", "expert_count", "expert_offset", "copy_slot", "y"]
RING = ["ring_x", "ring_y", "saved_au"]

CASES = [
    LayerConfig("fu_bf16_ragged", T=300, d=384, E=16, k=4, f=192, cid=31),
    LayerConfig("fu_bf16_multitile", T=1000, d=512, E=64, k=6, f=256, cid=32),
    LayerConfig("fu_bf16_skew", T=512, d=256, E=32, k=4, f=128, zipf_s=1.1, hot_ratio=8.0, cid=33),
    LayerConfig("fu_bf16_router128", T=330, d=1152, E=160, k=4, f=128, cid=43),
    LayerConfig("fu_bf16_k1", T=257, d=256, E=16, k=1, f=128, cid=70),
    LayerConfig("fu_bf16_kE", T=130, d=256, E=6, k=6, f=192, cid=71),
    LayerConfig("fu_bf16_e1", T=190, d=320, E=1, k=1, f=128, cid=72),
]


def snapshot(layer):
    return {n: layer.bufs[n].clone() for n in OUTS + RING + ["slot_copy"] if n in layer.bufs}


def used_slots(cfg, head, idx):
    disp = oracle.dispatch(idx, cfg.E, cfg.C, head)
    return torch.from_numpy(np.nonzero(disp.slot_copy >= 0)[0]).to(DEV), disp


def assert_same(a, b, sl, names):
    for n in names:
        if n in RING:
            assert torch.equal(a[n][sl], b[n][sl]), n
        elif n == "slot_copy":
            assert torch.equal(a[n][sl], b[n][sl]), n
        else:
            assert torch.equal(a[n], b[n]), n


def run_both(cfg, inp, head):
    chained = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    chained.forward(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down, head=head,
                    save_au=True)
    fused = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    fused.forward_fused(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                        head=head, save_au=True)
    torch.cuda.synchronize()
    assert fused.forward_status() == 0
    return snapshot(chained), snapshot(fused), fused


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_fused_equals_chained_and_oracle(cfg):
    print(f"\n[case] fused forward {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}",
          flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    ref_r = oracle.route(x, w_r, b, cfg.k)
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down)
    for head in (0, cfg.C - cfg.n // 2):
        a, f, layer = run_both(cfg, inp, head)
        sl, disp = used_slots(cfg, head, ref_r.idx)
        assert_same(a, f, sl, OUTS + RING + ["slot_copy"])
        np.testing.assert_array_equal(f["topk_idx"].cpu().numpy(), ref_r.idx)
        np.testing.assert_array_equal(f["copy_slot"].cpu().numpy(), disp.copy_slot)
        fw = oracle.forward(x, w_r, b, cfg.k, lw, cfg.C, head)
        err = rel(to_oracle(f["y"]), fw.y)
        print(f"  head={head}: bitwise equal to the chained calls; y max-abs-rel {err:.3e}", flush=True)
        assert err <= 2e-2
    again = []
    for _ in range(3):
        layer.forward_fused(inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down,
                            head=0, save_au=True)
        torch.cuda.synchronize()
        again.append(snapshot(layer))
    sl, _ = used_slots(cfg, 0, ref_r.idx)
    for s in again[1:]:
        assert_same(again[0], s, sl, OUTS + RING + ["slot_copy"])


@pytest.mark.parametrize("cfg", [FWD_BF16, SKEW_BWD.with_(backward=False)], ids=lambda c: c.name)
def test_fused_full_size_equals_chained(cfg):
    """The benchmark's workloads: the one-launch forward against the chained calls, bitwise,
    both ring heads (segments wrap at C - n/2); y on sampled tokens against the oracle."""
    print(f"\n[case] fused forward full size {cfg.name}", flush=True)
    inp = make_layer(cfg, DEV)
    x, w_r = to_oracle(inp.x), to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    ref_r = oracle.route(x, w_r, b, cfg.k)
    for head in (0, cfg.C - cfg.n // 2):
        a, f, layer = run_both(cfg, inp, head)
        sl, _ = used_slots(cfg, head, ref_r.idx)
        assert_same(a, f, sl, OUTS + RING + ["slot_copy"])
        print(f"  head={head}: bitwise equal to the chained calls", flush=True)
    toks = [0, cfg.T // 2, cfg.T - 1]
    ref_y = oracle.forward_tokens(toks, x, ref_r, LazyWeights(inp.w_gate, inp.w_up, inp.w_down))
    err = rel(to_oracle(f["y"][torch.tensor(toks, device=DEV)]), ref_y)
    print(f"  tokens {toks}: y max-abs-rel {err:.3e}", flush=True)
    assert err <= 2e-2
    del inp, layer
    torch.cuda.empty_cache()


def test_fused_barrier_gives_up_and_recovers():
    """A spin limit of one poll makes the grid barriers give up: every workgroup ends, the
    status bit is set, and calls do nothing until the caller clears the barrier words;
    after that the call is whole again, bitwise the chained result."""
    cfg = LayerConfig("fu_giveup", T=200, d=256, E=8, k=2, f=128, cid=78)
    print(f"\n[case] fused forward barrier give-up {cfg.name}", flush=True)
    inp = make_layer(cfg, DEV)
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    args = (inp.x, inp.w_router, inp.b_router, inp.w_gate, inp.w_up, inp.w_down)
    layer.forward_fused(*args, spin_limit=1)
    torch.cuda.synchronize()
    assert layer.forward_status() & 1
    layer.bufs["y"].fill_(0)
    layer.forward_fused(*args)                 # the bit is set: this call does nothing
    torch.cuda.synchronize()
    assert not layer.bufs["y"].any()
    layer.bufs[f"ws{moe.OP_FORWARD}"][:256].zero_()
    layer.forward_fused(*args)
    torch.cuda.synchronize()
    assert layer.forward_status() == 0
    chained = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C)
    y = chained.forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(layer.bufs["y"], y)
