"""GPU parity of the forward path through the C ABI against the fp64 oracle.

Routing indices, counts, the dispatch permutation and the ring contents are
compared bit for bit; outputs within max|gpu - ref| / max|ref| of 1e-5 (fp32),
2e-2 (bf16), 6e-2 (MXFP8); repeated runs must be bitwise identical."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_33_amd as moe
import oracle
from gen import (FWD_BF16, FWD_MXFP8, SHARE_BF16, SHARE_MXFP8, SKEW_BWD, TINY_F32, LayerConfig,
                 make_layer, make_share)
from layer_util import LazyWeights, mx_scale_rows, rel, to_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2}
DEV = "cuda"

MEDIUM = [
    TINY_F32,
    # f32 with widths off every tile multiple
    LayerConfig("med_f32", T=150, d=200, E=12, k=3, f=72, dtype="f32", cid=30),
    # bf16: f = 192 leaves a half-filled gate/up tile, d = 384 a half-filled down tile
    LayerConfig("med_bf16_ragged", T=300, d=384, E=16, k=4, f=192, cid=31),
    # bf16: ~94 rows per expert on average, so many experts take two row tiles
    LayerConfig("med_bf16_multitile", T=1000, d=512, E=64, k=6, f=256, cid=32),
    # bf16 with a skewed router bias: hot experts span several row tiles
    LayerConfig("med_bf16_skew", T=512, d=256, E=32, k=4, f=128, zipf_s=1.1, hot_ratio=8.0, cid=33),
    LayerConfig("med_mx", T=300, d=256, E=16, k=4, f=256, dtype="mxfp8", cid=34),
    LayerConfig("med_mx_skew", T=400, d=384, E=24, k=3, f=128, dtype="mxfp8", zipf_s=1.1,
                hot_ratio=6.0, cid=35),
    # more than 96 rows per expert on average: the 128-row tile shape (the cases above
    # take the 64-row one); ragged last row tiles
    LayerConfig("med_bf16_bigtile", T=600, d=320, E=8, k=2, f=192, cid=36),
    LayerConfig("med_mx_bigtile", T=700, d=256, E=6, k=2, f=256, dtype="mxfp8", cid=37),
    # at least 256 rows per expert on average: the bf16 256 x 256 tile with 64-byte K
    # slices; ragged in rows, columns and K
    LayerConfig("med_bf16_big256", T=1100, d=320, E=8, k=2, f=192, cid=38),
    # d = 1984 = 31 K slices of 64 and only 4 token tiles: the bf16 router splits K over
    # 3 workgroups (10, 10 and 11 slices) whose partial logit planes are added in order
    LayerConfig("med_bf16_ksplit", T=200, d=1984, E=40, k=4, f=128, cid=39),
    # at least two row tiles per expert (the regime of the per-GPU share shapes: K-start
    # rotation on in both GEMMs); bf16 256-row tiles, then MX 128-row tiles
    LayerConfig("med_bf16_tail", T=2600, d=320, E=4, k=2, f=192, cid=40),
    LayerConfig("med_mx_tail", T=1500, d=256, E=4, k=2, f=256, dtype="mxfp8", cid=41),
    # 160 experts: the router's 128 x 128 tile, the second expert tile a quarter full, the
    # last token tile ragged, and K (18 slices of 64) split over 2 workgroups
    LayerConfig("med_bf16_router128", T=330, d=1152, E=160, k=4, f=128, cid=43),
    # MX with at least 256 rows per expert: the 256 x 256 eight-wave tile; ragged rows, the
    # down GEMM's second column tile half full
    LayerConfig("med_mx_big256", T=1400, d=384, E=4, k=2, f=384, dtype="mxfp8", cid=44),
    # the method's degenerate cases: k = 1 (one expert per token, every gate 1), k = E
    # (every expert selected, gates = the full softmax) and E = 1 (a dense SwiGLU FFN)
    LayerConfig("med_bf16_k1", T=257, d=256, E=16, k=1, f=128, cid=70),
    LayerConfig("med_bf16_kE", T=130, d=256, E=6, k=6, f=192, cid=71),
    LayerConfig("med_bf16_e1", T=190, d=320, E=1, k=1, f=128, cid=72),
    LayerConfig("med_mx_k1", T=257, d=256, E=16, k=1, f=128, dtype="mxfp8", cid=73),
    LayerConfig("med_mx_kE", T=100, d=256, E=5, k=5, f=256, dtype="mxfp8", cid=74),
    LayerConfig("med_mx_e1", T=150, d=384, E=1, k=1, f=256, dtype="mxfp8", cid=75),
    LayerConfig("med_f32_kE", T=40, d=64, E=4, k=4, f=32, dtype="f32", cid=76),
]


def run_forward(layer, inp, head, scales, wq):
    y = layer.forward(inp.x, inp.w_router, inp.b_router, *wq, scales=scales, head=head)
    torch.cuda.synchronize()
    b = layer.bufs
    return {n: b[n].clone() for n in ["topk_idx", "topk_gate", "expert_count", "expert_offset",
                                       "copy_slot", "slot_copy", "ring_x", "ring_y"]
            if n in b} | ({"ring_x_scale": b["ring_x_scale"].clone()} if "ring_x_scale" in b else {}) | {"y": y.clone()}


def quantized_weights(inp, mx):
    if not mx:
        return (inp.w_gate, inp.w_up, inp.w_down), (None, None, None), None
    q = [moe.quantize_mx(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    return tuple(c for c, _ in q), tuple(s for _, s in q), q


def oracle_inputs(inp):
    x = to_oracle(inp.x)
    w_r = to_oracle(inp.w_router)
    b = None if inp.b_router is None else to_oracle(inp.b_router)
    return x, w_r, b


@pytest.mark.parametrize("cfg", MEDIUM, ids=lambda c: c.name)
def test_forward_parity(cfg):
    print(f"\n[case] forward parity {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} "
          f"{cfg.dtype}", flush=True)
    inp = make_layer(cfg, DEV)
    mx = cfg.dtype == "mxfp8"
    wq, scales, q = quantized_weights(inp, mx)
    x, w_r, b = oracle_inputs(inp)
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down,
                     mx_codes=tuple(q) if mx else None)
    if mx:   # the device quantiser matches the oracle's encoder bit for bit
        for e in range(cfg.E):
            for (c, s), (oc, os_) in zip([(c[e], s[e]) for c, s in lw.mx], lw.oracle_mx(e)):
                np.testing.assert_array_equal(c.cpu().numpy(), oc)
                np.testing.assert_array_equal(s.cpu().numpy(), os_)
    ref_r = oracle.route(x, w_r, b, cfg.k)
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype=cfg.dtype)
    n = cfg.n
    for head in (0, cfg.C - n // 2):
        out = run_forward(layer, inp, head, scales, wq)
        # router: bit-exact selection and counts, gates to fp32 accuracy
        np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), ref_r.idx)
        np.testing.assert_array_equal(out["expert_count"].cpu().numpy(), ref_r.count)
        assert rel(out["topk_gate"].cpu().numpy(), ref_r.gate) <= 1e-5   # fp32 router output
        # dispatch: bit-exact permutation and offsets
        disp = oracle.dispatch(ref_r.idx, cfg.E, cfg.C, head)
        np.testing.assert_array_equal(out["expert_offset"].cpu().numpy(), disp.offset)
        np.testing.assert_array_equal(out["copy_slot"].cpu().numpy(), disp.copy_slot)
        used = disp.slot_copy >= 0
        np.testing.assert_array_equal(out["slot_copy"].cpu().numpy()[used], disp.slot_copy[used])
        # ring contents: x rows (or their MX codes) bit for bit
        cs = disp.copy_slot
        ring = out["ring_x"]
        if mx:
            xc, xs = oracle.mx.quantize(x, axis=1)
            for j in range(cfg.k):
                np.testing.assert_array_equal(ring[torch.from_numpy(cs[:, j]).to(DEV)].cpu().numpy(), xc)
                np.testing.assert_array_equal(
                    mx_scale_rows(out["ring_x_scale"])[torch.from_numpy(cs[:, j]).to(DEV)].cpu().numpy(), xs)
        else:
            for j in range(cfg.k):
                got = ring[torch.from_numpy(cs[:, j]).to(DEV)]
                assert torch.equal(got, inp.x), f"ring rows of copy {j} differ from x"
        # expert FFN and combine
        fw = oracle.forward(x, w_r, b, cfg.k, lw, cfg.C, head, mx_path=mx)
        ry = to_oracle(out["ring_y"])
        assert rel(ry[used], fw.ring_y[used]) <= TOL[cfg.dtype]
        err = rel(to_oracle(out["y"]), fw.y)
        print(f"  head={head}: y max-abs-rel {err:.3e}", flush=True)
        assert err <= TOL[cfg.dtype]
    # determinism: repeated runs are bitwise identical
    first = run_forward(layer, inp, 0, scales, wq)
    for _ in range(4):
        again = run_forward(layer, inp, 0, scales, wq)
        for name, t in first.items():
            if name in ("ring_x", "ring_y", "ring_x_scale"):
                sl = torch.from_numpy(np.nonzero(oracle.dispatch(ref_r.idx, cfg.E, cfg.C, 0).slot_copy >= 0)[0]).to(DEV)
                a, b = t, again[name]
                if name == "ring_x_scale":   # [d/128][C][4] -> rows [C, d/32] before slot indexing
                    a, b = mx_scale_rows(a), mx_scale_rows(b)
                assert torch.equal(a[sl], b[sl]), name
            else:
                assert torch.equal(t, again[name]), name


@pytest.mark.parametrize("cfg", [FWD_BF16, FWD_MXFP8, SKEW_BWD.with_(backward=False)],
                         ids=lambda c: c.name)
def test_forward_full_size_sampled(cfg):
    """Full workload sizes in the benchmark's launch configuration; routing and dispatch
    checked everywhere, expert outputs on sampled experts, y on sampled tokens."""
    print(f"\n[case] full-size forward {cfg.name}", flush=True)
    inp = make_layer(cfg, DEV)
    mx = cfg.dtype == "mxfp8"
    wq, scales, q = quantized_weights(inp, mx)
    x, w_r, b = oracle_inputs(inp)
    ref_r = oracle.route(x, w_r, b, cfg.k)
    layer = moe.Layer.create(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, dtype=cfg.dtype)
    head = cfg.C - cfg.n // 2          # segments wrap around the ring end
    out = run_forward(layer, inp, head, scales, wq)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), ref_r.idx)
    np.testing.assert_array_equal(out["expert_count"].cpu().numpy(), ref_r.count)
    assert rel(out["topk_gate"].cpu().numpy(), ref_r.gate) <= 1e-5   # fp32 router output
    disp = oracle.dispatch(ref_r.idx, cfg.E, cfg.C, head)
    np.testing.assert_array_equal(out["expert_offset"].cpu().numpy(), disp.offset)
    np.testing.assert_array_equal(out["copy_slot"].cpu().numpy(), disp.copy_slot)
    used = disp.slot_copy >= 0
    np.testing.assert_array_equal(out["slot_copy"].cpu().numpy()[used], disp.slot_copy[used])
    lw = LazyWeights(inp.w_gate, inp.w_up, inp.w_down, mx_codes=tuple(q) if mx else None)
    rng = np.random.default_rng(0)
    hot = int(np.argmax(ref_r.count))
    experts = sorted({hot, int(np.argmin(np.where(ref_r.count > 0, ref_r.count, 1 << 30))),
                      *map(int, rng.choice(cfg.E, 2, replace=False))})
    ring_y = out["ring_y"]
    for e in experts:
        if mx:
            for (c, s), (oc, os_) in zip([(c[e], s[e]) for c, s in lw.mx], lw.oracle_mx(e)):
                np.testing.assert_array_equal(c.cpu().numpy(), oc)
                np.testing.assert_array_equal(s.cpu().numpy(), os_)
        slots = oracle.segment_slots(disp, e)
        if slots.size == 0:
            continue
        toks = disp.slot_copy[slots] // cfg.k
        xe = oracle.mx.fake_quant(x[toks], axis=1) if mx else x[toks]
        if mx:
            xc, xs = oracle.mx.quantize(x[toks], axis=1)
            sl = torch.from_numpy(slots).to(DEV)
            np.testing.assert_array_equal(layer.bufs["ring_x"][sl].cpu().numpy(), xc)
            np.testing.assert_array_equal(mx_scale_rows(layer.bufs["ring_x_scale"])[sl].cpu().numpy(), xs)
        ref = oracle.swiglu(xe, *lw(e), h_mx=mx)
        got = to_oracle(ring_y[torch.from_numpy(slots).to(DEV)])
        err = rel(got, ref)
        print(f"  expert {e} ({slots.size} rows): ring_y max-abs-rel {err:.3e}", flush=True)
        assert err <= TOL[cfg.dtype]
    toks = sorted(map(int, rng.choice(cfg.T, 3, replace=False)))
    ref_y = oracle.forward_tokens(toks, x, ref_r, lw, mx_path=mx)
    err = rel(to_oracle(out["y"][torch.tensor(toks, device=DEV)]), ref_y)
    print(f"  tokens {toks}: y max-abs-rel {err:.3e}", flush=True)
    assert err <= TOL[cfg.dtype]
    again = run_forward(layer, inp, head, scales, wq)
    assert torch.equal(again["y"], out["y"]) and torch.equal(again["topk_gate"], out["topk_gate"])
    sl = torch.from_numpy(np.nonzero(used)[0]).to(DEV)
    assert torch.equal(again["ring_y"][sl], out["ring_y"][sl])
    del layer, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scfg", [SHARE_BF16, SHARE_MXFP8], ids=lambda c: c.name)
def test_share_shape_sampled(scfg):
    """The grouped GEMMs at one GPU's expert-parallel share (4 experts x 16,384 rows),
    in the launch configuration the benchmark times; sampled rows of every expert."""
    print(f"\n[case] share-shape expert FFN {scfg.name}", flush=True)
    sh = make_share(scfg, DEV)
    mx = scfg.dtype == "mxfp8"
    shape = moe.make_shape(scfg.rows, scfg.d, scfg.E, 1, scfg.f, scfg.C, dtype=scfg.dtype)
    off = torch.tensor(np.concatenate([[0], np.cumsum(sh.counts)]), dtype=torch.int32, device=DEV)
    ws = moe.workspace(shape, moe.OP_EXPERT_FFN, DEV)
    ring_y = torch.empty((scfg.C, scfg.d), dtype=torch.bfloat16, device=DEV)
    if mx:
        xq, xs = moe.quantize_mx(sh.ring_x)
        q = [moe.quantize_mx(w) for w in (sh.w_gate, sh.w_up, sh.w_down)]
        wargs = [c for c, _ in q] + [s for _, s in q]
    else:
        xq, xs, q = sh.ring_x, None, None
        wargs = [sh.w_gate, sh.w_up, sh.w_down, None, None, None]
    moe.moe_expert_ffn(shape, xq, xs, off, 0, *wargs, ring_y, None, ws)
    torch.cuda.synchronize()
    lw = LazyWeights(sh.w_gate, sh.w_up, sh.w_down, mx_codes=tuple(q) if mx else None)
    rng = np.random.default_rng(1)
    offs = off.cpu().numpy()
    for e in range(scfg.E):
        rows = np.sort(rng.choice(np.arange(offs[e], offs[e + 1]), 6, replace=False))
        rows = np.unique(np.concatenate([rows, [offs[e], offs[e + 1] - 1]]))
        x = to_oracle(sh.ring_x[torch.from_numpy(rows).to(DEV)])
        xe = oracle.mx.fake_quant(x, axis=1) if mx else x
        ref = oracle.swiglu(xe, *lw(e), h_mx=mx)
        err = rel(to_oracle(ring_y[torch.from_numpy(rows).to(DEV)]), ref)
        print(f"  expert {e}: rows {rows.tolist()} max-abs-rel {err:.3e}", flush=True)
        assert err <= TOL[scfg.dtype]
    again = torch.empty_like(ring_y)
    moe.moe_expert_ffn(shape, xq, xs, off, 0, *wargs, again, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(again[: scfg.rows], ring_y[: scfg.rows])
