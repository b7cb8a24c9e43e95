"""Pins of the fp64 oracle against things other than itself: hand-derived closed forms,
a per-token brute force, library routines, the E4M3 format definition, finite
differences, torch autograd, and invariants of the method.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mx
from gen import TINY_F32, LayerConfig, make_layer, topk_gap, zipf_targets
from gen.inputs import calibrate_bias, draw_router_and_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, T, d, E, k, f, bias=False, margin=1e-3):
    """Small random fp64 layer whose routing has a clear k/(k+1) gap."""
    w_r = rng.standard_normal((E, d)) / math.sqrt(d)
    b = rng.standard_normal(E) * 0.3 if bias else None
    x = rng.standard_normal((T, d))
    for _ in range(100):
        l = x @ w_r.T + (0 if b is None else b)
        bad = np.nonzero(topk_gap(l, k) < margin)[0]
        if bad.size == 0:
            break
        x[bad] = rng.standard_normal((bad.size, d))
    wg = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, f)) / math.sqrt(f)
    return x, w_r, b, wg, wu, wd


# ----------------------------------------------------------------- closed forms (golden)


def load_cases():
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_closed_form_forward(case):
    x = np.array(case["x"])
    w_r = np.array(case["w_router"])
    W = oracle.weights_from_arrays(np.array(case["w_gate"]), np.array(case["w_up"]),
                                   np.array(case["w_down"]))
    k = case["k"]
    fw = oracle.forward(x, w_r, None, k, W, C=x.shape[0] * k)
    assert fw.routing.idx.tolist() == case["idx"]
    np.testing.assert_allclose(fw.routing.gate, case["gate"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(fw.y, case["y"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_closed_form_backward(case):
    x = np.array(case["x"])
    w_r = np.array(case["w_router"])
    wg, wu, wd = (np.array(case[n]) for n in ("w_gate", "w_up", "w_down"))
    W = oracle.weights_from_arrays(wg, wu, wd)
    r = oracle.route(x, w_r, None, case["k"])
    bw = oracle.backward(x, w_r, r, W, np.array(case["dy"]))
    np.testing.assert_allclose(bw.dw_router, case["dw_router"], rtol=0, atol=1e-15)
    if "dl" in case:
        np.testing.assert_allclose(bw.dl, case["dl"], rtol=0, atol=1e-15)
    if "dx" in case:
        np.testing.assert_allclose(bw.dx, case["dx"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(bw.dw_gate[0], case["dw_gate0"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(bw.dw_up[0], case["dw_up0"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(bw.dw_down[0], case["dw_down0"], rtol=0, atol=1e-14)
        # expert 1 was never selected: its weight gradients are exactly zero
        assert not bw.dw_gate[1].any() and not bw.dw_down[1].any()


# ----------------------------------------------------------------- E4M3 / MX (format definition)


def read_spec_points():
    pts = []
    with open(os.path.join(GOLDEN, "e4m3_spec_points.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()[:2]
                pts.append((float(v), int(c, 16)))
    return pts


def test_e4m3_spec_points():
    for v, c in read_spec_points():
        assert int(mx.encode_e4m3(np.array([v]))[0]) == c, (v, hex(c))
        assert mx.DECODE_TABLE[c] == v


def test_e4m3_table_shape():
    vals = mx.POS_VALUES
    assert vals.size == 127 and np.all(np.diff(vals) > 0)
    assert vals[-1] == 448.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    assert math.isnan(mx.DECODE_TABLE[0x7F]) and math.isnan(mx.DECODE_TABLE[0xFF])


def test_e4m3_against_torch_float8():
    """torch's float8_e4m3fn is an independent encoder; inside +-448 it rounds to nearest even."""
    codes = torch.tensor(mx.POS_VALUES, dtype=torch.float32).to(torch.float8_e4m3fn)
    assert codes.view(torch.uint8).tolist() == list(range(127))
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
        # exact midpoints between neighbours: the tie rule decides
        0.5 * (mx.POS_VALUES[1:] + mx.POS_VALUES[:-1]),
        -0.5 * (mx.POS_VALUES[1:] + mx.POS_VALUES[:-1]),
    ]).astype(np.float32)
    ours = mx.encode_e4m3(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch gives 0x00 for a negative value that rounds to zero; the oracle keeps the sign
    ref = np.where((ref == 0) & np.signbit(v), 0x80, ref)
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates():
    # torch's plain cast gives NaN here; the MX rule clamps to +-448 before rounding
    got = mx.encode_e4m3(np.array([449.0, 470.0, 500.0, 1e6, -470.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_mx_scale_rule():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    v[3, 32:64] = 0.0                                   # an all-zero block
    codes, scales = mx.quantize(v, axis=1)
    blk = np.abs(v).reshape(64, 8, 32).max(axis=2)
    X = scales.astype(np.int64) - 127
    nz = blk > 0
    # amax / 2^X lands in [256, 512): the block maximum uses the top E4M3 binade
    r = blk[nz] / np.exp2(X[nz])
    assert np.all((r >= 256) & (r < 512))
    assert np.all(X[nz] == np.floor(np.log2(blk[nz])) - 8)
    assert scales[3, 1] == 0 and not (codes[3, 32:64] & 0x7F).any()
    # dequantisation error: half an E4M3 step, or the saturation gap at the top binade
    deq = mx.dequantize(codes, scales, axis=1)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))) - 3)
    sub = np.exp2(X - 9)[:, np.repeat(np.arange(8), 32)]
    bound = np.maximum(0.5 * step, 0.5 * sub)
    sat = np.abs(v) / np.exp2(X)[:, np.repeat(np.arange(8), 32)] > 448
    err = np.abs(deq - v)
    assert np.all(err[~sat] <= bound[~sat] * (1 + 1e-12))
    assert np.all(err[sat] <= 64 * np.exp2(X)[:, np.repeat(np.arange(8), 32)][sat])


def test_mx_idempotent():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((16, 128))
    c, s = mx.quantize(v, axis=1)
    c2, s2 = mx.quantize(mx.dequantize(c, s, axis=1), axis=1)
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(s, s2)


def test_mx_axis0_equals_transposed_axis1():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((64, 40))
    c0, s0 = mx.quantize(v, axis=0)
    c1, s1 = mx.quantize(v.T, axis=1)
    np.testing.assert_array_equal(c0, c1.T)
    np.testing.assert_array_equal(s0, s1.T)


# ----------------------------------------------------------------- router


def test_router_against_library_and_closed_form():
    rng = np.random.default_rng(5)
    x, w_r, b, *_ = rand_layer(rng, 64, 32, 16, 4, 8, bias=True)
    r = oracle.route(x, w_r, b, 4)
    l = x @ w_r.T + b
    # the selected set is the top of a full library argsort
    lib = np.sort(np.argsort(l, axis=1)[:, ::-1][:, :4], axis=1)
    np.testing.assert_array_equal(r.idx, lib)
    # renormalising the softmax over the selected set equals a softmax of the selected logits
    lS = np.take_along_axis(l, r.idx, axis=1)
    z = np.exp(lS - lS.max(axis=1, keepdims=True))
    np.testing.assert_allclose(r.gate, z / z.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
    assert np.max(np.abs(r.gate.sum(axis=1) - 1)) <= 1e-15 * 4
    np.testing.assert_array_equal(r.count, np.bincount(r.idx.ravel(), minlength=16))
    assert np.all(np.diff(r.idx, axis=1) > 0)


def test_router_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((10, 12))
    w_r = rng.standard_normal((6, 12))
    r = oracle.route(x, w_r, None, 6)
    np.testing.assert_array_equal(r.idx, np.tile(np.arange(6), (10, 1)))
    sm = torch.softmax(torch.from_numpy(x @ w_r.T), dim=1).numpy()
    np.testing.assert_allclose(r.gate, sm, rtol=1e-13, atol=0)


def test_router_ties_go_to_lower_id():
    x = np.ones((1, 2))
    w_r = np.array([[0.0, 1.0], [1.0, 0.0], [0.5, 0.5], [0.0, 0.0]])   # logits 1, 1, 1, 0
    r = oracle.route(x, w_r, None, 2)
    assert r.idx.tolist() == [[0, 1]]


# ----------------------------------------------------------------- dispatch


def test_dispatch_against_tuple_sort_and_invariants():
    rng = np.random.default_rng(7)
    T, E, k = 50, 7, 3
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    n = T * k
    for C, head in [(n, 0), (int(1.25 * n) + 1, 0), (int(1.25 * n) + 1, int(1.25 * n) + 1 - n // 2)]:
        disp = oracle.dispatch(idx, E, C, head)
        # textbook: sort the (expert, token) keys, position = rank
        order = sorted(((idx[t, j], t, j) for t in range(T) for j in range(k)))
        for rank, (_, t, j) in enumerate(order):
            assert disp.copy_slot[t, j] == (head + rank) % C
        np.testing.assert_array_equal(np.diff(disp.offset), np.bincount(idx.ravel(), minlength=E))
        assert disp.offset[-1] == n
        used = np.sort(disp.copy_slot.ravel())
        np.testing.assert_array_equal(used, np.sort((head + np.arange(n)) % C))
        # round trip: ring[copy_slot[t, j]] == x[t]
        x = rng.standard_normal((T, 5))
        ring = oracle.ring_fill(x, disp)
        for j in range(k):
            np.testing.assert_array_equal(ring[disp.copy_slot[:, j]], x)
        # inverse permutation
        for s in range(C):
            c = disp.slot_copy[s]
            if c >= 0:
                assert disp.copy_slot.ravel()[c] == s
        # each segment holds only its expert, in ascending token order
        for e in range(E):
            cps = disp.slot_copy[oracle.segment_slots(disp, e)]
            assert np.all(idx.ravel()[cps] == e) and np.all(np.diff(cps // k) > 0)


def test_dispatch_rejects_small_capacity():
    with pytest.raises(ValueError):
        oracle.dispatch(np.zeros((4, 1), dtype=np.int64), 2, 3)


# ----------------------------------------------------------------- forward


def test_tiny_workload_against_brute_force():
    """The tiny fp32 workload exactly as drawn: oracle layer == per-token brute force."""
    inp = make_layer(TINY_F32, "cpu")
    x = oracle.from_f32(inp.x.numpy())
    w_r = oracle.from_f32(inp.w_router.numpy())
    W = oracle.weights_from_arrays(*(oracle.from_f32(t.numpy()) for t in (inp.w_gate, inp.w_up, inp.w_down)))
    cfg = TINY_F32
    fw = oracle.forward(x, w_r, None, cfg.k, W, cfg.C)
    bf = oracle.brute_force(x, w_r, None, cfg.k, W)
    np.testing.assert_allclose(fw.y, bf, rtol=0, atol=1e-12 * np.abs(bf).max())
    assert np.all(topk_gap(fw.routing.logits, cfg.k) >= cfg.margin)


@pytest.mark.parametrize("shape", [(9, 16, 5, 2, 8, False), (13, 8, 6, 3, 16, True),
                                   (7, 32, 4, 4, 8, False), (20, 16, 9, 1, 24, True)])
def test_random_layers_against_brute_force(shape):
    T, d, E, k, f, bias = shape
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias)
    W = oracle.weights_from_arrays(wg, wu, wd)
    C = int(math.ceil(1.25 * T * k))
    for head in (0, C - 1, C - T * k // 2):
        fw = oracle.forward(x, w_r, b, k, W, C, head)
        bf = oracle.brute_force(x, w_r, b, k, W)
        np.testing.assert_allclose(fw.y, bf, rtol=0, atol=1e-12 * np.abs(bf).max())
    np.testing.assert_allclose(oracle.forward_tokens(range(T), x, fw.routing, W), fw.y,
                               rtol=0, atol=1e-13 * np.abs(bf).max())


def test_single_expert_is_dense_swiglu():
    """E = 1, k = 1: the layer reduces to a dense SwiGLU FFN (torch's silu as the check)."""
    rng = np.random.default_rng(8)
    x, w_r, _, wg, wu, wd = rand_layer(rng, 12, 16, 1, 1, 24)
    fw = oracle.forward(x, w_r, None, 1, oracle.weights_from_arrays(wg, wu, wd), 12)
    X, Wg, Wu, Wd = (torch.from_numpy(a) for a in (x, wg[0], wu[0], wd[0]))
    ref = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    np.testing.assert_allclose(fw.y, ref.numpy(), rtol=1e-13, atol=1e-14)
    assert np.all(fw.routing.gate == 1.0)


def test_combine_k1_and_linearity():
    rng = np.random.default_rng(9)
    ring_y = rng.standard_normal((10, 4))
    slot = rng.permutation(10)[:6].reshape(6, 1)
    np.testing.assert_array_equal(oracle.combine(ring_y, slot, np.ones((6, 1))), ring_y[slot[:, 0]])
    slot2 = np.stack([rng.permutation(10)[:2] for _ in range(6)])
    g1, g2 = rng.random((6, 2)), rng.random((6, 2))
    np.testing.assert_allclose(oracle.combine(ring_y, slot2, 2 * g1 + 3 * g2),
                               2 * oracle.combine(ring_y, slot2, g1) + 3 * oracle.combine(ring_y, slot2, g2),
                               rtol=1e-13, atol=1e-13)


def test_mx_forward_on_exactly_representable_values_equals_plain():
    """When x, W and H are already MX-representable, the MX path equals the plain one;
    the check is the brute force on values built from the E4M3 table."""
    rng = np.random.default_rng(10)
    T, d, E, k, f = 6, 32, 3, 2, 32
    x, w_r, _, wg, wu, wd = rand_layer(rng, T, d, E, k, f)
    x = mx.fake_quant(x, axis=1)
    wg, wu, wd = (mx.fake_quant(w, axis=-1) for w in (wg, wu, wd))
    W = oracle.weights_from_arrays(wg, wu, wd)
    fm = oracle.forward(x, w_r, None, k, W, T * k, mx_path=True)
    fp = oracle.forward(x, w_r, None, k, W, T * k, mx_path=False)
    # only H differs (it is re-quantised in the MX path); its relative change is bounded
    assert oracle.max_abs_rel(fm.y, fp.y) < 0.1
    np.testing.assert_array_equal(fm.ring_x, fp.ring_x)


# ----------------------------------------------------------------- backward


def loss(x, w_r, b, k, wg, wu, wd, dy):
    fw = oracle.forward(x, w_r, b, k, oracle.weights_from_arrays(wg, wu, wd), x.shape[0] * k)
    return float(np.sum(fw.y * dy)), fw


def test_backward_finite_differences():
    rng = np.random.default_rng(11)
    T, d, E, k, f = 6, 8, 4, 2, 6
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=True)
    dy = rng.standard_normal((T, d))
    L0, fw = loss(x, w_r, b, k, wg, wu, wd, dy)
    bw = oracle.backward(x, w_r, fw.routing, oracle.weights_from_arrays(wg, wu, wd), dy)
    h = 1e-6
    params = {"x": (x, bw.dx), "w_r": (w_r, bw.dw_router), "wg": (wg, bw.dw_gate),
              "wu": (wu, bw.dw_up), "wd": (wd, bw.dw_down)}
    for name, (arr, grad) in params.items():
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, min(flat.size, 25), replace=False):
            old = flat[i]
            flat[i] = old + h
            Lp, fp = loss(x, w_r, b, k, wg, wu, wd, dy)
            flat[i] = old - h
            Lm, fm = loss(x, w_r, b, k, wg, wu, wd, dy)
            flat[i] = old
            assert np.array_equal(fp.routing.idx, fw.routing.idx)
            assert np.array_equal(fm.routing.idx, fw.routing.idx)
            fd = (Lp - Lm) / (2 * h)
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-7 * max(1.0, abs(fd)), (name, i)


def torch_layer(x, w_r, b, idx, wg, wu, wd):
    """A second, independent formulation for autograd: dense over all experts, masked by S."""
    l = x @ w_r.T + (0 if b is None else b)
    mask = torch.zeros_like(l, dtype=torch.bool).scatter_(1, idx, True)
    g = torch.softmax(l.masked_fill(~mask, float("-inf")), dim=1)       # [T, E]
    A = torch.einsum("td,efd->tef", x, wg)
    U = torch.einsum("td,efd->tef", x, wu)
    out = torch.einsum("tef,edf->ted", torch.nn.functional.silu(A) * U, wd)
    return (g[:, :, None] * out).sum(dim=1)


def test_backward_against_torch_autograd():
    rng = np.random.default_rng(12)
    T, d, E, k, f = 24, 16, 6, 3, 12
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=True)
    dy = rng.standard_normal((T, d))
    W = oracle.weights_from_arrays(wg, wu, wd)
    r = oracle.route(x, w_r, b, k)
    bw = oracle.backward(x, w_r, r, W, dy)
    ts = [torch.tensor(a, requires_grad=True) for a in (x, w_r, wg, wu, wd)]
    y = torch_layer(ts[0], ts[1], torch.from_numpy(b), torch.from_numpy(r.idx), *ts[2:])
    (y * torch.from_numpy(dy)).sum().backward()
    for got, t in zip((bw.dx, bw.dw_router, bw.dw_gate, bw.dw_up, bw.dw_down), ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_invariants_and_partial_forms():
    rng = np.random.default_rng(13)
    T, d, E, k, f = 30, 12, 10, 2, 8
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=True)
    # make expert 9 unreachable: nothing selects it
    b[9] = -50.0
    dy = rng.standard_normal((T, d))
    W = oracle.weights_from_arrays(wg, wu, wd)
    r = oracle.route(x, w_r, b, k)
    assert r.count[9] == 0
    bw = oracle.backward(x, w_r, r, W, dy)
    np.testing.assert_allclose(bw.dl.sum(axis=1), 0, atol=1e-15)
    assert not bw.dw_router[9].any() and not bw.dw_gate[9].any() and not bw.dw_down[9].any()
    toks = [0, 5, 29]
    dx, dg, dl = oracle.backward_tokens(toks, x, w_r, r, W, dy)
    np.testing.assert_allclose(dx, bw.dx[toks], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dl, bw.dl[toks], rtol=1e-12, atol=1e-14)
    rows = oracle.router_weight_grad_rows([1, 4], x, w_r, r, W, dy)
    np.testing.assert_allclose(rows, bw.dw_router[[1, 4]], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- workload recipe


def test_redraw_margin_and_zipf_skew():
    cfg = LayerConfig("t", T=512, d=64, E=64, k=4, f=32, zipf_s=1.1, hot_ratio=8.0, cid=99)
    w_r, b, x, _ = draw_router_and_tokens(cfg)
    xb = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    l = xb @ w_r.astype(np.float64).T + b.astype(np.float64)
    assert np.all(topk_gap(l, cfg.k) >= cfg.margin)
    t = zipf_targets(cfg.n, cfg.E, 1.1, 8.0)
    assert abs(t[0] / t.mean() - 8.0) < 1e-9 and abs(t.sum() - cfg.n) < 1e-6
    cnt = np.bincount(np.argsort(-l, axis=1)[:, :cfg.k].ravel(), minlength=cfg.E)
    assert 4.0 < cnt.max() / cnt.mean() < 12.0


# ----------------------------------------------------------------- MX wiring and the shared expert


def load_mx_shared():
    with open(os.path.join(GOLDEN, "mx_shared_cases.json")) as fh:
        return json.load(fh)


def _vec(n, nonzero):
    v = np.zeros(n)
    for i, val in nonzero.items():
        v[int(i)] = val
    return v


def _unit_rows(n_rows, n_cols, rows):
    """A matrix whose row r is the unit vector e_c for every r -> c in `rows`, zero elsewhere."""
    m = np.zeros((n_rows, n_cols))
    for r, c in rows.items():
        m[int(r), c] = 1.0
    return m


def mx_golden_check(mod):
    """The hand-derived MX case: x quantised along d, H along f (tests/golden/mx_shared_cases.json)."""
    for c in load_mx_shared()["mx_cases"]:
        d, f = c["d"], c["f"]
        x = _vec(d, c["x_nonzero"])[None, :]
        w_r = _vec(d, c["w_router_nonzero"])[None, :]
        wg = _unit_rows(f, d, c["w_gate_rows"])[None]
        wu = _unit_rows(f, d, c["w_up_rows"])[None]
        wd = _unit_rows(d, f, c["w_down_rows"])[None]
        W = mod.weights_from_arrays(wg, wu, wd)
        fw = mod.forward(x, w_r, None, c["k"], W, C=1, mx_path=True)
        np.testing.assert_array_equal(fw.ring_x[0], _vec(d, c["ring_x_nonzero"]))
        np.testing.assert_array_equal(fw.y[0], _vec(d, c["y_nonzero"]))
        got = mod.forward_tokens([0], x, fw.routing, W, mx_path=True)
        np.testing.assert_array_equal(got[0], _vec(d, c["y_nonzero"]))


def shared_golden_check(mod):
    """The hand-derived shared-expert case through forward and forward_tokens."""
    data = load_mx_shared()
    base = {b["name"]: b for b in load_cases()}
    for c in data["shared_cases"]:
        b = base[c["base_case"]]
        x, w_r = np.array(b["x"]), np.array(b["w_router"])
        W = mod.weights_from_arrays(np.array(b["w_gate"]), np.array(b["w_up"]), np.array(b["w_down"]))
        sh = tuple(np.array(c[n]) for n in ("ws_gate", "ws_up", "ws_down"))
        fw = mod.forward(x, w_r, None, b["k"], W, C=x.shape[0] * b["k"], shared=sh)
        np.testing.assert_allclose(fw.y, c["y"], rtol=0, atol=1e-15)
        got = mod.forward_tokens(range(x.shape[0]), x, fw.routing, W, shared=sh)
        np.testing.assert_allclose(got, c["y"], rtol=0, atol=1e-15)


def torch_mx_fake_quant(v, axis):
    """An MX round trip built on torch's own E4M3 cast (round to nearest even inside
    +-448), independent of oracle/mx.py: X = floor(log2 amax) - 8 per 32 elements from
    torch.frexp, v 2^-X clamped to +-448, cast, and scaled back."""
    t = torch.from_numpy(np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1).copy())
    blk = t.reshape(t.shape[:-1] + (t.shape[-1] // 32, 32))
    amax = blk.abs().amax(dim=-1, keepdim=True)
    _, e = torch.frexp(amax)
    X = torch.where(amax > 0, e.to(torch.float64) - 1 - 8, torch.full_like(amax, -127.0)).clamp(-127, 127)
    s = torch.clamp(blk * torch.exp2(-X), -448.0, 448.0)
    q = s.to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64) * torch.exp2(X)
    return np.moveaxis(q.reshape(t.shape).numpy(), -1, axis)


def torch_mx_layer(x, w_r, b, k, wg, wu, wd):
    """Dense per-token MX layer: y_t = sum_{e in S_t} g_e W_d[e] Q_f(silu(W_g[e] Q_d(x_t)) * W_u[e] Q_d(x_t)),
    with Q the torch-cast MX round trip above, routing on the unquantised x."""
    l = x @ w_r.T + (0 if b is None else b)
    xq = torch_mx_fake_quant(x, axis=1)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        S = np.argsort(-l[t], kind="stable")[:k]
        z = np.exp(l[t, S] - l[t, S].max())
        g = z / z.sum()
        for gi, e in zip(g, S):
            a = wg[e] @ xq[t]
            u = wu[e] @ xq[t]
            h = torch.nn.functional.silu(torch.from_numpy(a)).numpy() * u
            y[t] += gi * (wd[e] @ torch_mx_fake_quant(h[None, :], axis=1)[0])
    return y


def torch_mx_check(mod):
    """The MX layer of the oracle against the torch-cast formulation: a few experts with
    ragged loads, and one expert of 64 rows (so that a block along the wrong axis exists)."""
    for seed, (T, d, E, k, f) in ((14, (12, 64, 4, 2, 96)), (15, (64, 64, 1, 1, 64))):
        rng = np.random.default_rng(seed)
        x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=E > 1)
        wg, wu = torch_mx_fake_quant(wg, axis=2), torch_mx_fake_quant(wu, axis=2)
        wd = torch_mx_fake_quant(wd, axis=2)
        W = mod.weights_from_arrays(wg, wu, wd)
        ref = torch_mx_layer(x, w_r, b, k, wg, wu, wd)
        fw = mod.forward(x, w_r, b, k, W, C=T * k + 3, head=2, mx_path=True)
        np.testing.assert_allclose(fw.y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
        got = mod.forward_tokens(range(T), x, fw.routing, W, mx_path=True)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def shared_brute_check(mod):
    """forward / forward_tokens with a shared expert against the per-token brute force."""
    rng = np.random.default_rng(16)
    T, d, E, k, f = 9, 16, 5, 2, 12
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=True)
    sh = (rng.standard_normal((f, d)) / 4, rng.standard_normal((f, d)) / 4, rng.standard_normal((d, f)) / 3)
    W = mod.weights_from_arrays(wg, wu, wd)
    bf = oracle.brute_force(x, w_r, b, k, oracle.weights_from_arrays(wg, wu, wd), shared=sh)
    fw = mod.forward(x, w_r, b, k, W, C=T * k, shared=sh)
    np.testing.assert_allclose(fw.y, bf, rtol=0, atol=1e-12 * np.abs(bf).max())
    got = mod.forward_tokens(range(T), x, fw.routing, W, shared=sh)
    np.testing.assert_allclose(got, bf, rtol=0, atol=1e-12 * np.abs(bf).max())


def test_mx_golden_case():
    mx_golden_check(oracle.moe)
    c = load_mx_shared()["mx_cases"][0]
    codes, scales = mx.quantize(_vec(c["d"], c["x_nonzero"])[None, :], axis=1)
    assert scales.tolist() == [[c["x_scale_byte"]]]
    np.testing.assert_array_equal(codes[0], _vec(c["d"], {i: int(h, 16) for i, h in c["x_codes_nonzero"].items()}))
    h = np.zeros(c["f"])
    h[0] = 1.125 / (1 + math.exp(-1.125)) * 1.25
    h[1] = 9.0 / (1 + math.exp(-3.0))
    codes, scales = mx.quantize(h[None, :], axis=1)
    assert scales.tolist() == [[c["h_scale_byte"]]]
    np.testing.assert_array_equal(codes[0], _vec(c["f"], {i: int(v, 16) for i, v in c["h_codes_nonzero"].items()}))


def test_shared_expert_golden_case():
    shared_golden_check(oracle.moe)


def test_shared_expert_against_brute_force():
    shared_brute_check(oracle.moe)
    # the brute force's own shared term against a closed form: one token, E = 1
    x = np.array([[1.0, 0.0]])
    y = oracle.brute_force(x, np.array([[1.0, 0.0]]), None, 1,
                           oracle.weights_from_arrays(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), np.zeros((1, 2, 1))),
                           shared=(np.array([[2.0, 0.0]]), np.array([[0.5, 0.0]]), np.array([[1.0], [-2.0]])))
    s2 = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(y, [[s2, -2 * s2]], rtol=0, atol=1e-15)


def test_mx_layer_against_torch_float8():
    torch_mx_check(oracle.moe)


# ----------------------------------------------------------------- MXFP8 backward


def torch_token_quant(M):
    """MX round trip along the row axis with blocks aligned to the last row, written as: flip
    the rows, quantise blocks of 32 from the (new) top with the last block partial, flip back."""
    t = torch.from_numpy(np.ascontiguousarray(M[::-1]))
    n = t.shape[0]
    out = torch.empty_like(t)
    for r0 in range(0, n, 32):
        blk = t[r0:r0 + 32]
        full = torch.zeros((32,) + tuple(blk.shape[1:]), dtype=blk.dtype)
        full[: blk.shape[0]] = blk
        out[r0:r0 + 32] = torch.from_numpy(torch_mx_fake_quant(full.numpy(), axis=0))[: blk.shape[0]]
    return out.numpy()[::-1].copy()


def torch_mx_backward(x, w_r, b, k, wg, wu, wd, dy):
    """The MXFP8 layer's backward written out per token and per expert with torch's E4M3 cast:
    the routing from a library argsort, each expert's copies listed by scanning tokens."""
    T, d = x.shape
    E = w_r.shape[0]
    l = x @ w_r.T + (0 if b is None else b)
    S = np.sort(np.argsort(-l, axis=1, kind="stable")[:, :k], axis=1)
    q = lambda v, ax: torch_mx_fake_quant(v, axis=ax)
    dx = np.zeros((T, d))
    dg = np.zeros((T, k))
    dwg, dwu, dwd = np.zeros_like(wg), np.zeros_like(wu), np.zeros_like(wd)
    for e in range(E):
        ts = [t for t in range(T) if e in S[t]]
        if not ts:
            continue
        js = [int(np.nonzero(S[t] == e)[0][0]) for t in ts]
        rows = {"dA": [], "dU": [], "X": [], "dY": [], "gH": []}
        for t, j in zip(ts, js):
            lS = l[t, S[t]]
            g = np.exp(lS[j] - lS.max()) / np.exp(lS - lS.max()).sum()
            xq = q(x[t][None, :], 1)[0]
            bf = lambda v: torch.from_numpy(v).float().to(torch.bfloat16).double().numpy()
            a = bf(q(wg[e], 1) @ xq)
            u = bf(q(wu[e], 1) @ xq)
            sg = torch.sigmoid(torch.from_numpy(a)).numpy()
            h = a * sg * u
            dhr = q(dy[t][None, :], 1)[0] @ q(wd[e], 0)
            dg[t, j] = dhr @ h
            da = g * dhr * u * sg * (1 + a * (1 - sg))
            du = g * dhr * a * sg
            dx[t] += q(da[None, :], 1)[0] @ q(wg[e], 0) + q(du[None, :], 1)[0] @ q(wu[e], 0)
            for nm, v in (("dA", da), ("dU", du), ("X", x[t]), ("dY", dy[t]), ("gH", g * h)):
                rows[nm].append(v)
        R = {nm: torch_token_quant(np.array(v)) for nm, v in rows.items()}
        dwg[e], dwu[e] = R["dA"].T @ R["X"], R["dU"].T @ R["X"]
        dwd[e] = R["dY"].T @ R["gH"]
    gate = np.stack([np.exp(l[t, S[t]] - l[t, S[t]].max()) / np.exp(l[t, S[t]] - l[t, S[t]].max()).sum()
                     for t in range(T)])
    dl = gate * (dg - (gate * dg).sum(axis=1, keepdims=True))
    dwr = np.zeros_like(w_r)
    for t in range(T):
        for j in range(k):
            dwr[S[t, j]] += dl[t, j] * x[t]
            dx[t] += dl[t, j] * w_r[S[t, j]]
    return dx, dwg, dwu, dwd, dwr


def mx_backward_check(mod):
    """The oracle's MXFP8 backward against the torch formulation: 3 experts with 40-50 copies
    each (partial first token blocks), a bias, a wrapping ring head."""
    rng = np.random.default_rng(18)
    T, d, E, k, f = 70, 64, 3, 2, 64
    x, w_r, b, wg, wu, wd = rand_layer(rng, T, d, E, k, f, bias=True)
    dy = rng.standard_normal((T, d))
    r = mod.route(x, w_r, b, k)
    C = T * k + 5
    disp = mod.dispatch(r.idx, E, C, head=C - 9)
    assert all(n % 32 and n > 32 for n in r.count)
    bw = mod.backward_mx(x, w_r, r, mod.weights_from_arrays(wg, wu, wd), dy, disp)
    ref = torch_mx_backward(x, w_r, b, k, wg, wu, wd, dy)
    for got, want in zip((bw.dx, bw.dw_gate, bw.dw_up, bw.dw_down, bw.dw_router), ref):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_mx_backward_against_torch_float8():
    mx_backward_check(oracle.moe)


def test_token_quant_end_alignment():
    """Blocks of 32 rows aligned to the last row: with 40 rows, rows 8..39 form one block
    whose amax is set by row 39 (2^5 -> X = -3), rows 0..7 a partial block (amax 1 -> X = -8)."""
    M = np.zeros((40, 32))
    M[:, 0] = 1.1          # not MX-representable at X = -3 (1.1 * 8 = 8.8 -> 9 -> 1.125)
    M[39, 0] = 32.0
    Q = oracle.token_quant(M)
    assert Q[39, 0] == 32.0 and Q[8, 0] == 1.125 and Q[38, 0] == 1.125
    # the partial first block, amax 1.1: X = -8, 1.1 * 256 = 281.6 -> 288 -> 1.125
    assert Q[0, 0] == 1.125 and Q[7, 0] == 1.125
    # a value far below its block's maximum is subnormal there: 0.0013 in the block of 32.0
    # (X = -3): 0.0013 * 8 = 0.0104 -> 5 steps of 2^-9 -> 5 * 2^-12; in the partial block
    # of 0.0013 alone (X = floor(log2 0.0013) - 8 = -18): 340.8 -> 352 -> 352 * 2^-18.
    # Blocks aligned to the start would put row 8 with rows 0..31 (the second value).
    M[:, 0] = 0.0013
    M[39, 0] = 32.0
    Q = oracle.token_quant(M)
    assert Q[8, 0] == 5 * 2.0 ** -12 and Q[38, 0] == 5 * 2.0 ** -12
    assert Q[0, 0] == 352 * 2.0 ** -18 and Q[7, 0] == 352 * 2.0 ** -18


def test_round_bf16_against_torch():
    """The saved pre-activations' rounding: fp64 -> fp32 -> bf16, both round to nearest even,
    against torch's own conversions, on values spread over 40 binades and on exact bf16 ties."""
    rng = np.random.default_rng(19)
    v = rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))
    ties = (np.arange(1, 2001) * 2 + 1).astype(np.float64) * 2.0 ** -8   # odd multiples of half a bf16 step near 1..16
    for a in (v, ties, -ties):
        ref = torch.from_numpy(a).float().to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(oracle.moe.round_bf16(a), ref)
