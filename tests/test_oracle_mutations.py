"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins
catch every one: a dropped term, a wrong sign, a wrong index, a swapped operand."""
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import mx as real_mx

HERE = os.path.dirname(__file__)
MOE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "moe.py")
MX_SRC = os.path.join(os.path.dirname(HERE), "oracle", "mx.py")


def mutant(path, old, new, name, extra=None):
    src = open(path).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    if extra:
        mod.__dict__.update(extra)
    sys.modules[name] = mod        # dataclasses look their module up while the class is built
    try:
        exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    if extra:                      # re-bind names the source imported over the injected ones
        mod.__dict__.update(extra)
    return mod


def small_layer(seed=0, T=10, d=8, E=5, k=2, f=8):
    rng = np.random.default_rng(seed)
    w_r = rng.standard_normal((E, d)) / math.sqrt(d)
    b = rng.standard_normal(E) * 0.3
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, f)) / math.sqrt(f)
    dy = rng.standard_normal((T, d))
    return x, w_r, b, k, wg, wu, wd, dy


def check_brute(mod):
    x, w_r, b, k, wg, wu, wd, _ = small_layer()
    W = mod.weights_from_arrays(wg, wu, wd)
    fw = mod.forward(x, w_r, b, k, W, 2 * x.shape[0] * k, head=3)
    bf = oracle.brute_force(x, w_r, b, k, oracle.weights_from_arrays(wg, wu, wd))
    np.testing.assert_allclose(fw.y, bf, rtol=0, atol=1e-12)


def check_dispatch(mod):
    rng = np.random.default_rng(1)
    T, E, k = 20, 5, 2
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    C, head = 50, 37
    disp = mod.dispatch(idx, E, C, head)
    order = sorted(((idx[t, j], t, j) for t in range(T) for j in range(k)))
    for rank, (_, t, j) in enumerate(order):
        assert disp.copy_slot[t, j] == (head + rank) % C


def check_closed_forms(mod):
    with open(os.path.join(HERE, "golden", "closed_form_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        x, w_r = np.array(c["x"]), np.array(c["w_router"])
        W = mod.weights_from_arrays(np.array(c["w_gate"]), np.array(c["w_up"]), np.array(c["w_down"]))
        fw = mod.forward(x, w_r, None, c["k"], W, c["k"])
        np.testing.assert_allclose(fw.y, c["y"], atol=1e-15, rtol=0)
        bw = mod.backward(x, w_r, fw.routing, W, np.array(c["dy"]))
        np.testing.assert_allclose(bw.dw_router, c["dw_router"], atol=1e-15, rtol=0)
        if "dx" in c:
            np.testing.assert_allclose(bw.dx, c["dx"], atol=1e-14, rtol=0)
            np.testing.assert_allclose(bw.dw_down[0], c["dw_down0"], atol=1e-14, rtol=0)


def check_autograd(mod):
    from test_oracle_pins import torch_layer
    x, w_r, b, k, wg, wu, wd, dy = small_layer(2)
    r = oracle.route(x, w_r, b, k)
    bw = mod.backward(x, w_r, r, mod.weights_from_arrays(wg, wu, wd), dy)
    ts = [torch.tensor(a, requires_grad=True) for a in (x, w_r, wg, wu, wd)]
    y = torch_layer(ts[0], ts[1], torch.from_numpy(b), torch.from_numpy(r.idx), *ts[2:])
    (y * torch.from_numpy(dy)).sum().backward()
    for got, t in zip((bw.dx, bw.dw_router, bw.dw_gate, bw.dw_up, bw.dw_down), ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_mx_wiring(mod):
    from test_oracle_pins import mx_golden_check, torch_mx_check
    mx_golden_check(mod)
    torch_mx_check(mod)


def check_shared(mod):
    from test_oracle_pins import shared_brute_check, shared_golden_check
    shared_golden_check(mod)
    shared_brute_check(mod)


def check_mx_backward(mod):
    from test_oracle_pins import mx_backward_check
    mx_backward_check(mod)
    M = np.zeros((40, 32))
    M[:, 0] = 0.0013
    M[39, 0] = 32.0
    assert mod.token_quant(M)[8, 0] == 5 * 2.0 ** -12


MOE_CHECKS = [check_brute, check_dispatch, check_closed_forms, check_autograd, check_mx_wiring,
              check_shared, check_mx_backward]

MOE_MUTATIONS = [
    ("silu sign", "H = A * sigmoid(A) * U", "H = A * sigmoid(-A) * U"),
    ("gates not renormalised", "g = pS / pS.sum(axis=1, keepdims=True)", "g = pS"),
    ("bottom-k instead of top-k", 'np.argsort(-l, axis=1, kind="stable")', 'np.argsort(l, axis=1, kind="stable")'),
    ("bias dropped", "l = l + b[None, :]", "l = l"),
    ("gate/up operands swapped", "A = X @ wg.T", "A = X @ wu.T"),
    ("ring head ignored", "slot = (head + rank) % C", "slot = rank % C"),
    ("tokens reversed in a segment", 'perm = np.argsort(keys, kind="stable")',
     'perm = (len(keys) - 1 - np.argsort(keys[::-1], kind="stable"))'),
    ("combine index", "ring_y[copy_slot[:, j]]", "ring_y[copy_slot[:, 0]]"),
    ("silu' term dropped", "dA = dH * U * s * (1.0 + A * (1.0 - s))", "dA = dH * U * s"),
    ("router grad sign", "return gate * (dg - np.sum(gate * dg, axis=1, keepdims=True))",
     "return gate * (dg + np.sum(gate * dg, axis=1, keepdims=True))"),
    ("gate dropped in dW_down", "(g[:, None] * dy[ts]).T @ H", "dy[ts].T @ H"),
    ("W_down rows reversed in dgrad", "dHraw = dy[ts] @ wd", "dHraw = dy[ts] @ wd[::-1]"),
    ("router term missing in dx", "dx += dl[:, j, None] * w_r[routing.idx[:, j]]", "pass"),
    ("H not quantised", "H = mx.fake_quant(H, axis=1)", "H = H"),
    ("H quantised along rows", "H = mx.fake_quant(H, axis=1)", "H = mx.fake_quant(H, axis=0)"),
    ("x not quantised in forward", "rows = mx.fake_quant(x, axis=1) if mx_path else x", "rows = x"),
    ("x quantised along tokens in forward", "rows = mx.fake_quant(x, axis=1) if mx_path else x",
     "rows = mx.fake_quant(x, axis=0) if mx_path else x"),
    ("x not quantised in forward_tokens", "xq = mx.fake_quant(xs, axis=1) if mx_path else xs", "xq = xs"),
    ("shared expert dropped in forward", "y = y + swiglu(x, *shared)", "y = y"),
    ("shared expert gated in forward", "y = y + swiglu(x, *shared)", "y = y + r.gate[:, :1] * swiglu(x, *shared)"),
    ("shared expert halved in forward_tokens", "y += swiglu(xs, *shared)", "y += 0.5 * swiglu(xs, *shared)"),
    ("shared expert dropped in forward_tokens", "y += swiglu(xs, *shared)", "pass"),
    ("MX bwd: dY not quantised", "dHraw = mx.fake_quant(dY, axis=1) @", "dHraw = dY @"),
    ("MX bwd: W_down quantised along f", "@ mx.fake_quant(wd, axis=0)", "@ mx.fake_quant(wd, axis=1)"),
    ("MX bwd: dA not quantised", "dxc = (mx.fake_quant(dA, axis=1) @", "dxc = (dA @"),
    ("MX bwd: W_gate quantised along d", "mx.fake_quant(dA, axis=1) @ mx.fake_quant(wg, axis=0)",
     "mx.fake_quant(dA, axis=1) @ mx.fake_quant(wg, axis=1)"),
    ("MX bwd: dU paired with W_gate", "+ mx.fake_quant(dU, axis=1) @ mx.fake_quant(wu, axis=0)",
     "+ mx.fake_quant(dU, axis=1) @ mx.fake_quant(wg, axis=0)"),
    ("MX bwd: token blocks aligned to the start",
     "P = np.concatenate([np.zeros((pad,) + M.shape[1:]), M], axis=0)\n    return mx.fake_quant(P, axis=0)[pad:]",
     "P = np.concatenate([M, np.zeros((pad,) + M.shape[1:])], axis=0)\n    return mx.fake_quant(P, axis=0)[:n]"),
    ("MX bwd: gH not token-quantised", "token_quant(g[:, None] * H)", "(g[:, None] * H)"),
    ("MX bwd: X not token-quantised", "Xt = token_quant(X)", "Xt = X"),
    ("MX bwd: A from unquantised x", "A = round_bf16(Xq @ mx.fake_quant(wg, axis=1).T)",
     "A = round_bf16(X @ mx.fake_quant(wg, axis=1).T)"),
    ("MX bwd: U not rounded as saved", "U = round_bf16(Xq @ mx.fake_quant(wu, axis=1).T)",
     "U = Xq @ mx.fake_quant(wu, axis=1).T"),
    ("MX bwd: copies in token order, not ring order", "copies = disp.slot_copy[segment_slots(disp, e)]",
     "copies = np.sort(disp.slot_copy[segment_slots(disp, e)])[::-1]"),
]


@pytest.mark.parametrize("m", MOE_MUTATIONS, ids=lambda m: m[0])
def test_moe_mutation_is_caught(m):
    _, old, new = m
    mod = mutant(MOE_SRC, old, new, "oracle_moe_mutant")
    caught = 0
    for chk in MOE_CHECKS:
        try:
            chk(mod)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"mutation not caught: {m[0]}"


def check_mx(mod):
    from test_oracle_pins import read_spec_points
    for v, c in read_spec_points():
        assert int(mod.encode_e4m3(np.array([v]))[0]) == c
    rng = np.random.default_rng(0)
    v = rng.standard_normal((8, 64)) * 3
    _, s = mod.quantize(v, axis=1)
    blk = np.abs(v).reshape(8, 2, 32).max(axis=2)
    assert np.all(s.astype(int) - 127 == np.floor(np.log2(blk)) - 8)
    mids = (0.5 * (real_mx.POS_VALUES[1:] + real_mx.POS_VALUES[:-1])).astype(np.float32)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mod.encode_e4m3(mids.astype(np.float64)), ref)


MX_MUTATIONS = [
    ("scale exponent off by one", "X = e.astype(np.int64) - 1 - 8", "X = e.astype(np.int64) - 1 - 7"),
    ("ties to odd", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    ("subnormal step", "return s * m * 2.0 ** -9", "return s * m * 2.0 ** -10"),
    ("exponent bias", "return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "return s * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
]


@pytest.mark.parametrize("m", MX_MUTATIONS, ids=lambda m: m[0])
def test_mx_mutation_is_caught(m):
    _, old, new = m
    mod = mutant(MX_SRC, old, new, "oracle_mx_mutant")
    with pytest.raises(AssertionError):
        check_mx(mod)


def test_unmutated_oracle_passes_every_check():
    for chk in MOE_CHECKS:
        chk(oracle.moe)
    check_mx(real_mx)
