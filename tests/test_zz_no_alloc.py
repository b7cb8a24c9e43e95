"""moe_decode_noalloc (the decode entry point that allocates nothing and runs on the
library's static scratch) against moe_decode with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller input, each bitwise equal to moe_decode."""
import ctypes

import pytest
import torch

import mixture_experts_layer_33_amd as moe
from mixture_experts_layer_33_amd import _lib
from gen import LayerConfig, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _p(t):
    return None if t is None else t.data_ptr()


def run_both(cfg):
    inp = make_layer(cfg, DEV)
    s = moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, fs=cfg.fs)
    outs = []
    for noalloc in (False, True):
        y = torch.full((cfg.T, cfg.d), -1.0, dtype=torch.bfloat16, device=DEV)
        idx = torch.full((cfg.T, cfg.k), -1, dtype=torch.int32, device=DEV)
        gate = torch.full((cfg.T, cfg.k), -1.0, dtype=torch.float32, device=DEV)
        w = [_p(inp.x), _p(inp.w_router), _p(inp.b_router), _p(inp.w_gate), _p(inp.w_up),
             _p(inp.w_down), _p(inp.ws_gate), _p(inp.ws_up), _p(inp.ws_down), _p(y), _p(idx),
             _p(gate)]
        st = torch.cuda.current_stream().cuda_stream
        if noalloc:
            rc = _lib.lib().moe_decode_noalloc(s, *w, st)
        else:
            ws = moe.workspace(s, moe.OP_DECODE, DEV)
            rc = _lib.lib().moe_decode(s, *w, _p(ws), ws.numel(), st)
        assert rc == _lib.MOE_OK, _lib.lib().moe_status_string(rc)
        torch.cuda.synchronize()
        outs.append((y, idx, gate))
    (y0, i0, g0), (y1, i1, g1) = outs
    assert torch.equal(i0, i1) and torch.equal(g0.view(torch.int32), g1.view(torch.int32))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    return y1


def test_noalloc_decode_matches_decode_twice_second_smaller():
    big = LayerConfig("noalloc_b8", T=8, d=2048, E=64, k=8, f=1024, fs=1024, cid=60)
    small = LayerConfig("noalloc_b2", T=2, d=1024, E=16, k=2, f=512, fs=0, cid=61)
    for cfg in (big, small):
        print(f"\n[case] moe_decode_noalloc {cfg.name}", flush=True)
        run_both(cfg)


def test_noalloc_decode_rejects_shapes_beyond_its_scratch():
    s = moe.make_shape(8, 1024, 64, 16, 4096, fs=4096)
    assert moe.workspace_bytes(s, moe.OP_DECODE) > (1 << 20)
    rc = _lib.lib().moe_decode_noalloc(s, *([0x1000] * 12), None)
    assert rc == _lib.MOE_ERR_SCRATCH
