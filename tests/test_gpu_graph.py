"""HIP-graph replay of the decode calls equals eager execution, replay after replay.

The library enqueues plain kernels on the caller's stream (no memsets, no host
synchronisation), so torch can capture a decode step into a graph.  Each replay
is checked bit for bit against the eager result, with eager work in between.
"""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
from hybrid_swa_kv_amd import synth
from tests.helpers import announce

pytestmark = pytest.mark.gpu


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy()


def test_graph_replay_decode_step():
    announce("graph_replay")
    B, Hq, Hkv, D, W = 8, 32, 8, 128, 128
    layers = 3
    sets = []
    for i in range(layers):
        sets.append(dict(
            q=synth.normal_gpu(200, 10 + i, (B, Hq, D)),
            kn=synth.normal_gpu(200, 20 + i, (B, Hkv, D)),
            vn=synth.normal_gpu(200, 30 + i, (B, Hkv, D)),
            rk=synth.normal_gpu(200, 40 + i, (B, Hkv, W, D)),
            rv=synth.normal_gpu(200, 50 + i, (B, Hkv, W, D))))
    pos = torch.arange(1000, 1000 + B, dtype=torch.int32, device="cuda")
    T8, Th = 1024, 100
    kx = synth.normal_gpu(201, 1, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    vx = synth.normal_gpu(201, 2, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    kc, ks = hsk.kv_quant_int8_b32(kx[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(vx[:, :, :T8].contiguous())
    kh, vh = kx[:, :, T8:].contiguous(), vx[:, :, T8:].contiguous()
    qi = synth.normal_gpu(201, 3, (B, Hq, D))
    ws = torch.empty(hsk.attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(s["q"]) for s in sets]
    slots = torch.empty(B, dtype=torch.int32, device="cuda")
    iout = torch.empty_like(qi)

    def step():
        for s, o in zip(sets, outs):
            hsk.swa_decode_ring(s["q"], s["kn"], s["vn"], s["rk"], s["rv"], pos, out=o, slot_out=slots)
        hsk.attn_decode_int8kv(qi, kc, ks, vc, vs, kh, vh, out=iout, workspace=ws)

    step()   # eager reference (the ring appends are idempotent: same token, same slot)
    ref = [_bits(o) for o in outs] + [_bits(iout)]
    ref_ring = [(_bits(s["rk"]), _bits(s["rv"])) for s in sets]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs + [iout]:
            o.fill_(0)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = [_bits(o) for o in outs] + [_bits(iout)]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep} differs from eager"
        for s, (rk, rv) in zip(sets, ref_ring):
            assert np.array_equal(_bits(s["rk"]), rk) and np.array_equal(_bits(s["rv"]), rv)
        assert np.array_equal(slots.cpu().numpy(), (pos.cpu().numpy() % W))
