"""One decode step of a hybrid stack (sliding-window ring layers and full-attention
layers, [MiMo-inf] section 1: 60 of 70 layers use a 128-token window, 10 the full
context), run as one HIP graph and replayed: every layer equals the oracle."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


def test_hybrid_decode_step_graph():
    B, Hq, Hkv, D, W, ctx = 2, 8, 2, 128, 128, 1024
    kinds = [(i % 7) == 6 for i in range(14)]        # 12 window layers, 2 full layers
    announce("hybrid_step", layers=len(kinds), ctx=ctx)
    pos = ctx - 1                                    # the new token's position
    d_pos = torch.full((B,), pos, dtype=torch.int32, device="cuda")
    slots = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(hsk.attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, 0, ctx), dtype=torch.uint8,
                     device="cuda")
    to_bits = lambda x: synth.f32_to_bf16_bits(x.astype(np.float32))
    layers, refs = [], []
    for i, full in enumerate(kinds):
        seed = 900 + i
        kseq = synth.head_major(seed, synth.K, B, Hkv, ctx, D)     # positions 0..pos
        vseq = synth.head_major(seed, synth.V, B, Hkv, ctx, D)
        q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
        kf, vf = f64(kseq), f64(vseq)
        refs.append(oracle.swa_decode(f64(q), kf, vf, [0] * B, [pos] * B, 0 if full else W))
        if full:
            layers.append(("full", gpu_bf16(q), gpu_bf16(kseq), gpu_bf16(vseq)))
        else:
            rk = oracle.ring_fill(kf, [0] * B, [pos - 1] * B, W, np.zeros((B, Hkv, W, D)))
            rv = oracle.ring_fill(vf, [0] * B, [pos - 1] * B, W, np.zeros((B, Hkv, W, D)))
            layers.append(("swa", gpu_bf16(q), gpu_bf16(np.ascontiguousarray(kseq[:, :, pos])),
                           gpu_bf16(np.ascontiguousarray(vseq[:, :, pos])),
                           gpu_bf16(to_bits(rk)), gpu_bf16(to_bits(rv))))
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in kinds]

    def step():
        for ly, o in zip(layers, outs):
            if ly[0] == "full":
                hsk.attn_decode_int8kv(ly[1], None, None, None, None, ly[2], ly[3], out=o, workspace=ws)
            else:
                hsk.swa_decode_ring(ly[1], ly[2], ly[3], ly[4], ly[5], d_pos, out=o, slot_out=slots)

    step()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            ex = bf16_excess(out_f64(o), ref)
            assert ex <= 0, (rep, i, kinds[i], ex, max_abs(out_f64(o), ref))
    assert np.array_equal(slots.cpu().numpy(), oracle.ring_slot(np.full(B, pos), W))

