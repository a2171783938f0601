#!/usr/bin/env python3
"""Throughput of the hybrid sliding-window / INT8 / block-sparse attention path on one MI355X.

One step is one pass over every operation of the path, each at its workload size:

  ring    swa_decode_ring   batch 32, context 32768, 32 q / 8 kv heads, head_dim 128,
                            window 128; 60 distinct ring sets per step (one per
                            sliding-window layer of a 70-layer hybrid stack)
  swa     swa_prefill       L 131072, 64 q / 8 kv heads, head_dim 128, window 1024
  full    swa_prefill       same shape, full causal
  chunk4096 / chunk8192  swa_prefill_chunk: the window prefill as 32 (16) chunks,
            each continuing from the ring the previous chunk left
  quant   kv_quant_int8_b32 K and V of batch 16, 63488 warm tokens, 8 kv heads
  int8    attn_decode_int8kv batch 16, context 65536 (2048 hot bf16 tokens), 32/8 heads
  int8sparse  attn_decode_int8kv_sparse on the same pool: the hot tail plus each
            head's top-64 32-token INT8 blocks (scored by q . block mean)
  sparse  blocksparse_select_attend  L 131072, 32/8 heads, 64-token blocks, top-64, window 1024
  tiny    swa_prefill       fp32, L 512, 2/2 heads, head_dim 64, window 128 (absolute time)
  hybrid70  one decode step of a 70-layer hybrid stack: 60 swa_decode_ring layers
            (window 128) and 10 full-attention layers (attn_decode_int8kv over an
            all-bf16 context), batch 32, context 32768, one HIP graph; also the
            10 full layers alone, to price an all-full step

The JSON line's headline is the ring-decode workload (KV bytes per second of the
60 ring-decode launches in each step, captured once as a HIP graph and replayed,
timed with HIP events on the stream they run on); every other operation is
reported under "rows" with its own roofline.
Inputs are seeded synthetic tensors (N(0,1), 1% x8 outliers for the INT8 cache)
drawn on the GPU and resident in HBM before timing starts.  The CPU oracle is
timed beside every row on one host core ("cpu_baseline" of each row; the
top-level one is the ring row's): in full where a sample of whole calls fits a
few seconds, otherwise on sampled rows, heads or units and extrapolated by
visible-pair, head, chunk or unit count (marked "extrapolated").
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s and decode KV GB/s, % of MI355X peak; oracle-exact"
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12   # dense bf16 MFMA, 2516.6 TFLOP/s
PEAK_HBM_GBS = 8000.0                           # HBM3E, 8 TB/s

# workload shapes
TINY = dict(L=512, Hq=2, Hkv=2, D=64, W=128)   # the fp32 correctness-sized window prefill
RING = dict(B=32, Hq=32, Hkv=8, D=128, W=128, ctx=32768, layers=60)
PREFILL = dict(L=131072, Hq=64, Hkv=8, D=128, W=1024)
INT8 = dict(B=16, Hq=32, Hkv=8, D=128, ctx=65536, hot=2048)
SPARSE = dict(L=131072, Hq=32, Hkv=8, D=128, block=64, topk=64, W=1024)
# one decode step of the 70-layer hybrid stack: 60 sliding-window layers (ring,
# W = 128) and 10 full-attention layers (every 7th), batch 32 at context 32768
HYBRID = dict(B=32, Hq=32, Hkv=8, D=128, W=128, ctx=32768, layers=70, full_every=7)


# HBM traffic of the headline kernel, from the two rocprofv3 --pmc passes recorded
# in this file; it is reported only while the kernel's sources hash to the value
# recorded there (a changed kernel reports null until it is measured again).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ring_decode_kernel_b32_w128_hbm_traffic.txt")
RING_SOURCES = ("decode_ring.hip", "decode_mfma.hpp", "common.hpp", "kernels.hpp")


def ring_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in RING_SOURCES:
        with open(os.path.join(ROOT, "hybrid_swa_kv_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per launch recorded for the current ring kernel sources, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith((" ", "#")))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != ring_source_hash():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pairs_prefill(L: int, W: int) -> int:
    if W <= 0 or W >= L:
        return L * (L + 1) // 2
    return W * (W + 1) // 2 + (L - W) * W


def ring_bytes_per_call(c=RING) -> int:
    """Ring K+V read, q read, out write, new-token K/V write (bf16)."""
    ring = 2 * c["B"] * c["Hkv"] * c["W"] * c["D"] * 2
    q = c["B"] * c["Hq"] * c["D"] * 2
    return ring + 2 * q + 2 * c["B"] * c["Hkv"] * c["D"] * 2


def full_decode_bytes(c=HYBRID) -> int:
    """One full-attention decode layer: K and V of the whole context, q read, out write."""
    return 2 * c["B"] * c["Hkv"] * c["ctx"] * c["D"] * 2 + 2 * c["B"] * c["Hq"] * c["D"] * 2


def hybrid_layers(c=HYBRID):
    """Layer kinds of the stack in order: True for a full-attention layer."""
    return [(i % c["full_every"]) == c["full_every"] - 1 for i in range(c["layers"])]


def int8_decode_bytes(c=INT8) -> int:
    t8 = c["ctx"] - c["hot"]
    codes = 2 * c["B"] * c["Hkv"] * t8 * c["D"]
    scales = 2 * c["B"] * c["Hkv"] * (t8 // 32) * 4
    hot = 2 * c["B"] * c["Hkv"] * c["hot"] * c["D"] * 2
    q = c["B"] * c["Hq"] * c["D"] * 2
    return codes + scales + hot + 2 * q


def int8_sparse_bytes(sel, c=INT8) -> int:
    """Bytes the block-sparse decode moves: per (sequence, KV head) the union of the
    group's kept blocks (K and V codes + scales), the bf16 hot tail, the block
    means read by the scoring, q and out."""
    import numpy as np

    B, Hq, topk = sel.shape
    G = Hq // c["Hkv"]
    nblk = (c["ctx"] - c["hot"]) // 32
    blocks = 0
    for b in range(B):
        for g in range(c["Hkv"]):
            s = sel[b, g * G:(g + 1) * G].ravel()
            blocks += len(np.unique(s[s >= 0]))
    per_block = 2 * (32 * c["D"] + 4)
    hot = 2 * B * c["Hkv"] * c["hot"] * c["D"] * 2
    means = B * c["Hkv"] * c["D"] * nblk * 4
    return blocks * per_block + hot + means + 2 * B * Hq * c["D"] * 2


def int8_quant_bytes(c=INT8) -> int:
    n = 2 * c["B"] * c["Hkv"] * (c["ctx"] - c["hot"]) * c["D"]
    return n * 2 + n + (n // (32 * c["D"])) * 4


def sparse_pairs(sel, L: int, block: int, W: int) -> int:
    """Exact visible (query, key) pairs of the block-sparse pattern, from the selection."""
    import numpy as np

    Hq, nb, topk = sel.shape
    rows = np.arange(L, dtype=np.int64).reshape(nb, block)            # [qb, r]
    win = np.minimum(rows + 1, W).sum(axis=1)                        # window keys per block
    total = int(win.sum()) * Hq
    start = rows - W + 1                                             # first window key per row
    for h in range(Hq):
        s = sel[h].astype(np.int64)                                  # [qb, topk]
        valid = s >= 0
        # keys of a selected block that lie before the row's window start
        extra = np.clip(start[:, None, :] - (block * s)[:, :, None], 0, block)   # [qb, topk, r]
        total += int((extra * valid[:, :, None]).sum())
    return total


def sparse_tile_bytes(sel, L: int, block: int, W: int, Hkv: int, D: int) -> int:
    """K and V bytes the attention kernel stages for the block-sparse pattern: per
    (query head, query block) every selected block before the window plus the
    window's blocks, one 64-token K tile and V tile (bf16) each."""
    import numpy as np

    Hq, nb, _ = sel.shape
    qb = np.arange(nb, dtype=np.int64)
    kw0 = np.maximum(0, qb * block - W + 1) // block                 # first window block
    tiles = int((qb - kw0 + 1).sum()) * Hq
    s = sel.astype(np.int64)
    tiles += int(((s >= 0) & (s < kw0[None, :, None])).sum())
    return tiles * 2 * block * D * 2


class ClockSampler:
    """Engine clock (MHz) from the driver's pp_dpm_sclk (the line marked '*'),
    sampled by a host thread; each sample carries its host time."""

    def __init__(self):
        import glob
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = None
        self._th = None

    def read(self):
        import re
        vals = []
        for p in self.paths:
            try:
                for ln in open(p).read().splitlines():
                    if ln.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", ln, re.I)
                        if m:
                            vals.append(int(m.group(1)))
            except OSError:
                pass
        return max(vals) if vals else None

    def start(self):
        import threading
        if not self.paths:
            return
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                v = self.read()
                if v is not None:
                    self.samples.append((time.perf_counter(), v))
                time.sleep(0.0005)

        self._th = threading.Thread(target=loop, daemon=True)
        self._th.start()

    def stop(self):
        if self._th is not None:
            self._stop.set()
            self._th.join()

    def per_window(self, windows):
        """windows: (name, t_begin, t_end) in host time -> {name: clock stats}."""
        out = {}
        for name, a, b in windows:
            out.setdefault(name, []).extend(v for t, v in self.samples if a <= t < b)
        stats = {}
        for name, v in out.items():
            if v:
                v = sorted(v)
                stats[name] = {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v)}
        return stats


class Timer:
    """HIP events around work enqueued on torch's current stream (the library's stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.ms = {}
        self.order = []  # (name, end event) in enqueue order

    def run(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.ms.setdefault(name, []).append((a, b))
        self.order.append((name, b))

    def mean_ms(self, name, skip=0):
        ev = self.ms[name][skip:]
        return sum(a.elapsed_time(b) for a, b in ev) / max(1, len(ev))

    def spread(self, name, skip=0, per=1):
        """median, min and p90 of the timed calls of a row (ms, divided by `per`)."""
        v = sorted(a.elapsed_time(b) / per for a, b in self.ms[name][skip:])
        if not v:
            return None
        p90 = v[min(len(v) - 1, int(0.9 * (len(v) - 1) + 0.5))]
        return {"median_ms": round(v[len(v) // 2], 5), "min_ms": round(v[0], 5), "p90_ms": round(p90, 5),
                "calls": len(v)}


def _oracle_pool():
    """Limits BLAS to one thread: every oracle baseline uses exactly one core."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def _timed(fn, budget_s, min_calls=1):
    """Calls fn() until budget_s has passed (at least min_calls); returns (calls, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while n < min_calls or time.perf_counter() - t0 < budget_s:
        fn()
        n += 1
    return n, time.perf_counter() - t0


def _baseline(value, unit, sample, extrapolated, seconds):
    return {"value": value, "unit": unit, "cores": 1, "kind": "oracle", "sample": sample,
            "extrapolated": extrapolated, "oracle_seconds": round(seconds, 2)}


def cpu_ring(budget_s):
    """The oracle on whole ring-decode steps (every ring layer's append + window attention)."""
    import numpy as np

    import oracle
    from hybrid_swa_kv_amd import synth

    c = RING
    B, Hq, Hkv, D, W = c["B"], c["Hq"], c["Hkv"], c["D"], c["W"]
    pos = np.full(B, c["ctx"] - 1, dtype=np.int64)
    kseq = synth.bf16_bits_to_f32(synth.head_major(2, synth.K, B, Hkv, W + 1, D)).astype(np.float64)
    vseq = synth.bf16_bits_to_f32(synth.head_major(2, synth.V, B, Hkv, W + 1, D)).astype(np.float64)
    q = synth.bf16_bits_to_f32(synth.normal(2, synth.Q, (B, Hq, D), 1)).astype(np.float64)
    start = pos - W
    ring_k = oracle.ring_fill(kseq, start, pos - 1, W, np.zeros((B, Hkv, W, D)))
    ring_v = oracle.ring_fill(vseq, start, pos - 1, W, np.zeros((B, Hkv, W, D)))

    def one_step():
        for _ in range(c["layers"]):
            oracle.ring_append(ring_k, pos, kseq[:, :, W])
            oracle.ring_append(ring_v, pos, vseq[:, :, W])
            oracle.swa_decode(q, kseq, vseq, start, pos, W)

    with _oracle_pool():
        steps, el = _timed(one_step, budget_s)
    calls = steps * c["layers"]
    b = _baseline(round(calls * ring_bytes_per_call() / el / 1e9, 4), "GB/s",
                  f"{steps} full steps = {calls} ring-decode calls (append + window attention, batch {B}, "
                  f"{Hq}/{Hkv} heads, window {W}), numpy fp64, one BLAS thread", False, el)
    b["us_per_call"] = round(el / calls * 1e6, 1)
    return b


def cpu_tiny(budget_s):
    """The whole tiny fp32 window prefill (L 512, 2/2 heads, head_dim 64, window 128)."""
    import oracle
    from hybrid_swa_kv_amd import synth

    c = TINY
    q = synth.token_major(1, synth.Q, c["L"], c["Hq"], c["D"], dtype="f32")
    k = synth.token_major(1, synth.K, c["L"], c["Hkv"], c["D"], dtype="f32")
    v = synth.token_major(1, synth.V, c["L"], c["Hkv"], c["D"], dtype="f32")
    with _oracle_pool():
        n, el = _timed(lambda: oracle.swa_prefill(q, k, v, c["W"]), budget_s, 3)
    return _baseline(round(el / n * 1e6, 1), "us", f"{n} whole calls, numpy fp64", False, el)


def cpu_prefill(name, budget_s):
    """C3 rows: query rows of one head timed, extrapolated to every row and head by
    visible (query, key) pairs.  A window row's work does not depend on L, so the
    window rows come from a shorter sequence; full-causal rows span the whole
    131072-token sequence."""
    import numpy as np

    import oracle
    from hybrid_swa_kv_amd import synth

    c = PREFILL
    W = c["W"] if name == "swa" else 0
    L = 4096 if W else c["L"]
    q = synth.token_major(31, synth.Q, L, 1, c["D"], dtype="f32")
    k = synth.token_major(31, synth.K, L, 1, c["D"], dtype="f32")
    v = synth.token_major(31, synth.V, L, 1, c["D"], dtype="f32")
    rng = np.random.default_rng(5)
    done_rows, pairs = 0, 0
    t0 = time.perf_counter()
    with _oracle_pool():
        while done_rows == 0 or time.perf_counter() - t0 < budget_s:
            rows = np.sort(rng.integers(W, L, size=8)) if W else np.sort(rng.integers(0, L, size=8))
            oracle.swa_prefill(q, k, v, W, rows=rows, row_block=1 if W else 8)
            done_rows += len(rows)
            pairs += int(len(rows) * W) if W else int((rows + 1).sum())
    el = time.perf_counter() - t0
    total_pairs = c["Hq"] * pairs_prefill(c["L"], W)
    total_s = el * total_pairs / pairs
    flops = 4 * c["D"] * c["Hq"] * pairs_prefill(c["L"], W)
    return _baseline(round(flops / total_s / 1e12, 6), "TFLOP/s",
                     f"{done_rows} query rows of one head ({pairs} visible pairs, numpy fp64), extrapolated by "
                     f"visible-pair count to all {c['L']} rows x {c['Hq']} heads ({total_s:.0f} s)", True, el)


def cpu_chunk(C, budget_s):
    """One chunk of the window prefill (one query head) timed, extrapolated to every
    head and chunk by head and chunk count."""
    import numpy as np

    import oracle
    from hybrid_swa_kv_amd import synth

    c = PREFILL
    W, D = c["W"], c["D"]
    q = synth.normal(32, synth.Q, (1, C, 1, D), 1, "f32")
    k = synth.normal(32, synth.K, (1, C, 1, D), 1, "f32")
    v = synth.normal(32, synth.V, (1, C, 1, D), 1, "f32")
    rk = synth.normal(32, synth.K_NEW, (1, 1, W, D), 1, "f32")
    rv = synth.normal(32, synth.V_NEW, (1, 1, W, D), 1, "f32")
    with _oracle_pool():
        n, el = _timed(lambda: oracle.swa_prefill_chunk(q, k, v, rk, rv, C, W), budget_s)
    per = el / n
    chunks = c["L"] // C
    total_s = per * c["Hq"] * chunks
    flops = 4 * D * c["Hq"] * pairs_prefill(c["L"], W)
    return _baseline(round(flops / total_s / 1e12, 6), "TFLOP/s",
                     f"{n} calls of one {C}-token chunk at position {C} (one head, numpy fp64), extrapolated by "
                     f"head and chunk count to {c['Hq']} heads x {chunks} chunks ({total_s:.0f} s)", True, el)


def _int8_unit(seed, T, hot, D, G):
    """One (sequence, KV head) unit of the INT8 workload: bf16 K/V values (fp32), q."""
    from hybrid_swa_kv_amd import synth

    kx = synth.bf16_bits_to_f32(synth.head_major(seed, synth.K, 1, 1, T, D, outlier_p=0.01))
    vx = synth.bf16_bits_to_f32(synth.head_major(seed, synth.V, 1, 1, T, D, outlier_p=0.01))
    q = synth.bf16_bits_to_f32(synth.normal(seed, synth.Q, (1, G, D), 1)).astype("float64")
    return kx, vx, q


def cpu_int8(name, budget_s):
    """INT8 rows, by (sequence, KV head) unit: the encoder on a unit's K and V, the
    dense decode or the block-sparse decode of its four query heads; extrapolated
    to the 128 units by unit count."""
    import numpy as np

    import oracle

    c = INT8
    T, hot, D = c["ctx"], c["hot"], c["D"]
    T8, G = T - hot, c["Hq"] // c["Hkv"]
    units = c["B"] * c["Hkv"]
    kx, vx, q = _int8_unit(41, T, hot, D, G)
    kc, ks = oracle.kv_quant_int8_b32(kx[:, :, :T8])
    vc, vs = oracle.kv_quant_int8_b32(vx[:, :, :T8])
    kh, vh = kx[:, :, T8:], vx[:, :, T8:]
    unit_bytes = None
    if name == "quant":
        fn = lambda: (oracle.kv_quant_int8_b32(kx[:, :, :T8]), oracle.kv_quant_int8_b32(vx[:, :, :T8]))
        total_bytes = int8_quant_bytes()
        what = "K and V of one unit encoded"
    elif name == "int8":
        fn = lambda: oracle.attn_decode_int8kv(q, kc, ks, vc, vs, kh, vh)
        total_bytes = int8_decode_bytes()
        what = "one unit's dense decode (4 heads)"
    else:
        def fn():
            means = oracle.int8_block_means(kc, ks)
            sel = oracle.sparse_select(q, means, 64)
            oracle.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, kh, vh, sel)
        means = oracle.int8_block_means(kc, ks)
        sel = oracle.sparse_select(q, means, 64)
        kept = len(np.unique(sel[sel >= 0]))
        unit_bytes = (kept * 2 * (32 * D + 4) + 2 * hot * D * 2 + D * (T8 // 32) * 4 + 2 * G * D * 2)
        total_bytes = unit_bytes * units
        what = "one unit's block means, top-64 selection and sparse decode (4 heads)"
    with _oracle_pool():
        n, el = _timed(fn, budget_s)
    total_s = el / n * units
    return _baseline(round(total_bytes / total_s / 1e9, 4), "GB/s",
                     f"{n} x {what} (numpy; fp32 encoder, fp64 attention), extrapolated by unit count to "
                     f"{units} units ({total_s:.1f} s)", True, el)


def cpu_sparse(budget_s, pairs_total):
    """Block-sparse prefill: one query head's selection (block sums, scores, top-64)
    and whole 64-row output tiles timed; extrapolated to 32 heads and every tile."""
    import numpy as np

    import oracle
    from hybrid_swa_kv_amd import synth

    c = SPARSE
    L, D, blk = c["L"], c["D"], c["block"]
    nb = L // blk
    q = synth.token_major(51, synth.Q, L, 1, D, dtype="f32")
    k = synth.token_major(51, synth.K, L, 1, D, dtype="f32")
    v = synth.token_major(51, synth.V, L, 1, D, dtype="f32")
    t0 = time.perf_counter()
    with _oracle_pool():
        sel = oracle.block_select(q, k, blk, c["topk"])
        t_sel = time.perf_counter() - t0
        rng = np.random.default_rng(9)
        tiles, t1 = 0, time.perf_counter()
        while tiles == 0 or time.perf_counter() - t0 < budget_s:
            qb = int(rng.integers(0, nb))
            oracle.blocksparse_attend(q, k, v, sel, blk, c["W"], rows=np.arange(qb * blk, (qb + 1) * blk))
            tiles += 1
        t_tile = (time.perf_counter() - t1) / tiles
    el = time.perf_counter() - t0
    total_s = c["Hq"] * (t_sel + nb * t_tile)
    flops = 4 * D * pairs_total
    return _baseline(round(flops / total_s / 1e12, 6), "TFLOP/s of visible pairs",
                     f"one head's selection ({t_sel:.1f} s) and {tiles} random 64-row output tiles (numpy fp64), "
                     f"extrapolated to {c['Hq']} heads x {nb} tiles ({total_s:.0f} s)", True, el)


def cpu_hybrid(budget_s, ring_us_per_call):
    """70-layer step: the ring layers priced at the ring baseline's time per call, a
    full layer by (sequence, KV head) unit of its decode over 32768 bf16 tokens."""
    import numpy as np

    import oracle
    from hybrid_swa_kv_amd import synth

    c = HYBRID
    D, G, ctx = c["D"], c["Hq"] // c["Hkv"], c["ctx"]
    kx = synth.bf16_bits_to_f32(synth.head_major(61, synth.K, 1, 1, ctx, D)).astype(np.float64)
    vx = synth.bf16_bits_to_f32(synth.head_major(61, synth.V, 1, 1, ctx, D)).astype(np.float64)
    q = synth.bf16_bits_to_f32(synth.normal(61, synth.Q, (1, G, D), 1)).astype(np.float64)
    with _oracle_pool():
        n, el = _timed(lambda: oracle.swa_decode(q, kx, vx, [0], [ctx - 1], 0), budget_s)
    nfull = sum(hybrid_layers())
    nswa = c["layers"] - nfull
    full_layer_s = el / n * c["B"] * c["Hkv"]
    step_s = nfull * full_layer_s + nswa * ring_us_per_call * 1e-6
    step_bytes = nswa * ring_bytes_per_call() + nfull * full_decode_bytes()
    return _baseline(round(step_bytes / step_s / 1e9, 4), "GB/s",
                     f"{n} x one unit of a full layer's decode (4 heads, {ctx} tokens, numpy fp64), extrapolated "
                     f"to {c['B'] * c['Hkv']} units x {nfull} full layers, plus {nswa} ring layers at the ring "
                     f"baseline's time per call ({step_s:.1f} s per step)", True, el)


def host_info():
    """CPU model, logical CPUs and numpy's BLAS thread pools of the host."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas_pools": blas,
            "oracle_threads": 1}


def source_info():
    """git commit when the tree is a checkout, and a hash of the library sources."""
    import hashlib
    import subprocess

    sha = None
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=5).stdout.strip() or None
    except Exception:
        pass
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_swa_kv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return {"git_sha": sha, "csrc_sha256": h.hexdigest()[:16]}


# seeds of the GPU inputs (synth.normal_gpu(workload, tensor_id, ...), torch Philox)
SEEDS = {
    "ring": "workload 2: ring K/V tensor ids 100 + 2l / 101 + 2l, q 1000 + l, k_new 2000 + l, v_new 3000 + l "
            "for ring set l",
    "tiny": "synth.token_major(1, Q/K/V) fp32 (PCG64 per head)",
    "prefill": "workload 3: q, k, v tensor ids 0, 1, 2",
    "int8": "workload 4: K, V tensor ids 1, 2 (1 % x8 outliers), q 0",
    "sparse": "workload 5: q, k, v tensor ids 0, 1, 2",
    "hybrid70": "workload 6: q 100 + i, full-layer K/V 1000 + 2i / 1001 + 2i, rings 3000 + 2i / 3001 + 2i, "
                "new K/V 5000 + 2i / 5001 + 2i for layer i",
    "cpu_baseline": "oracle inputs from synth (PCG64) workloads 2, 1, 31, 32, 41, 51, 61",
}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", default="ring,int8,int8sparse,quant,swa,full,chunk4096,chunk8192,sparse,hybrid70,tiny")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="oracle time for the headline (ring) baseline; every other row gets a third of it")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device-to-device copy (the reference kernel for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}): the kernels work on "
              "one GPU's share; how they would shard is described, not implemented", file=sys.stderr)
        return 2
    rows = [r for r in args.rows.split(",") if r]

    import numpy as np
    import torch

    import hybrid_swa_kv_amd as hsk
    from hybrid_swa_kv_amd import _lib, synth

    _lib.load()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] device {torch.cuda.get_device_name(0)}; rows {rows}", file=sys.stderr, flush=True)

    work = {}
    # ---------------------------------------------------------------- setup --
    if "ring" in rows:
        c = RING
        sets = []
        for layer in range(c["layers"]):
            rk = synth.normal_gpu(2, 100 + 2 * layer, (c["B"], c["Hkv"], c["W"], c["D"]))
            rv = synth.normal_gpu(2, 101 + 2 * layer, (c["B"], c["Hkv"], c["W"], c["D"]))
            q = synth.normal_gpu(2, 1000 + layer, (c["B"], c["Hq"], c["D"]))
            kn = synth.normal_gpu(2, 2000 + layer, (c["B"], c["Hkv"], c["D"]))
            vn = synth.normal_gpu(2, 3000 + layer, (c["B"], c["Hkv"], c["D"]))
            sets.append((q, kn, vn, rk, rv, torch.empty_like(q)))
        pos = torch.full((c["B"],), c["ctx"] - 1, dtype=torch.int32, device=dev)
        slots = torch.empty(c["B"], dtype=torch.int32, device=dev)

        def ring_step(sets=sets, pos=pos, slots=slots):
            for (q, kn, vn, rk, rv, out) in sets:
                hsk.swa_decode_ring(q, kn, vn, rk, rv, pos, out=out, slot_out=slots)

        # a decode step is replayed as one HIP graph (no per-launch host overhead)
        ring_step()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ring_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ring_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ring_graph):
            ring_step()
        work["ring"] = ring_graph.replay
    if any(r in rows for r in ("swa", "full", "chunk4096", "chunk8192")):
        c = PREFILL
        pq = synth.normal_gpu(3, synth.Q, (c["L"], c["Hq"], c["D"]))
        pk = synth.normal_gpu(3, synth.K, (c["L"], c["Hkv"], c["D"]))
        pv = synth.normal_gpu(3, synth.V, (c["L"], c["Hkv"], c["D"]))
        pout = torch.empty_like(pq)
        if "swa" in rows:
            work["swa"] = lambda: hsk.swa_prefill(pq, pk, pv, PREFILL["W"], out=pout)
        if "full" in rows:
            work["full"] = lambda: hsk.swa_prefill(pq, pk, pv, 0, out=pout)
        for C in (4096, 8192):
            name = f"chunk{C}"
            if name in rows:
                # the window prefill in chunks of C tokens, each continuing from the ring
                cring_k = torch.empty((1, c["Hkv"], c["W"], c["D"]), dtype=torch.bfloat16, device=dev)
                cring_v = torch.empty_like(cring_k)
                cq, ck, cv, co = pq[None], pk[None], pv[None], pout[None]
                chunk_outs = [torch.empty_like(cq[:, p0:p0 + C]) for p0 in range(0, c["L"], C)]

                def chunk_run(C=C, rk=cring_k, rv=cring_v, outs=chunk_outs):
                    for i, p0 in enumerate(range(0, PREFILL["L"], C)):
                        hsk.swa_prefill_chunk(cq[:, p0:p0 + C], ck[:, p0:p0 + C], cv[:, p0:p0 + C], rk, rv, p0,
                                              out=outs[i])
                work[name] = chunk_run
    if any(r in rows for r in ("quant", "int8", "int8sparse")):
        c = INT8
        t8 = c["ctx"] - c["hot"]
        kx = synth.normal_gpu(4, synth.K, (c["B"], c["Hkv"], c["ctx"], c["D"]), outlier_p=0.01)
        vx = synth.normal_gpu(4, synth.V, (c["B"], c["Hkv"], c["ctx"], c["D"]), outlier_p=0.01)
        kwarm, vwarm = kx[:, :, :t8].contiguous(), vx[:, :, :t8].contiguous()
        khot, vhot = kx[:, :, t8:].contiguous(), vx[:, :, t8:].contiguous()
        del kx, vx
        iq = synth.normal_gpu(4, synth.Q, (c["B"], c["Hq"], c["D"]))
        kc = torch.empty(kwarm.shape, dtype=torch.int8, device=dev)
        vc = torch.empty_like(kc)
        ks = torch.empty((c["B"], c["Hkv"], t8 // 32), dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
        hsk.kv_quant_int8_b32(kwarm, kc, ks)
        hsk.kv_quant_int8_b32(vwarm, vc, vs)
        iout = torch.empty_like(iq)
        iws = torch.empty(hsk.attn_decode_int8kv_workspace_size(c["B"], c["Hq"], c["Hkv"], c["D"], t8, c["hot"]),
                          dtype=torch.uint8, device=dev)
        if "quant" in rows:
            def quant_step():
                hsk.kv_quant_int8_b32(kwarm, kc, ks)
                hsk.kv_quant_int8_b32(vwarm, vc, vs)
            work["quant"] = quant_step
        if "int8" in rows:
            work["int8"] = lambda: hsk.attn_decode_int8kv(iq, kc, ks, vc, vs, khot, vhot, out=iout, workspace=iws)
        if "int8sparse" in rows:
            # the same pool decoded block-sparsely: hot tail + each head's top-64 INT8 blocks
            kmeans = hsk.kv_block_means_int8(kc, ks)
            isel = torch.empty((c["B"], c["Hq"], 64), dtype=torch.int32, device=dev)
            isws = torch.empty(hsk.attn_decode_int8kv_sparse_workspace_size(c["B"], c["Hq"], c["Hkv"], c["D"], t8,
                                                                           c["hot"], 64), dtype=torch.uint8, device=dev)
            work["int8sparse"] = lambda: hsk.attn_decode_int8kv_sparse(iq, kc, ks, vc, vs, kmeans, khot, vhot, topk=64,
                                                                       out=iout, sel=isel, workspace=isws)
    if "sparse" in rows:
        c = SPARSE
        sq = synth.normal_gpu(5, synth.Q, (c["L"], c["Hq"], c["D"]))
        sk = synth.normal_gpu(5, synth.K, (c["L"], c["Hkv"], c["D"]))
        sv = synth.normal_gpu(5, synth.V, (c["L"], c["Hkv"], c["D"]))
        sout = torch.empty_like(sq)
        ssel = torch.empty((c["Hq"], c["L"] // c["block"], c["topk"]), dtype=torch.int32, device=dev)
        sws = torch.empty(hsk.blocksparse_workspace_size(c["L"], c["Hq"], c["Hkv"], c["D"], c["block"], c["topk"]),
                          dtype=torch.uint8, device=dev)
        work["sparse"] = lambda c=c: hsk.blocksparse_select_attend(sq, sk, sv, c["block"], c["topk"], c["W"],
                                                                   out=sout, sel=ssel, workspace=sws)
    if "hybrid70" in rows:
        c = HYBRID
        kinds = hybrid_layers()
        hpos = torch.full((c["B"],), c["ctx"] - 1, dtype=torch.int32, device=dev)
        hslots = torch.empty(c["B"], dtype=torch.int32, device=dev)
        hws = torch.empty(hsk.attn_decode_int8kv_workspace_size(c["B"], c["Hq"], c["Hkv"], c["D"], 0, c["ctx"]),
                          dtype=torch.uint8, device=dev)
        hlayers = []
        for i, full in enumerate(kinds):
            q = synth.normal_gpu(6, 100 + i, (c["B"], c["Hq"], c["D"]))
            if full:   # the layer's whole K/V cache, [B, Hkv, ctx, D]
                kf = synth.normal_gpu(6, 1000 + 2 * i, (c["B"], c["Hkv"], c["ctx"], c["D"]))
                vf = synth.normal_gpu(6, 1001 + 2 * i, (c["B"], c["Hkv"], c["ctx"], c["D"]))
                hlayers.append(("full", q, kf, vf, torch.empty_like(q)))
            else:      # the layer's ring and the new token's K/V
                rk = synth.normal_gpu(6, 3000 + 2 * i, (c["B"], c["Hkv"], c["W"], c["D"]))
                rv = synth.normal_gpu(6, 3001 + 2 * i, (c["B"], c["Hkv"], c["W"], c["D"]))
                kn = synth.normal_gpu(6, 5000 + 2 * i, (c["B"], c["Hkv"], c["D"]))
                vn = synth.normal_gpu(6, 5001 + 2 * i, (c["B"], c["Hkv"], c["D"]))
                hlayers.append(("swa", q, kn, vn, rk, rv, torch.empty_like(q)))

        def run_layer(layer):
            if layer[0] == "full":
                _, q, kf, vf, o = layer
                hsk.attn_decode_int8kv(q, None, None, None, None, kf, vf, out=o, workspace=hws)
            else:
                _, q, kn, vn, rk, rv, o = layer
                hsk.swa_decode_ring(q, kn, vn, rk, rv, hpos, out=o, slot_out=hslots)

        def capture(layers):
            for ly in layers:
                run_layer(ly)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for ly in layers:
                    run_layer(ly)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for ly in layers:
                    run_layer(ly)
            return g

        hybrid_graph = capture(hlayers)
        full_graph = capture([ly for ly in hlayers if ly[0] == "full"])   # the 10 full layers alone
        work["hybrid70"] = hybrid_graph.replay
    if "tiny" in rows:
        c = TINY
        tq = synth.to_torch(synth.token_major(1, synth.Q, c["L"], c["Hq"], c["D"], dtype="f32"), dev)
        tk = synth.to_torch(synth.token_major(1, synth.K, c["L"], c["Hkv"], c["D"], dtype="f32"), dev)
        tv = synth.to_torch(synth.token_major(1, synth.V, c["L"], c["Hkv"], c["D"], dtype="f32"), dev)
        tout = torch.empty_like(tq)
        work["tiny"] = lambda: hsk.swa_prefill(tq, tk, tv, TINY["W"], out=tout)
    if args.calib_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] calibration copy of 1 GiB done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    print("[bench] inputs resident; warming up", file=sys.stderr, flush=True)

    # ----------------------------------------------------------------- timing --
    timer = Timer(torch)

    def step():
        for name in rows:
            timer.run(name, work[name])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] timing", file=sys.stderr, flush=True)
    clock = ClockSampler()
    timer.order.clear()
    clock.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        print(f"[bench] step {i + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
    # wait for each row's end in GPU order, noting when it completes: the engine
    # clock samples between two completions belong to the row that ended second
    windows, prev = [], t0
    for name, ev in timer.order:
        ev.synchronize()
        now = time.perf_counter()
        windows.append((name, prev, now))
        prev = now
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.stop()
    sclk = clock.per_window(windows)
    ms_step = wall * 1e3 / args.steps

    res = {}
    if "ring" in rows:
        ms = timer.mean_ms("ring", args.warmup)
        per_launch_us = ms * 1e3 / RING["layers"]
        gbs = ring_bytes_per_call() / (per_launch_us * 1e-6) / 1e9
        # the same 60 calls launched one by one from Python, for reference
        eager = Timer(torch)
        for _ in range(3):
            eager.run("ring", ring_step)
        torch.cuda.synchronize()
        eager_us = eager.mean_ms("ring", 1) * 1e3 / RING["layers"]
        res["ring"] = {"ms_per_step": round(ms, 4), "us_per_launch": round(per_launch_us, 3),
                       "bytes_per_launch": ring_bytes_per_call(), "GB/s": round(gbs, 1),
                       "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "launch": "hip graph of 60 calls",
                       "eager_us_per_launch": round(eager_us, 3)}
    for name, W in (("swa", PREFILL["W"]), ("full", 0)):
        if name in rows:
            c = PREFILL
            ms = timer.mean_ms(name, args.warmup)
            flops = 4 * c["D"] * c["Hq"] * pairs_prefill(c["L"], W)
            tf = flops / (ms * 1e-3) / 1e12
            res[name] = {"ms": round(ms, 3), "flop": flops, "TFLOP/s": round(tf, 1),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    if "swa" in rows and "full" in rows:
        res["full_over_swa_flop_ratio"] = round(res["full"]["flop"] / res["swa"]["flop"], 4)
    for C in (4096, 8192):
        name = f"chunk{C}"
        if name in rows:
            c = PREFILL
            ms = timer.mean_ms(name, args.warmup)
            flops = 4 * c["D"] * c["Hq"] * pairs_prefill(c["L"], c["W"])
            tf = flops / (ms * 1e-3) / 1e12
            res[name] = {"ms": round(ms, 3), "chunks": c["L"] // C, "flop": flops, "TFLOP/s": round(tf, 1),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    if "quant" in rows:
        ms = timer.mean_ms("quant", args.warmup)
        gbs = int8_quant_bytes() / (ms * 1e-3) / 1e9
        res["quant"] = {"ms": round(ms, 4), "bytes": int8_quant_bytes(), "GB/s": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if "int8" in rows:
        ms = timer.mean_ms("int8", args.warmup)
        gbs = int8_decode_bytes() / (ms * 1e-3) / 1e9
        res["int8"] = {"ms": round(ms, 4), "bytes": int8_decode_bytes(), "GB/s": round(gbs, 1),
                       "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if "int8sparse" in rows:
        ms = timer.mean_ms("int8sparse", args.warmup)
        nb = int8_sparse_bytes(isel.cpu().numpy())
        gbs = nb / (ms * 1e-3) / 1e9
        res["int8sparse"] = {"ms": round(ms, 4), "topk_blocks": 64, "bytes": nb, "GB/s": round(gbs, 1),
                             "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                             "vs_dense_bytes": round(nb / int8_decode_bytes(), 4)}
    if "sparse" in rows:
        c = SPARSE
        ms = timer.mean_ms("sparse", args.warmup)
        pairs = sparse_pairs(ssel.cpu().numpy(), c["L"], c["block"], c["W"])  # exact, from sel
        flops = 4 * c["D"] * pairs
        tf = flops / (ms * 1e-3) / 1e12
        sel_np = ssel.cpu().numpy()
        tb = sparse_tile_bytes(sel_np, c["L"], c["block"], c["W"], c["Hkv"], c["D"])
        res["sparse"] = {"ms": round(ms, 3), "visible_pairs": pairs, "flop": flops, "TFLOP/s": round(tf, 1),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                         "kv_tile_bytes": tb, "kv_tile_GB/s": round(tb / (ms * 1e-3) / 1e9, 1)}

    if "tiny" in rows:
        c = TINY
        ms = timer.mean_ms("tiny", args.warmup)
        flops = 4 * c["D"] * c["Hq"] * pairs_prefill(c["L"], c["W"])
        res["tiny"] = {"us": round(ms * 1e3, 2), "flop": flops, "dtype": "f32",
                       "note": "correctness-sized fp32 window prefill (L 512, 2/2 heads, head_dim 64, "
                               "window 128): absolute time only"}
    if "hybrid70" in rows:
        c = HYBRID
        ms = timer.mean_ms("hybrid70", args.warmup)
        nfull = sum(hybrid_layers())
        nswa = c["layers"] - nfull
        step_bytes = nswa * ring_bytes_per_call() + nfull * full_decode_bytes()
        # the full layers alone, to price an all-full 70-layer step
        ft = Timer(torch)
        for _ in range(3):
            ft.run("full", full_graph.replay)
        torch.cuda.synchronize()
        full_us = ft.mean_ms("full", 1) * 1e3 / nfull
        all_full_bytes = c["layers"] * full_decode_bytes()
        gbs = step_bytes / (ms * 1e-3) / 1e9
        res["hybrid70"] = {"ms_per_step": round(ms, 4), "layers": f"{nswa} swa (W {c['W']}) + {nfull} full",
                           "bytes_per_step": step_bytes, "GB/s": round(gbs, 1),
                           "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                           "full_layer_us": round(full_us, 2),
                           "kv_bytes_ratio_vs_all_full": round(step_bytes / all_full_bytes, 4),
                           "time_ratio_vs_all_full": round(ms * 1e3 / (c["layers"] * full_us), 4)}

    # the engine clock sampled while each row ran in the timed steps
    for name, st in sclk.items():
        if name in res and isinstance(res[name], dict):
            res[name]["sclk_mhz"] = st
    # spread of the timed calls (per launch for the ring row, whose step is 60 launches)
    for name in rows:
        if name in res and isinstance(res[name], dict):
            per = RING["layers"] if name == "ring" else 1
            res[name]["per_launch_ms" if name == "ring" else "call_ms"] = timer.spread(name, args.warmup, per)

    line = {
        "metric": METRIC,
        "value": res["ring"]["GB/s"] if "ring" in res else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swa_ring_decode", "batch": RING["B"], "context": RING["ctx"],
                   "q_heads": RING["Hq"], "kv_heads": RING["Hkv"], "head_dim": RING["D"],
                   "window": RING["W"], "ring_sets_per_step": RING["layers"],
                   "value_basis": "KV bytes of the ring-decode launches / their HIP-event time; "
                                  "ms_per_step covers every row"},
    }
    if "ring" in res:
        line["roofline"] = {"kernel": "ring_decode_kernel", "bound": "hbm",
                            "achieved": res["ring"]["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": res["ring"]["frac_hbm_peak"], "traffic": recorded_traffic()}
    line["rows"] = res
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                      "compute_units": props.multi_processor_count,
                      "peaks_used": {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                                     "basis": "256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk; 8 TB/s HBM3E"}}
    line["host"] = host_info()
    line["source"] = source_info()
    line["seeds"] = SEEDS
    if not args.no_cpu:
        # the oracle beside every row, on the host, one thread (rank 0, one GPU)
        per = args.cpu_seconds / 3
        for name in rows:
            if name not in res or not isinstance(res[name], dict):
                continue
            print(f"[bench] cpu baseline (oracle): {name}", file=sys.stderr, flush=True)
            if name == "ring":
                b = cpu_ring(args.cpu_seconds)
            elif name == "tiny":
                b = cpu_tiny(per)
            elif name in ("swa", "full"):
                b = cpu_prefill(name, per)
            elif name.startswith("chunk"):
                b = cpu_chunk(int(name[5:]), per)
            elif name in ("quant", "int8", "int8sparse"):
                b = cpu_int8(name, per)
            elif name == "sparse":
                b = cpu_sparse(per, res["sparse"]["visible_pairs"])
            elif name == "hybrid70":
                ring_us = res.get("ring", {}).get("cpu_baseline", {}).get("us_per_call")
                if ring_us is None:
                    ring_us = cpu_ring(per)["us_per_call"]
                b = cpu_hybrid(per, ring_us)
            else:
                continue
            res[name]["cpu_baseline"] = b
        if "ring" in res:
            line["cpu_baseline"] = res["ring"]["cpu_baseline"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
