#!/usr/bin/env python3
"""Decode-time quantized matvec benchmark on one MI355X.

A step is one batch-1 decode token of the 8B Llama-shaped layer set in Q8_0:
32 layers x (q 4096x4096, k/v 1024x4096, o 4096x4096, gate/up 14336x4096,
down 4096x14336) + lm_head 128256x4096 = 225 matvecs, 7,973,699,584 bytes of
weights, every matrix in its own device buffer (the working set is ~31x the
256 MB last-level cache, so every step streams from HBM).  Weights are drawn
N(0, 0.02^2) and encoded per 32-weight block; activations N(0, 1).  The
matvecs run in decode dependency order, one launch per dependency level:
q||k||v (one input) in one qmv_chain call, then o, gate||up (one input) in
one call, down, and lm_head (129 launches).  The step is captured once as a
HIP graph and replayed.

Output: one JSON line per extra workload ("sweep") on stdout as it finishes,
each with the oracle's time on the host for the same workload; the full
per-matrix tables on stderr (and in --detail FILE); and, last, one compact
JSON line with the headline: the step's achieved GB/s (algorithmic weight +
activation + output bytes / wall time, whole job), the equivalent decode
tok/s, a roofline object for the dominant kernel measured with HIP events
on the launch stream, the measured stream-read ceiling, the oracle's time
on the host (cpu_baseline) and a one-number summary per sweep.

Extra workloads: the Q8_0 1024 x 1024 matvec over 480 rotated copies (so
every call reads HBM), Q4_0 / Q4_1 / Q4_K / Q6_K at batch 1, 2, 4, 8, the int8 requant path
on Qwen3-0.6B shapes and the MoE expert path (plain and fused) at batch
1, 2, 4, 8, with Q4_K experts (plain and fused) at batch 1 and 8.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweeps all|none|a,b] [--detail FILE]
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20     # MI355X last-level (Infinity) cache
LABEL_BATCHES = 5         # per-label timing: median of 5 batches (p10/p90 = min/max of 5)

# HBM traffic per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE runs
# (copy-calibrated: FETCH x2.0, WRITE x1.0; one counter per run), recorded
# per kernel family for the sources with this SHA-256 (of the files in
# order) and reported as null once a source differs (the kernel changed
# since the counters were taken).  "ratio": traffic / algorithmic bytes on
# the workload named; the summaries are in profiles/*_hbm_counters.md.
_IMPL = ["bandwidth_bound_block_amd/csrc/qmv_blocks_impl.h", "bandwidth_bound_block_amd/csrc/qmv_block_decode.h",
         "bandwidth_bound_block_amd/csrc/qmv_host.h"]
TRAFFIC_RECORDS = {
    # the dominant kernel of the decode step, in the step's 32:32:32:1 mix
    # of q+k+v, o, gate+up and lm_head launches: bytes per launch
    "qmv_kernel_c<Q8_0, 2, 8, 2, float, 1>": {
        "key": "kernel_c_q8_0",
        "sources": _IMPL + ["bandwidth_bound_block_amd/csrc/qmv_fmt_q8_0.hip"],
        "sha256": "aa19641f66816f500969c8e79d12c4dff372c82fcf2ca6061f80f4bbb7c36ca8", "bytes_per_launch": 61898701, "ratio": 1.0033,
        "workload": "8B Q8_0 decode step, batch 1"},
    "qmv_kernel_c<Q8_0, 4, 16, 2, float, 1>": {
        "key": "kernel_c16_q8_0_down",
        "sources": _IMPL + ["bandwidth_bound_block_amd/csrc/qmv_fmt_q8_0.hip"],
        "sha256": "aa19641f66816f500969c8e79d12c4dff372c82fcf2ca6061f80f4bbb7c36ca8", "ratio": 1.0079, "workload": "8B Q8_0 down (4096 x 14336), batch 1"},
    "i8_stream_kernel": {
        "key": "i8_stream",
        "sources": ["bandwidth_bound_block_amd/csrc/qmv_int8.hip", "bandwidth_bound_block_amd/csrc/qmv_host.h"],
        "sha256": "e1adefc3766601d9ed03a988e2885af680da6d56e109ad0b2654c87a37676d21", "ratio": 1.0380,
        "workload": "Qwen3-0.6B int8 step (28 layers + lm_head), batch 1, per-matrix launches"},
}


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, field="ratio"):
    rec = TRAFFIC_RECORDS.get(kernel)
    if rec is None:
        return None
    try:
        h = sources_sha256(rec["sources"])
    except OSError:
        return None
    return rec.get(field) if h == rec["sha256"] else None


METRIC = "achieved HBM GB/s (% of MI355X peak) for batch-1 quant matvec; equiv. decode tok/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- sweeps
_FLOAT_CACHE = {}
_ENC_CACHE = {}


def encoded(wl, fmt, tag, N, K):
    """Seeded weights for (tag, N, K) encoded as fmt; the float draw is
    shared by the formats (the same draw as workloads.quant_weights)."""
    key = (fmt, tag, N, K)
    if key not in _ENC_CACHE:
        fk = (tag, N, K)
        if fk not in _FLOAT_CACHE:
            _FLOAT_CACHE[fk] = wl.weights_f32(tag, N, K)
        _ENC_CACHE[key] = wl.ENCODERS[fmt](_FLOAT_CACHE[fk])
    return _ENC_CACHE[key]


class Sweep:
    """A list of independent launches making up one step, with the bytes
    each launch must move (weights once, activations once, outputs once)."""

    def __init__(self, name, batch):
        self.name = name
        self.batch = batch
        self.launches = []      # (label, cfunc, args_without_stream, bytes)
        self.keep = []          # device tensors kept alive

    def add(self, label, cfn, args, nbytes):
        self.launches.append((label, cfn, tuple(args), int(nbytes)))

    @property
    def bytes_per_step(self):
        return sum(l[3] for l in self.launches)

    def run(self, stream_ptr):
        s = ctypes.c_void_p(stream_ptr)
        for label, cfn, args, _ in self.launches:
            rc = cfn(*args, s)
            if rc != 0:
                import bandwidth_bound_block_amd as qmv
                raise RuntimeError(f"{self.name}/{label}: rc={rc}: {qmv.last_error()}")


def _dense_sweep(torch, qmv, wl, fmt, batch, layers, layer_mats, head, tagbase, name, fuse=None):
    """fuse: optional list of (fused_name, [member names]) whose rows are
    stored concatenated (same input vector), e.g. q||k||v and gate||up."""
    import numpy as np
    cfn = {"q8_0": qmv.lib().qmv_q8_0, "q4_0": qmv.lib().qmv_q4_0, "q4_1": qmv.lib().qmv_q4_1,
           "q4_k": qmv.lib().qmv_q4_k, "q6_k": qmv.lib().qmv_q6_k}[fmt]
    sw = Sweep(name, batch)
    dev = "cuda:0"
    t0 = time.time()
    mats = {}
    enc = {m: encoded(wl, fmt, f"{tagbase}/{m}", N, K) for m, N, K in layer_mats + [head]}
    shapes = {m: (N, K) for m, N, K in layer_mats}
    if fuse:
        merged = []
        used = set()
        for fname, members in fuse:
            N = sum(shapes[m][0] for m in members)
            K = shapes[members[0]][1]
            enc[fname] = np.concatenate([enc[m] for m in members], axis=0)   # rows of an encoded matrix are independent
            merged.append((fname, N, K))
            used |= set(members)
        layer_mats = []
        for m, N, K in wl.LLAMA8B_LAYER if tagbase == "llama8b" else []:
            if m not in used:
                layer_mats.append((m, N, K))
            else:
                for fname, members in fuse:
                    if members[0] == m:
                        layer_mats.append([t for t in merged if t[0] == fname][0])
    for mname, N, K in layer_mats + [head]:
        mats[mname] = torch.from_numpy(enc[mname]).to(dev)
    log(f"[{name}] encoded weights in {time.time() - t0:.1f}s")
    xs = {}
    for layer in range(layers + 1):
        for K in sorted({m[2] for m in layer_mats + [head]}):
            xs[(layer, K)] = torch.from_numpy(wl.activations(f"{tagbase}/x/{layer}/{K}/{batch}", batch, K)).to(dev)
    for layer in range(layers):
        for mname, N, K in layer_mats:
            W = mats[mname].clone()          # every layer in its own buffer
            y = torch.empty((batch, N), dtype=torch.float32, device=dev)
            x = xs[(layer, K)]
            sw.keep += [W, y]
            nbytes = W.numel() + 4 * batch * K + 4 * batch * N
            sw.add(mname, cfn, (W.data_ptr(), N, K, x.data_ptr(), K, batch, y.data_ptr(), N), nbytes)
    mname, N, K = head
    W = mats[mname]
    y = torch.empty((batch, N), dtype=torch.float32, device=dev)
    x = xs[(layers, K)]
    sw.keep += [W, y, xs]
    sw.add(mname, cfn, (W.data_ptr(), N, K, x.data_ptr(), K, batch, y.data_ptr(), N),
           W.numel() + 4 * batch * K + 4 * batch * N)
    sw.keep.append(mats)
    return sw


FUSED_8B = [("qkv", ["q", "k", "v"]), ("gate_up", ["gate", "up"])]


def build_llama(torch, qmv, wl, fmt, batch, fused=False):
    return _dense_sweep(torch, qmv, wl, fmt, batch, wl.LLAMA8B_LAYERS, wl.LLAMA8B_LAYER, wl.LLAMA8B_LM_HEAD,
                        "llama8b", f"llama8b_{fmt}{'_fused' if fused else ''}_b{batch}",
                        FUSED_8B if fused else None)


# Stages that read outputs of earlier stages in a decode step (the others
# share their input with the stage before them).
DECODE_WAITS = {"q": 1, "k": 0, "v": 0, "qkv": 1, "o": 1, "gate": 1, "up": 0, "gate_up": 1, "down": 1,
                "lm_head": 1}


def build_llama_chain(torch, qmv, wl, fmt, fused=False):
    """The batch-1 8B decode step as one qmv_chain call: the same matrices,
    buffers and order as build_llama, with a stage barrier wherever a decode
    step has a data dependency (q/qkv, o, gate/gate_up, down, lm_head)."""
    dense = build_llama(torch, qmv, wl, fmt, 1, fused=fused)
    sw = Sweep(dense.name.replace("_b1", "_chain_b1"), 1)
    sw.keep = dense.keep
    arr = (qmv.ChainStage * len(dense.launches))()
    total = 0
    for i, (label, _, args, nb) in enumerate(dense.launches):
        Wp, N, K, xp, _, _, yp, _ = args
        arr[i] = qmv.ChainStage(Wp, xp, yp, N, K, DECODE_WAITS[label], 0)
        total += nb
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    sw.keep += [arr, ws]
    sw.add("chain", qmv.lib().qmv_chain,
           (qmv.FORMATS[fmt], ctypes.cast(arr, ctypes.c_void_p), len(arr), ws.data_ptr(), ws.numel()), total)
    sw.workspace = ws
    return sw


# Matvecs of a decode step that share their input and do not depend on one
# another: one qmv_chain call each (no stage waits inside a group).
DECODE_GROUPS = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",))]


def build_llama_grouped(torch, qmv, wl, fmt):
    """The batch-1 8B decode step with the separate matrices and buffers of
    build_llama, launched in dependency order with one launch per
    dependency level: q, k and v (one input) in one qmv_chain call; o;
    gate and up (one input, o's output) in one call; down; then lm_head."""
    dense = build_llama(torch, qmv, wl, fmt, 1, fused=False)
    sw = Sweep(dense.name.replace("_b1", "_grouped_b1"), 1)
    sw.keep = dense.keep
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    sw.keep.append(ws)
    sw.workspace = ws
    by_label = {}
    per_layer = [l for l in dense.launches if l[0] != "lm_head"]
    order = [m for _, ms in DECODE_GROUPS for m in ms]
    nl = len(per_layer) // len(order)
    for layer in range(nl):
        mats = {l[0]: l for l in per_layer[layer * len(order):(layer + 1) * len(order)]}
        for gname, members in DECODE_GROUPS:
            if len(members) == 1:
                label, cfn, args, nb = mats[members[0]]
                sw.add(label, cfn, args, nb)
                continue
            arr = (qmv.ChainStage * len(members))()
            total = 0
            for i, m in enumerate(members):
                _, _, (Wp, N, K, xp, _, _, yp, _), nb = mats[m]
                arr[i] = qmv.ChainStage(Wp, xp, yp, N, K, 0, 0)
                total += nb - (4 * K if i > 0 else 0)   # the members share x: it is read once
            sw.keep.append(arr)
            sw.add(gname, qmv.lib().qmv_chain,
                   (qmv.FORMATS[fmt], ctypes.cast(arr, ctypes.c_void_p), len(members), ws.data_ptr(), ws.numel()),
                   total)
    for l in dense.launches:
        if l[0] == "lm_head":
            sw.add(*l)
    return sw


C1_COPIES = 480      # 480 x 1,114,112 B = 535 MB, over twice the 256 MB last-level cache


def build_c1(torch, qmv, wl):
    """The Q8_0 1024 x 1024 batch-1 matvec, one launch per distinct copy of
    the matrix (480 copies, so every launch reads its weights from HBM)."""
    N = K = 1024
    sw = Sweep("q8_0_1024_b1", 1)
    dev = "cuda:0"
    W0 = torch.from_numpy(wl.quant_weights("q8_0", "c1/W", N, K)).to(dev)
    x = torch.from_numpy(wl.activations("c1/x", 1, K)).to(dev)
    cfn = qmv.lib().qmv_q8_0
    for _ in range(C1_COPIES):
        W = W0.clone()
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        sw.keep += [W, y]
        sw.add("q8_0_1024", cfn, (W.data_ptr(), N, K, x.data_ptr(), K, 1, y.data_ptr(), N), W.numel() + 4 * K + 4 * N)
    sw.keep.append(x)
    return sw


FUSED_QWEN = [("qkv", ["q", "k", "v"]), ("gate_up", ["gate", "up"])]


def build_int8(torch, qmv, wl, fused=False):
    """28 Qwen3-0.6B-shaped int8 layers + the tied lm_head at batch 1.  With
    fused, q||k||v and gate||up are stored row-concatenated (weights and
    per-row mult/shift) and run as one launch each: 113 launches instead of
    197 (a caller layout choice; the kernel and ABI are the same)."""
    sw = Sweep(f"qwen06b_int8{'_fused' if fused else ''}_b1", 1)
    dev = "cuda:0"
    cfn = qmv.lib().qmv_i8_requant
    mats = {}
    for mname, N, K in wl.QWEN06B_LAYER + [wl.QWEN06B_LM_HEAD]:
        W = torch.from_numpy(wl.int8_uniform(f"qwen/W/{mname}", (N, K))).to(dev)
        mult, shift = wl.requant_params(f"qwen/ms/{mname}", N)
        mats[mname] = (W, torch.from_numpy(mult).to(dev), torch.from_numpy(shift).to(dev))
    layer_list = list(wl.QWEN06B_LAYER)
    if fused:
        shapes = {m: (N, K) for m, N, K in wl.QWEN06B_LAYER}
        layer_list = []
        groups = {g: members for g, members in FUSED_QWEN}
        done = set()
        for mname, N, K in wl.QWEN06B_LAYER:
            g = next((g for g, mem in FUSED_QWEN if mname in mem), None)
            if g is None:
                layer_list.append((mname, N, K))
            elif g not in done:
                mem = groups[g]
                mats[g] = tuple(torch.cat([mats[m][i] for m in mem]) for i in range(3))
                layer_list.append((g, sum(shapes[m][0] for m in mem), K))
                done.add(g)
    # the gate projection's output goes through a frozen SiLU table (the
    # page's integer engine applies SiLU that way); in the row-fused layout
    # gate and up share one launch, so there the table step is not applied
    lut = torch.from_numpy(wl.int8_table("qwen/silu_table")).to(dev)
    sw.keep.append(lut)
    for layer in range(wl.QWEN06B_LAYERS + 1):
        mlist = layer_list if layer < wl.QWEN06B_LAYERS else [wl.QWEN06B_LM_HEAD]
        for mname, N, K in mlist:
            W0, mult, shift = mats[mname]
            W = W0.clone() if layer < wl.QWEN06B_LAYERS else W0
            x = torch.from_numpy(wl.int8_uniform(f"qwen/x/{layer}/{mname}", (1, K))).to(dev)
            y = torch.empty((1, N), dtype=torch.int8, device=dev)
            sw.keep += [W, x, y, mult, shift]
            if mname == "gate":
                sw.add(mname, qmv.lib().qmv_i8_requant_lut,
                       (W.data_ptr(), N, K, x.data_ptr(), K, 1, mult.data_ptr(), shift.data_ptr(), lut.data_ptr(),
                        y.data_ptr(), N), N * K + K + 8 * N + N)
            else:
                sw.add(mname, cfn, (W.data_ptr(), N, K, x.data_ptr(), K, 1, mult.data_ptr(), shift.data_ptr(),
                                    y.data_ptr(), N), N * K + K + 8 * N + N)
    return sw


def build_moe(torch, qmv, wl, batch, fmt="q4_0"):
    """48 MoE layers: per layer one launch for gate||up (each expert's gate
    and up rows concatenated, 1536 x 2048) and one for down (2048 x 768, one
    input per token and slot).  Bytes count each distinct routed expert once."""
    import numpy as np
    sw = Sweep(f"moe30b_{fmt}_b{batch}", batch)
    dev = "cuda:0"
    cfn = qmv.lib().qmv_moe
    fcode = qmv.FORMATS[fmt]
    E, T, H, F = wl.MOE_EXPERTS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    t0 = time.time()
    key = f"moe_{fmt}"
    if key not in _ENC_CACHE:
        gate = wl.quant_weights(fmt, "moe/gate", E * F, H).reshape(E, -1)
        up = wl.quant_weights(fmt, "moe/up", E * F, H).reshape(E, -1)
        _ENC_CACHE[key] = (np.concatenate([gate, up], axis=1).reshape(-1),
                           wl.quant_weights(fmt, "moe/down", E * H, F).reshape(-1))
    gu = torch.from_numpy(_ENC_CACHE[key][0]).to(dev)
    down = torch.from_numpy(_ENC_CACHE[key][1]).to(dev)
    log(f"[moe {fmt}] experts ready in {time.time() - t0:.1f}s")
    gu_stride = 2 * wl.block_bytes(fmt, F, H)
    dn_stride = wl.block_bytes(fmt, H, F)
    uniq = []
    for layer in range(wl.MOE_LAYERS):
        ids_np = wl.moe_ids(f"moe/ids/{layer}/{batch}", batch, T, E)
        nu = len(np.unique(ids_np))
        uniq.append(nu)
        ids = torch.from_numpy(ids_np).to(dev)
        Wgu, Wdn = gu.clone(), down.clone()
        x = torch.from_numpy(wl.activations(f"moe/x/gu/{layer}/{batch}", batch, H)).to(dev)
        ygu = torch.empty((batch, T, 2 * F), dtype=torch.float32, device=dev)
        xd = torch.from_numpy(wl.activations(f"moe/x/dn/{layer}/{batch}", batch * T, F)).to(dev)
        yd = torch.empty((batch, T, H), dtype=torch.float32, device=dev)
        sw.keep += [ids, Wgu, Wdn, x, ygu, xd, yd]
        sw.add("gate_up", cfn, (fcode, Wgu.data_ptr(), gu_stride, E, 2 * F, H, ids.data_ptr(), batch, T,
                                x.data_ptr(), H, 0, ygu.data_ptr()),
               nu * gu_stride + 4 * batch * H + 4 * batch * T * 2 * F + 4 * batch * T)
        sw.add("down", cfn, (fcode, Wdn.data_ptr(), dn_stride, E, H, F, ids.data_ptr(), batch, T,
                             xd.data_ptr(), T * F, F, yd.data_ptr()),
               nu * dn_stride + 4 * batch * T * F + 4 * batch * T * H + 4 * batch * T)
    sw.mean_unique = float(np.mean(uniq))
    return sw


def build_moe_block(torch, qmv, wl, batch, fmt="q4_0"):
    """48 MoE blocks with the steps around the expert matvecs fused: per
    layer qmv_moe_swiglu over gate||up (h = SiLU(gate x) * (up x), 768 per
    slot) and qmv_moe_combine over down (out = sum_s w_s * down_s h_s),
    the second reading the first's output.  Bytes count each distinct
    routed expert once (the method's bytes); the combine kernel reads an
    expert once per token routed to it."""
    import numpy as np
    sw = Sweep(f"moe30b_block_{fmt}_b{batch}", batch)
    dev = "cuda:0"
    fcode = qmv.FORMATS[fmt]
    E, T, H, F = wl.MOE_EXPERTS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    key = f"moe_{fmt}"
    if key not in _ENC_CACHE:
        gate = wl.quant_weights(fmt, "moe/gate", E * F, H).reshape(E, -1)
        up = wl.quant_weights(fmt, "moe/up", E * F, H).reshape(E, -1)
        _ENC_CACHE[key] = (np.concatenate([gate, up], axis=1).reshape(-1),
                           wl.quant_weights(fmt, "moe/down", E * H, F).reshape(-1))
    gu = torch.from_numpy(_ENC_CACHE[key][0]).to(dev)
    down = torch.from_numpy(_ENC_CACHE[key][1]).to(dev)
    gu_stride = 2 * wl.block_bytes(fmt, F, H)
    dn_stride = wl.block_bytes(fmt, H, F)
    uniq = []
    for layer in range(wl.MOE_LAYERS):
        ids_np = wl.moe_ids(f"moe/ids/{layer}/{batch}", batch, T, E)
        nu = len(np.unique(ids_np))
        uniq.append(nu)
        ids = torch.from_numpy(ids_np).to(dev)
        w = torch.from_numpy(wl.router_weights(f"moe/w/{layer}/{batch}", batch, T)).to(dev)
        Wgu, Wdn = gu.clone(), down.clone()
        x = torch.from_numpy(wl.activations(f"moe/x/gu/{layer}/{batch}", batch, H)).to(dev)
        h = torch.empty((batch, T, F), dtype=torch.float32, device=dev)
        out = torch.empty((batch, H), dtype=torch.float32, device=dev)
        sw.keep += [ids, w, Wgu, Wdn, x, h, out]
        sw.add("swiglu", qmv.lib().qmv_moe_swiglu,
               (fcode, Wgu.data_ptr(), gu_stride, E, F, H, ids.data_ptr(), batch, T, x.data_ptr(), H, 0, h.data_ptr()),
               nu * gu_stride + 4 * batch * H + 4 * batch * T * F + 4 * batch * T)
        sw.add("combine", qmv.lib().qmv_moe_combine,
               (fcode, Wdn.data_ptr(), dn_stride, E, H, F, ids.data_ptr(), w.data_ptr(), batch, T, h.data_ptr(), T * F, F,
                out.data_ptr()),
               nu * dn_stride + 4 * batch * T * F + 4 * batch * H + 8 * batch * T)
    sw.mean_unique = float(np.mean(uniq))
    return sw


# ---------------------------------------------------------------- timing
def time_sweep(torch, sw, steps, warmup, use_graph=True):
    """Wall clock and HIP-event timings of a sweep.

    Timed region: `steps` replays of the step's HIP graph (or eager launches)
    bracketed by synchronize, with events on the launch stream around them.
    Per matrix: the launches of that matrix (the per-layer copies, so each is
    cache-cold), repeated to >= 100 per batch where the copies exceed twice
    the last-level cache, back to back between two events on the launch
    stream; the median of 5 batches (with their min and max as p10 / p90).
    The per-launch time includes the gaps between launches."""
    stream = torch.cuda.current_stream()
    for _ in range(max(1, warmup)):
        sw.run(stream.cuda_stream)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                sw.run(torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            for _ in range(2):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: time eager launches
            log(f"[{sw.name}] graph capture failed ({e}); timing eager launches")
            graph = None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        if graph is not None:
            graph.replay()
        else:
            sw.run(stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1) / steps

    by_label = {}
    for label, cfn, args, nb in sw.launches:
        e = by_label.setdefault(label, {"launches": [], "bytes": 0})
        e["launches"].append((cfn, args))
        e["bytes"] += nb
    s = ctypes.c_void_p(stream.cuda_stream)
    per = {}
    for label, e in by_label.items():
        n = len(e["launches"])
        # passes over the label's copies per batch: enough for >= 100 launches
        # where the copies together exceed twice the 256 MB last-level cache
        # (so a repeat is still cache-cold); one pass otherwise
        passes = -(-100 // n) if e["bytes"] > LLC_BYTES * 2 else 1
        per_batch = []
        for _ in range(LABEL_BATCHES):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(passes):
                for cfn, args in e["launches"]:
                    cfn(*args, s)
            b.record(stream)
            torch.cuda.synchronize()
            per_batch.append(a.elapsed_time(b) / (passes * n) * 1e3)   # us per launch
        per_batch.sort()
        med = per_batch[len(per_batch) // 2]
        per[label] = {"launches": n, "us_per_launch": med, "bytes_per_launch": e["bytes"] // n,
                      "gbs": e["bytes"] / n / (med * 1e-6) / 1e9,
                      "us_p10": per_batch[0], "us_p90": per_batch[-1], "launches_per_batch": passes * n}
    kernel_ms = sum(v["us_per_launch"] * v["launches"] for v in per.values()) / 1e3
    ms_step = wall / steps * 1e3
    bps = sw.bytes_per_step
    out = {
        "steps": steps, "graph": graph is not None,
        "launches_per_step": len(sw.launches), "bytes_per_step": bps,
        "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu_ms,
        "gbs_wall": bps / (ms_step * 1e-3) / 1e9,
        "gbs_gpu": bps / (gpu_ms * 1e-3) / 1e9,
        "kernel_ms_per_step": kernel_ms,
        "gbs_kernel": bps / (kernel_ms * 1e-3) / 1e9,
        "tok_s_wall": sw.batch / (ms_step * 1e-3),
        "tok_s_kernel": sw.batch / (kernel_ms * 1e-3),
        "per_matrix": per,
    }
    out["pct_peak_wall"] = 100 * out["gbs_wall"] / PEAK_GBS
    out["pct_peak_kernel"] = 100 * out["gbs_kernel"] / PEAK_GBS
    return out


# ---------------------------------------------------------------- CPU baseline
def read_ceiling(torch, qmv, nbytes=4 << 30, reps=7):
    """The device's stream-read ceiling: qmv_stream_read over a 4 GiB buffer
    (16-byte non-temporal loads, the load form of the whole-line matvec
    kernel), each launch timed with HIP events on the launch stream.  A
    measured denominator reported beside the 8 TB/s spec."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    out = torch.empty(1 << 20, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    for _ in range(2):
        qmv.qmv_stream_read(buf, out, st)
    secs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        qmv.qmv_stream_read(buf, out, st)
        e1.record(st)
        e1.synchronize()
        secs.append(e0.elapsed_time(e1) * 1e-3)
    del buf, out
    torch.cuda.empty_cache()
    med = sorted(secs)[len(secs) // 2]
    return {"value": nbytes / med / 1e9, "best": nbytes / min(secs) / 1e9, "unit": "GB/s", "bytes": nbytes,
            "frac_of_peak": nbytes / med / 1e9 / PEAK_GBS, "launches": reps, "statistic": "median",
            "kernel": "stream_read_kernel (qmv_stream_read)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def oracle_dense(wl, fmt, batch=1, layers_timed=None):
    """The oracle (single-threaded C, fp64 dequantize-then-dot) on one full
    batch-`batch` token of the 8B layer set in fmt: the 7 matrices of a layer
    timed once each and counted 32 times (the oracle's time does not depend
    on the values) plus the full lm_head.  Returns (seconds per token,
    bytes per token)."""
    import oracle
    secs, nbytes = 0.0, 0
    for mname, N, K in wl.LLAMA8B_LAYER:
        W = encoded(wl, fmt, f"llama8b/{mname}", N, K)
        x = wl.activations(f"llama8b/x/0/{K}/{batch}", batch, K)
        secs += wl.LLAMA8B_LAYERS * _timed(lambda: oracle.matvec(fmt, W, N, K, x))
        nbytes += wl.LLAMA8B_LAYERS * (W.size + 4 * batch * (K + N))
    mname, N, K = wl.LLAMA8B_LM_HEAD
    W = encoded(wl, fmt, f"llama8b/{mname}", N, K)
    x = wl.activations(f"llama8b/x/{wl.LLAMA8B_LAYERS}/{K}/{batch}", batch, K)
    secs += _timed(lambda: oracle.matvec(fmt, W, N, K, x))
    nbytes += W.size + 4 * batch * (K + N)
    return secs, nbytes


def oracle_c1(wl):
    import oracle
    N = K = 1024
    W = wl.quant_weights("q8_0", "c1/W", N, K)
    x = wl.activations("c1/x", 1, K)
    reps = 20
    secs = _timed(lambda: [oracle.matvec("q8_0", W, N, K, x) for _ in range(reps)]) / reps
    return secs, W.size + 8 * K


def oracle_int8(wl):
    """One int8 token: 28 layers (one layer's matrices timed, counted 28
    times) plus the tied lm_head, with requant."""
    import oracle
    secs, nbytes = 0.0, 0
    for mname, N, K in wl.QWEN06B_LAYER:
        W = wl.int8_uniform(f"qwen/W/{mname}", (N, K))
        mult, shift = wl.requant_params(f"qwen/ms/{mname}", N)
        x = wl.int8_uniform(f"qwen/x/0/{mname}", (1, K))
        secs += wl.QWEN06B_LAYERS * _timed(lambda: oracle.matvec_i8(W, x, mult, shift))
        nbytes += wl.QWEN06B_LAYERS * (N * K + K + 9 * N)
    mname, N, K = wl.QWEN06B_LM_HEAD
    W = wl.int8_uniform(f"qwen/W/{mname}", (N, K))
    mult, shift = wl.requant_params(f"qwen/ms/{mname}", N)
    x = wl.int8_uniform(f"qwen/x/{wl.QWEN06B_LAYERS}/{mname}", (1, K))
    secs += _timed(lambda: oracle.matvec_i8(W, x, mult, shift))
    nbytes += N * K + K + 9 * N
    return secs, nbytes


def oracle_moe(wl, batch):
    """One MoE step at `batch` tokens: one layer's gate||up and down calls
    (128 Q4_0 experts, top-8) timed and counted 48 times.  The oracle loops
    over (token, slot) pairs, so it reads an expert once per pair."""
    import numpy as np
    import oracle
    E, T, H, F = wl.MOE_EXPERTS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    gate = wl.quant_weights("q4_0", "moe/gate", E * F, H).reshape(E, -1)
    up = wl.quant_weights("q4_0", "moe/up", E * F, H).reshape(E, -1)
    gu = np.concatenate([gate, up], axis=1).reshape(-1)
    dn = wl.quant_weights("q4_0", "moe/down", E * H, F).reshape(-1)
    ids = wl.moe_ids(f"moe/ids/0/{batch}", batch, T, E)
    x = wl.activations(f"moe/x/gu/0/{batch}", batch, H)
    xd = wl.activations(f"moe/x/dn/0/{batch}", batch * T, F).reshape(batch, T, F)
    gus, dns = 2 * wl.block_bytes("q4_0", F, H), wl.block_bytes("q4_0", H, F)
    secs = _timed(lambda: oracle.moe("q4_0", gu, gus, E, 2 * F, H, ids, x))
    secs += _timed(lambda: oracle.moe("q4_0", dn, dns, E, H, F, ids, None, x_slots=xd))
    nu = len(np.unique(ids))
    return wl.MOE_LAYERS * secs, wl.MOE_LAYERS * nu * (gus + dns)


def oracle_entry(secs, nbytes, tokens, sample):
    return {"kind": "oracle", "cores": 1, "s_per_token": secs / tokens, "gbs": nbytes / secs / 1e9,
            "tok_s": tokens / secs, "sample": sample}


def cpu_baseline(wl):
    """The oracle on one full token of the headline workload (Q8_0, batch
    1), single-threaded, on this host."""
    secs, nbytes = oracle_dense(wl, "q8_0")
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one batch-1 Q8_0 8B token: a layer's 7 matrices timed once x32 + lm_head, "
                      f"{nbytes} B in {secs:.2f} s, 1 thread",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "tok_s_equiv": 1.0 / secs}


# ---------------------------------------------------------------- main
def final_line(head, ceiling, cpu, summary, steps, warmup):
    """The compact last stdout line: the headline step, the dominant
    kernel's roofline, the read ceiling, the oracle baseline and one
    [GB/s, tok/s] pair per extra workload (kept well under 4 KB)."""
    # Roofline of the dominant kernel.  The q||k||v (6144 rows), o (4096
    # rows), gate||up (28672 rows) and lm_head (128256 rows) launches, 97 of
    # the step's 129 and ~70% of its time, run one instantiation: the
    # contiguous-chunk kernel qmv_kernel_c<Q8_0, XU=2, 8 waves, PD=2>; down
    # (K = 14336) runs the 16-wave one.  achieved =
    # that kernel's algorithmic bytes over its summed per-launch event
    # times (each launch of a label back to back on the launch stream).
    dom = [k for k in ("qkv", "o", "gate_up", "lm_head") if k in head["per_matrix"]]
    pm = head["per_matrix"]
    dom_bytes = sum(pm[k]["bytes_per_launch"] * pm[k]["launches"] for k in dom)
    dom_us = sum(pm[k]["us_per_launch"] * pm[k]["launches"] for k in dom)
    dom_n = sum(pm[k]["launches"] for k in dom)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": _r(achieved), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": _r(achieved / PEAK_GBS, 4),
            "traffic": recorded_traffic("qmv_kernel_c<Q8_0, 2, 8, 2, float, 1>", "bytes_per_launch"),
            "kernel": "qmv_kernel_c<Q8_0, 2, 8, 2, float, 1>",
            "basis": "HIP events on the launch stream, each label's cache-cold launches back to back",
            "launches_per_step": dom_n, "us_per_launch": _r(dom_us / dom_n, 3),
            "bytes_per_launch": int(dom_bytes / dom_n), "frac_of_read_ceiling": _r(achieved / ceiling["value"], 4)}
    line = {
        "metric": METRIC,
        "value": _r(head["gbs_wall"]),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": _r(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama8b_q8_0_decode_sweep_b1", "format": "q8_0", "batch": 1,
                   "layers": 32, "matvecs_per_step": 225, "launches_per_step": head["launches_per_step"],
                   "launch": "one per dependency level: qkv, o, gate_up, down; lm_head",
                   "bytes_per_step": head["bytes_per_step"], "hip_graph": head["graph"]},
        "pct_of_peak": _r(head["pct_peak_wall"], 2),
        "tok_s_equiv": _r(head["tok_s_wall"]),
        "gpu_time": {"gbs": _r(head["gbs_gpu"]), "ms_per_step": _r(head["gpu_ms_per_step"], 4)},
        "kernel_time": {"gbs": _r(head["gbs_kernel"]), "ms_per_step": _r(head["kernel_ms_per_step"], 4)},
        "roofline": roof,
        "read_ceiling": {k: (_r(v, 4) if isinstance(v, float) else v) for k, v in ceiling.items()},
        "cpu_baseline": None if cpu is None else {k: (_r(v, 4) if isinstance(v, float) else v) for k, v in cpu.items()},
        "sweeps_gbs_toks": summary,
        # HBM traffic / algorithmic bytes per kernel family (recorded counters;
        # null where the kernel's sources changed since)
        "traffic_ratio": {r["key"]: recorded_traffic(k) for k, r in TRAFFIC_RECORDS.items()},
    }
    return line


def _r(v, nd=1):
    return None if v is None else round(float(v), nd)


def run_headline(torch, qmv, wl, args, detail):
    """The headline step: the 8B Q8_0 batch-1 decode token, one launch per
    dependency level, timed as a replayed HIP graph."""
    sw = build_llama_grouped(torch, qmv, wl, "q8_0")
    log(f"[{sw.name}] {len(sw.launches)} launches, {sw.bytes_per_step} bytes/step")
    head = time_sweep(torch, sw, args.steps, args.warmup, not args.no_graph)
    detail[sw.name] = head
    log(f"[{sw.name}] {head['ms_per_step']:.3f} ms/step wall, {head['gbs_wall']:.0f} GB/s wall, "
        f"{head['gbs_gpu']:.0f} GB/s events, {head['gbs_kernel']:.0f} GB/s per-matrix sum")
    log(f"[{sw.name}] per matrix: " + json.dumps(head["per_matrix"]))
    del sw
    torch.cuda.empty_cache()
    return head


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweeps", default="all",
                    help="extra workloads: all, none, or a comma list of c1,q8_0,q4_0,q4_1,q4_k,q6_k,int8,moe, or of "
                         "FMT@B / FMT@Bf / FMT@1g (one 8B sweep of format FMT at batch B, f: row-fused layout, "
                         "1g: batch 1 with one launch per dependency level), moe@B[:q4_k] / moeblock@B[:q4_k] (one MoE "
                         "sweep at batch B)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip every oracle timing")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline step (profiling runs of single sweeps); no final line is printed")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--detail", default=None, help="write the full per-matrix tables of every workload here (JSON)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (scale for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the path runs on one MI355X's share; --gpus {args.gpus} "
              "is not supported (the path runs on one GPU; sharding across GPUs is a design note, not run).", file=sys.stderr)
        sys.exit(2)

    import torch
    import bandwidth_bound_block_amd as qmv
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return

    detail = {}
    if args.no_headline:
        head = None
    else:
        head = run_headline(torch, qmv, wl, args, detail)


    summary = {}          # sweep name -> [GB/s wall, tok/s wall] (the compact last line)
    oracles = {}          # memoized oracle timings per workload kind

    def oracle_for(key, fn):
        if args.no_cpu_baseline:
            return None
        if key not in oracles:
            t0 = time.time()
            oracles[key] = fn()
            log(f"[oracle] {key}: {oracles[key]['s_per_token']:.3f} s per token ({time.time() - t0:.1f} s)")
        return oracles[key]

    def record(s, r, oracle_info=None, **more):
        detail[s.name] = r
        line = {"sweep": s.name, "batch": s.batch, "gbs": _r(r["gbs_wall"]), "pct_of_peak": _r(r["pct_peak_wall"], 2),
                "tok_s": _r(r["tok_s_wall"]), "ms_per_step": _r(r["ms_per_step"], 4),
                "gbs_kernel_sum": _r(r["gbs_kernel"]), "launches_per_step": r["launches_per_step"],
                "bytes_per_step": r["bytes_per_step"]}
        line.update(more)
        if oracle_info is not None:
            line["oracle"] = {k: (_r(v, 4) if isinstance(v, float) else v) for k, v in oracle_info.items()}
            line["speedup_vs_oracle"] = _r(r["tok_s_wall"] / s.batch / oracle_info["tok_s"], 0)
        print(json.dumps(line), flush=True)
        log(f"[{s.name}] {r['gbs_wall']:.0f} GB/s wall, {r['gbs_kernel']:.0f} GB/s per-matrix sum, "
            f"{r['tok_s_wall']:.0f} tok/s (wall); per matrix: " + json.dumps(r["per_matrix"]))
        summary[s.name] = [int(round(r["gbs_wall"])), int(round(r["tok_s_wall"]))]

    def dense_oracle(fmt):
        secs, nb = oracle_dense(wl, fmt)
        return oracle_entry(secs, nb, 1, f"one batch-1 {fmt} token of the 8B layer set (a layer's 7 matrices "
                                          f"timed once, x32, + lm_head); per column at batch B: B times this")

    names = [] if args.sweeps == "none" else (
        ["c1", "q8_0", "q4_0", "q4_1", "q4_k", "q6_k", "int8", "moe"] if args.sweeps == "all"
        else args.sweeps.split(","))
    ksteps = max(5, min(args.steps, 20))
    for nm in names:
        if nm.startswith(("moe@", "moeblock@")):
            # one MoE sweep: moe@B / moeblock@B (Q4_0 experts, or moe@B:q4_k / moeblock@B:q4_k)
            what, spec = nm.split("@")
            B, _, fmt = spec.partition(":")
            if what == "moe":
                s = build_moe(torch, qmv, wl, int(B), fmt or "q4_0")
            else:
                s = build_moe_block(torch, qmv, wl, int(B), fmt or "q4_0")
            record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph),
                   mean_distinct_experts=_r(s.mean_unique, 2))
            del s
            torch.cuda.empty_cache()
        elif "@" in nm:
            fmt, spec = nm.split("@")
            if spec == "1g":
                s = build_llama_grouped(torch, qmv, wl, fmt)
            else:
                s = build_llama(torch, qmv, wl, fmt, int(spec.rstrip("f")), fused=spec.endswith("f"))
            record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph))
            del s
            torch.cuda.empty_cache()
        elif nm == "c1":
            s = build_c1(torch, qmv, wl)
            r = time_sweep(torch, s, ksteps, args.warmup, not args.no_graph)
            pm = r["per_matrix"]["q8_0_1024"]
            o = oracle_for("c1", lambda: oracle_entry(*oracle_c1(wl), 1, "one 1024x1024 Q8_0 matvec, mean of 20"))
            record(s, r, o, us_per_matvec_wall=_r(r["ms_per_step"] * 1e3 / C1_COPIES, 3),
                   us_per_matvec_events=_r(pm["us_per_launch"], 3), copies=C1_COPIES,
                   matvecs_per_s=_r(C1_COPIES / (r["ms_per_step"] * 1e-3), 0),
                   note="a step is one call on each of the 480 copies; tok_s counts steps")
            del s
            torch.cuda.empty_cache()
        elif nm == "q8_0":
            for fused in (False, True):
                s = build_llama(torch, qmv, wl, "q8_0", 1, fused=fused)
                record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph))
                del s
                torch.cuda.empty_cache()
            for fused in (False, True):
                s = build_llama_chain(torch, qmv, wl, "q8_0", fused=fused)
                r = time_sweep(torch, s, ksteps, args.warmup, not args.no_graph)
                record(s, r, barrier_error_flag=int(s.workspace.view(torch.int32)[2].item()))
                del s
                torch.cuda.empty_cache()
        elif nm in ("q4_0", "q4_1"):
            s = build_llama_grouped(torch, qmv, wl, nm)
            o = oracle_for(nm, lambda: dense_oracle(nm))
            record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph), o)
            del s
            torch.cuda.empty_cache()
            for B, fused in ((1, False), (1, True), (2, False), (4, False), (8, False), (2, True), (4, True),
                             (8, True)):
                s = build_llama(torch, qmv, wl, nm, B, fused=fused)
                record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph))
                del s
                torch.cuda.empty_cache()
        elif nm in ("q4_k", "q6_k"):
            o = oracle_for(nm, lambda: dense_oracle(nm))
            # one launch per dependency level (qmv_chain groups q, k, v and gate, up)
            s = build_llama_grouped(torch, qmv, wl, nm)
            record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph))
            del s
            torch.cuda.empty_cache()
            for B, fused in ((1, False), (1, True), (2, False), (4, False), (8, False)):
                s = build_llama(torch, qmv, wl, nm, B, fused=fused)
                record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph), o if B == 1 else None)
                del s
                torch.cuda.empty_cache()
        elif nm == "int8":
            o = oracle_for("int8", lambda: oracle_entry(*oracle_int8(wl), 1, "one int8 token: a layer's 7 matrices "
                                                                           "timed once, x28, + lm_head"))
            for fused in (False, True):
                s = build_int8(torch, qmv, wl, fused=fused)
                record(s, time_sweep(torch, s, ksteps, args.warmup, not args.no_graph), o)
                del s
                torch.cuda.empty_cache()
        elif nm == "moe":
            for B in (1, 2, 4, 8):
                o = oracle_for(f"moe{B}", lambda: oracle_entry(*oracle_moe(wl, B), B,
                                                               f"one MoE layer at batch {B} timed once, x48"))
                for build in (build_moe, build_moe_block):
                    s = build(torch, qmv, wl, B)
                    r = time_sweep(torch, s, ksteps, args.warmup, not args.no_graph)
                    record(s, r, o, mean_distinct_experts=_r(s.mean_unique, 2))
                    del s
                    torch.cuda.empty_cache()
            # Q4_K experts (one grid row per token and slot), plain and the
            # fused block, batch 1 and 8
            for B in (1, 8):
                for build in (build_moe, build_moe_block):
                    s = build(torch, qmv, wl, B, "q4_k")
                    r = time_sweep(torch, s, ksteps, args.warmup, not args.no_graph)
                    record(s, r, mean_distinct_experts=_r(s.mean_unique, 2))
                    del s
                    torch.cuda.empty_cache()

    if head is None:
        return
    ceiling = read_ceiling(torch, qmv)
    log(f"[read_ceiling] {ceiling['value']:.0f} GB/s median, {ceiling['best']:.0f} best "
        f"({100 * ceiling['frac_of_peak']:.1f}% of {PEAK_GBS:.0f})")

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(wl)
        log(f"[cpu_baseline] {cpu['value']:.3f} GB/s in {time.time() - t0:.1f}s")

    line = final_line(head, ceiling, cpu, summary, args.steps, args.warmup)
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"headline": line, "detail": detail}, f)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
