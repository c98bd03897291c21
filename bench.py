"""Benchmark of one MoE layer's hot path on one MI355X.

One step = route -> permute (+ load statistics) -> grouped SwiGLU GEMMs -> combine for one
batch of synthetic tokens (moe_forward), with inputs already resident in HBM. Default
workload: the packed RL microbatch (T=16384 tokens in variable-length sequences, d=4096,
E=128, top-8, I=1536, bf16, routing replay), the largest single-GPU layer; the
training-shaped layer (T=4096, d=2048, E=64, I=1408, router with a Zipf(1.1) log bias,
with its backward and router-variant reports) and the heavily imbalanced replay layer
(T=32768, d=2048, E=256, I=768) are timed in the same run under "other_configs".

Prints ONE JSON line with the throughput (tokens/s from the median step), a roofline entry
for the dominant kernel (the fused gate/up + SwiGLU grouped GEMM, timed live with HIP events
recorded by the library around it on the launch stream), the bf16 peak derived from the
device's CU count and clock next to the published one, and the CPU oracle timed on a
bounded sample of the same workload. Progress lines go to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 MI355X; grouped-GEMM TFLOP/s as % bf16 MFMA peak"
PEAK_FP32_TFLOPS = 157.3
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published figure
PEAK_HBM_GBS = 8000.0
# dense bf16 MFMA work per compute unit per clock on gfx950: four SIMDs, each retiring one
# v_mfma_f32_16x16x32_bf16 (16*16*32*2 = 16384 FLOP) every 16 cycles = 1024 FLOP/clk
BF16_FLOP_PER_CLK_CU = 4096
# hipDeviceAttribute_t values (hip_runtime_api.h, ROCm 7)
_HIP_ATTR_CLOCK_KHZ, _HIP_ATTR_CU_COUNT = 5, 63


def log(msg: str):
    """Progress of the run itself, on stderr (stdout carries the one JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)

WORKLOADS = {
    "c2": "training-shaped bf16 MoE layer: T=4096 tokens, d=2048, E=64 experts, top-8, SwiGLU "
          "inter=1408, router logits + per-expert Zipf(1.1) log bias",
    "c3": "packed RL microbatch: T=16384 tokens in lognormal-length sequences, d=4096, E=128, "
          "top-8, inter=1536, bf16, routing replay with per-sequence Dirichlet demand",
    "c4": "heavily imbalanced replay: T=32768, d=2048, E=256, top-8, inter=768, bf16",
    "c5": "decode-shaped bf16 MoE layer: T = 1..64 tokens, d=4096, E=128, top-8, SwiGLU "
          "inter=1536, router logits (memory-bound)",
}


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the launch stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.rt.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a),
                                           ctypes.c_void_p(b)) == 0
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))

    def attribute(self, attr: int, dev: int = 0) -> int:
        v = ctypes.c_int()
        assert self.rt.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr),
                                             ctypes.c_int(dev)) == 0
        return v.value


def derived_peak(hip) -> dict:
    """The bf16 dense MFMA peak from this device's own figures: compute units x peak clock
    x bf16 FLOP per clock per CU, next to the published 2.5 PFLOP/s."""
    cus = hip.attribute(_HIP_ATTR_CU_COUNT)
    mhz = hip.attribute(_HIP_ATTR_CLOCK_KHZ) / 1000.0
    tf = cus * mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12
    return {"compute_units": cus, "peak_clock_mhz": mhz,
            "bf16_flop_per_clk_per_cu": BF16_FLOP_PER_CLK_CU,
            "derived_bf16_tflops": round(tf, 1), "published_bf16_tflops": PEAK_BF16_TFLOPS}


def cpu_baseline(L, sample_tokens: int):
    """The oracle, untuned, on the first ``sample_tokens`` tokens of the workload: every
    stage (router or replay check, permutation + statistics, gather, expert FFN,
    combine). Returns (tokens/s, seconds, threads)."""
    import oracle
    oracle.lib()
    toks = np.arange(min(sample_tokens, L.T))
    t0 = time.perf_counter()
    x = np.ascontiguousarray(L.x[toks])
    if L.mode == "router":
        lg = oracle.router_logits(x, L.w_router, L.logit_bias, L.dtype)
        idx, w, _, _ = oracle.route_from_logits(lg, L.k)
    else:
        idx, w = L.idx_in[toks], L.w_in[toks]
        oracle.replay_check(idx, w, L.E)
    counts, offsets, perm, inv, _ = oracle.permute(idx, L.E)
    oracle.weighted_counts(idx, L.E, None)
    xp = oracle.gather(x, perm, L.k)
    rowexp = np.repeat(np.arange(L.E, dtype=np.int32), counts)
    h, y = oracle.expert_ffn(xp, rowexp, L.w13, L.w2, L.dtype)
    oracle.combine(y, inv, w, L.dtype)
    dt = time.perf_counter() - t0
    return len(toks) / dt, dt, oracle.num_threads()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stage_rates(L, dims, inp, K, hip, stream):
    """The memory-bound stages through their own entry points (router or replay check,
    permutation with the materialised gather, combine), each timed over K calls with HIP
    events, as effective HBM GB/s = algorithmic bytes / median time. Algorithmic bytes:
    route = x + w_router + logits + top-k ids/weights; replay = ids/weights in and out;
    permute = ids + x + x_perm + perm/inv + counts; combine = Y + inv/weights + out."""
    import torch

    import moe_layer_routing_amd as M
    dev = inp["x"].device
    eb = 2 if L.dtype == "bf16" else 4
    T, d, E, k, A = L.T, L.d, L.E, L.k, L.T * L.k
    b = M.alloc_forward_buffers(dims, dev, router=(L.mode == "router"), weighted=False)
    ws = M.alloc_workspace(dims, dev)
    b["y"].normal_()

    def timed(fn):
        fn()
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            fn()
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        ms = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
        hip.destroy(ev)
        return ms

    out = {}
    if L.mode == "router":
        nb = T * d * eb + E * d * eb + T * E * 4 + T * k * 8
        ms = timed(lambda: M.route(dims, inp["x"], inp["w_router"], inp["logit_bias"],
                                   b["topk_idx"], b["topk_w"], logits=b["logits"],
                                   d_err=b["d_err"], workspace=ws))
        out["route"] = {"ms": round(ms, 5), "bytes": nb, "gbs": round(nb / ms / 1e6, 1)}
    else:
        nb = 2 * T * k * 8
        ms = timed(lambda: M.route_replay(dims, inp["idx_in"], inp["w_in"], b["topk_idx"],
                                          b["topk_w"], d_err=b["d_err"]))
        out["replay"] = {"ms": round(ms, 5), "bytes": nb, "gbs": round(nb / ms / 1e6, 1)}
    nb = T * k * 4 + T * d * eb + A * d * eb + A * 8 + (2 * E + 1) * 4
    ms = timed(lambda: M.permute(dims, b["topk_idx"], inp["x"], b["x_perm"], b["perm"],
                                 b["inv"], b["counts"], b["offsets"], d_err=b["d_err"],
                                 workspace=ws))
    out["permute"] = {"ms": round(ms, 5), "bytes": nb, "gbs": round(nb / ms / 1e6, 1)}
    nb = A * d * 4 + A * 4 + T * k * 4 + T * d * eb
    ms = timed(lambda: M.combine(dims, b["y"], b["inv"], b["topk_w"], b["out"]))
    out["combine"] = {"ms": round(ms, 5), "bytes": nb, "gbs": round(nb / ms / 1e6, 1)}
    out["peak_gbs"] = PEAK_HBM_GBS
    return out


def variant_report(L, dims, inp, K, hip, stream, vocab=131072):
    """Router variants on the same layer ("0 train-infer mismatch ...", "Choosing GLM's
    eight experts" and "Hash and learned expert routing"): the router alone (logits, choice,
    weights, lse) for the softmax router, sigmoid and sqrt-softplus scores with a correction
    bias, and hash routing over a vocabulary of ``vocab`` ids (a 128K-entry vocabulary is
    assumed; the pages give none), as median ms and effective GB/s; the whole step with the
    GLM-style router (sigmoid + bias, routed scaling factor 2.5) and the hash router next
    to the softmax step; and the objective statistics (z-loss, load-balancing loss,
    expert-bias update; HARTS eq. (20)). Algorithmic bytes: x + w_router + logits + ids and
    weights (+ bias + lse, + token ids and table rows for hash)."""
    import torch

    import moe_layer_routing_amd as M
    import workloads as W
    dev = inp["x"].device
    eb = 2 if L.dtype == "bf16" else 4
    T, d, E, k = L.T, L.d, L.E, L.k
    bias = torch.from_numpy(W.correction_bias(E, L.seed)).to(dev)
    table = torch.from_numpy(W.hash_table(vocab, E, k, L.seed)).to(dev)
    tok = torch.from_numpy(W.token_ids(T, vocab, L.seed)).to(dev)
    q = torch.from_numpy(W.token_multiplicities(T, L.seed)).to(dev)
    ws = M.alloc_workspace(dims, dev)
    b = M.alloc_forward_buffers(dims, dev, router=True, weighted=True)
    lse = torch.empty(T, dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            fn()
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        ms = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
        hip.destroy(ev)
        return ms

    base = T * d * eb + E * d * eb + T * E * 4 + T * k * 8
    routers = {
        "softmax": (dict(score="softmax"), base),
        "sigmoid_bias": (dict(score="sigmoid", corr_bias=bias), base + E * 4),
        "sqrt_softplus_bias": (dict(score="sqrt_softplus", corr_bias=bias), base + E * 4),
        "hash_sqrt_softplus": (dict(score="sqrt_softplus", hash_table=table, token_ids=tok),
                               base + T * 4 + T * k * 4),
    }
    out = {"vocab": vocab}
    for name, (kw, nb) in routers.items():
        nb += T * 4                                     # lse
        ms = timed(lambda: M.route_scored(dims, inp["x"], inp["w_router"], inp["logit_bias"],
                                          b["topk_idx"], b["topk_w"], logits=b["logits"],
                                          d_err=b["d_err"], workspace=ws, lse=lse, **kw))
        out["route_" + name] = {"ms": round(ms, 5), "bytes": nb, "gbs": round(nb / ms / 1e6, 1)}

    fb = M.alloc_forward_buffers(dims, dev, router=True, weighted=True)
    del fb["x_perm"]
    fb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
              logit_bias=inp["logit_bias"], token_mult=q)
    steps = {"softmax": (None, 0.0),
             "glm_sigmoid_bias_scale2.5": (dict(score="sigmoid", corr_bias=bias, lse=lse), 2.5),
             "hash_sqrt_softplus": (dict(score="sqrt_softplus", hash_table=table, token_ids=tok,
                                         lse=lse), 0.0)}
    for name, (rkw, scale) in steps.items():
        ms = timed(lambda: M.forward(dims, fb, ws, router=rkw, routed_scale=scale))
        out["step_ms_" + name] = round(ms, 5)
    assert int(fb["d_err"].item()) == 0
    ob = torch.zeros(3, dtype=torch.float64, device=dev)
    bias_w = bias.clone()
    nb = T * 8 + E * (8 + 4 + 8) + 24
    ms = timed(lambda: M.objectives(dims, ob, lse=lse, token_mult=q,
                                    weighted_counts=fb["weighted_counts"],
                                    prob_mass=fb["prob_mass"], bias_rate=1e-3,
                                    corr_bias=bias_w))
    z, aux, S = host_list(ob)
    out["objectives"] = {"ms": round(ms, 5), "bytes": nb, "z_loss": round(z, 6),
                         "aux_loss": round(aux, 6), "S": int(S)}
    return out


def ranks_report(L, dims, inp, K, hip, stream, inter_shared=2048):
    """Expert-parallel output emulated on one GPU ("0 train-infer mismatch ...", "Sharding the
    experts"): for R = 8 and 16 ranks, the shared expert sharded over the ranks
    (inter_shared features in all; the pages give no size, 2048 is assumed) as TFLOP/s of
    6*T*d*inter_shared, the rank combine (R partials + FP64 pairwise tree) as GB/s of its
    algorithmic bytes (Y + inv + weights + ids + shared shards + out), and the whole step
    with both, next to the plain step."""
    import torch

    import moe_layer_routing_amd as M
    dev = inp["x"].device
    eb = 2 if L.dtype == "bf16" else 4
    T, d, E, k = L.T, L.d, L.E, L.k
    A = T * k
    rng = np.random.default_rng(L.seed)

    def timed(fn):
        fn()
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            fn()
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        ms = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
        hip.destroy(ev)
        return ms

    ws = M.alloc_workspace(dims, dev)
    fb = M.alloc_forward_buffers(dims, dev, router=(L.mode == "router"))
    del fb["x_perm"]
    fb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"])
    if L.mode == "router":
        fb["w_router"], fb["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        fb["idx_in"], fb["w_in"] = inp["idx_in"], inp["w_in"]
    out = {"inter_shared": inter_shared,
           "step_ms_plain": round(timed(lambda: M.forward(dims, fb, ws)), 5)}
    sd = fb["out"].dtype
    for R in (8, 16):
        if E % R:
            continue
        S = inter_shared // R
        std = 1.0 / np.sqrt(d)
        w13s = torch.from_numpy((rng.standard_normal((R, 2 * S, d)) * std).astype(np.float32))
        w2s = torch.from_numpy((rng.standard_normal((R, d, S)) * std).astype(np.float32))
        w13s, w2s = w13s.to(dev).to(sd), w2s.to(dev).to(sd)
        hs = torch.empty((R, T, S), dtype=sd, device=dev)
        ys = torch.empty((R, T, d), dtype=torch.float32, device=dev)
        sws = M.alloc_shared_workspace(dims, R, inter_shared, dev)
        ms_sh = timed(lambda: M.shared_ffn(dims, R, inter_shared, inp["x"], w13s, w2s, hs, ys,
                                           workspace=sws))
        flops = 6.0 * T * d * inter_shared
        nb = A * d * 4 + A * 4 + T * k * 8 + R * T * d * 4 + T * d * eb
        ms_c = timed(lambda: M.combine_ranks(dims, R, fb["y"], fb["inv"], fb["topk_w"],
                                             fb["topk_idx"], fb["out"], y_shared=ys,
                                             routed_scale=2.5))
        fb.update(w13_shared=w13s, w2_shared=w2s, h_shared=hs, y_shared=ys)
        ms_step = timed(lambda: M.forward(dims, fb, ws, routed_scale=2.5, ranks=R,
                                          inter_shared=inter_shared, shared_workspace=sws))
        for n in ("w13_shared", "w2_shared", "h_shared", "y_shared"):
            del fb[n]
        out[f"R{R}"] = {"shared_ffn_ms": round(ms_sh, 5),
                        "shared_ffn_tflops": round(flops / (ms_sh * 1e-3) / 1e12, 1),
                        "combine_ranks_ms": round(ms_c, 5), "combine_ranks_bytes": nb,
                        "combine_ranks_gbs": round(nb / ms_c / 1e6, 1),
                        "step_ms": round(ms_step, 5)}
    assert int(fb["d_err"].item()) == 0
    return out


def backward_report(L, dims, inp, K, hip, stream):
    """Backward of the layer (moe_backward) after one forward, with the router's gradients:
    the median time of K calls, and the gradient GEMMs' rate against the FP32 MFMA peak
    (their operands are FP32): 16*T*k*d*I FLOP per call = the recomputed gate/up
    pre-activations (4), the data gradients dh (2) and dx (4), the weight gradients dw2 (2)
    and dw13 (4)."""
    import torch

    import moe_layer_routing_amd as M
    dev = inp["x"].device
    ws = M.alloc_workspace(dims, dev)
    fb = M.alloc_forward_buffers(dims, dev, router=True)
    del fb["x_perm"]
    fb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
              logit_bias=inp["logit_bias"])
    M.forward(dims, fb, ws)
    # bf16 layers: no gu buffer, the gate/up recomputation forms d_gu in its epilogue
    bb = M.alloc_backward_buffers(dims, dev, router=True, keep_gu=(L.dtype != "bf16"))
    g = torch.Generator(device=dev).manual_seed(L.seed)
    dout = torch.randn((L.T, L.d), generator=g, device=dev).to(fb["out"].dtype)
    bb.update(x=inp["x"], w13=inp["w13"], w2=inp["w2"], w_router=inp["w_router"],
              logit_bias=inp["logit_bias"], logits=fb["logits"], offsets=fb["offsets"],
              perm=fb["perm"], inv=fb["inv"], topk_w=fb["topk_w"], h=fb["h"], y=fb["y"],
              d_out=dout)
    def run(bufs, gd):
        M.backward(dims, bufs, ws, grad_dtype=gd)
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            M.backward(dims, bufs, ws, grad_dtype=gd)
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        ts = [hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]
        hip.destroy(ev)
        return float(np.median(ts)), ts

    ms, ts = run(bb, M.MOE_F32)
    flops = 16.0 * L.T * L.k * L.d * L.I
    out = {"ms": round(ms, 5), "p10": round(float(np.percentile(ts, 10)), 5),
           "p90": round(float(np.percentile(ts, 90)), 5), "gemm_flop": flops,
           "tflops_overall": round(flops / (ms * 1e-3) / 1e12, 2),
           "peak_fp32_mfma_tflops": PEAK_FP32_TFLOPS,
           "frac_overall": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
           "forward_ms_for_reference": None}
    if L.dtype == "bf16":
        b16 = M.alloc_backward_buffers(dims, dev, router=True, grad_dtype=M.MOE_BF16,
                                       keep_gu=False)
        b16.update({n: bb[n] for n in ("x", "w13", "w2", "w_router", "logit_bias", "logits",
                                       "offsets", "perm", "inv", "topk_w", "h", "y", "d_out")})
        del bb
        ms16, ts16 = run(b16, M.MOE_BF16)
        out["bf16_operands"] = {
            "ms": round(ms16, 5), "p10": round(float(np.percentile(ts16, 10)), 5),
            "p90": round(float(np.percentile(ts16, 90)), 5),
            "tflops_overall": round(flops / (ms16 * 1e-3) / 1e12, 2),
            "frac_bf16_peak_overall": round(flops / (ms16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "dy and d_gu rounded once to bf16; bf16 MFMA for every gradient GEMM; "
                    "the data gradients read w2 and w13 K-major as stored; the gate/up recomputation forms d_gu in its epilogue (no gu buffer)"}
        # the forward keeps g and u (FP32) and the backward reads them instead of
        # recomputing: forward and backward timed over K calls each
        gu = torch.empty((L.T * L.k, 2 * L.I), dtype=torch.float32, device=dev)
        fb["gu"] = gu
        M.forward(dims, fb, ws)
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            M.forward(dims, fb, ws)
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        fwd_gu = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
        hip.destroy(ev)
        b16["gu"] = gu
        M.backward(dims, b16, ws, grad_dtype=M.MOE_BF16, gu_saved=True)
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream.cuda_stream)
            M.backward(dims, b16, ws, grad_dtype=M.MOE_BF16, gu_saved=True)
            hip.record(ev[2 * i + 1], stream.cuda_stream)
        torch.cuda.synchronize()
        bwd_gu = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
        hip.destroy(ev)
        del fb["gu"], b16["gu"], gu
        flops_saved = 12.0 * L.T * L.k * L.d * L.I      # no recomputation
        out["bf16_operands_saved_gu"] = {
            "forward_ms": round(fwd_gu, 5), "backward_ms": round(bwd_gu, 5),
            "tflops_backward": round(flops_saved / (bwd_gu * 1e-3) / 1e12, 2),
            "note": "the forward also stores g and u (FP32, 8*T*k*inter bytes); the backward "
                    "reads them instead of recomputing the gate/up GEMM (12*T*k*d*I FLOP "
                    "left); the same gradients bit for bit"}
    assert int(fb["d_err"].item()) == 0
    return out


def ep_share_report(K, hip, stream, cfg="c3", ranks=8):
    """One GPU's share of the packed-microbatch layer under expert parallelism (8 data-
    parallel ranks x 8 expert-parallel ranks): the grouped FFN of the 16 experts rank 0
    owns, over the rows the 8 ranks' batches route to them (each batch shaped like the
    packed-microbatch layer, with its own seed). Synthetic bf16 rows and weights on the
    device; TFLOP/s of 6*A*d*I against the bf16 peak."""
    import torch

    import moe_layer_routing_amd as M
    import workloads as W
    c = W.CONFIGS[cfg]
    d, I, H = c["d"], c["inter"] if "inter" in c else c["I"], c["E"] // ranks
    counts = W.ep_share_counts(cfg, ranks)
    A = int(counts.sum())
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    std = 1.0 / np.sqrt(d)
    x_perm = torch.randn((A, d), generator=g, device=dev).to(torch.bfloat16)
    w13 = (torch.randn((H, 2 * I, d), generator=g, device=dev) * std).to(torch.bfloat16)
    w2 = (torch.randn((H, d, I), generator=g, device=dev) * std).to(torch.bfloat16)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
    h = torch.empty((A, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((A, d), dtype=torch.float32, device=dev)
    dims = M.make_dims(A, d, H, 1, I, M.MOE_BF16)
    ws = M.alloc_workspace(dims, dev)
    M.grouped_ffn(dims, x_perm, offsets, w13, w2, h, y, workspace=ws)
    ev = hip.create(2 * K)
    for i in range(K):
        hip.record(ev[2 * i], stream.cuda_stream)
        M.grouped_ffn(dims, x_perm, offsets, w13, w2, h, y, workspace=ws)
        hip.record(ev[2 * i + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = float(np.median([hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(K)]))
    hip.destroy(ev)
    flops = 6.0 * A * d * I
    return {"workload": f"{cfg} under DP{ranks} x EP{ranks}: rank 0's {H} experts",
            "rows": A, "rows_per_expert": counts.tolist(), "d": d, "inter": I,
            "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def host_list(t):
    return [float(v) for v in t.cpu().tolist()]


def placement_report(L, dims, inp, counts, K, hip, stream, P=8):
    """Logical -> physical expert placement over P expert-parallel ranks (layer-local LPT of
    "RoutePack ...", Sec. 3) from this step's expert counts: rank-load coefficient of
    variation for the identity and the LPT placement, the host planner's time, and the
    step time with the LPT placement (weights stored in slot order) next to the identity
    one, plus the placed and plain permutation alone."""
    import torch

    import moe_layer_routing_amd as M
    E, H = L.E, L.E // P
    loads = counts.astype(np.int64)
    ident = np.array([loads[p * H:(p + 1) * H].sum() for p in range(P)], dtype=np.float64)
    cv_id = float(np.sqrt(((ident - ident.mean()) ** 2).mean()) / ident.mean())
    t0 = time.perf_counter()
    for _ in range(100):
        slots, rank_load, cv = M.place_lpt(loads, P)
    plan_us = (time.perf_counter() - t0) / 100 * 1e6
    dev = inp["x"].device
    slot_t = torch.from_numpy(slots).to(dev)
    expert_of_slot = torch.empty_like(slot_t)
    expert_of_slot[slot_t.long()] = torch.arange(E, dtype=slot_t.dtype, device=dev)
    w13p = inp["w13"][expert_of_slot.long()].contiguous()
    w2p = inp["w2"][expert_of_slot.long()].contiguous()

    def step_ms(slot, w13, w2):
        b = M.alloc_forward_buffers(dims, dev, router=(L.mode == "router"))
        del b["x_perm"]
        b.update(x=inp["x"], w13=w13, w2=w2, slot_of_expert=slot)
        if L.mode == "router":
            b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
        else:
            b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
        ws = M.alloc_workspace(dims, dev)
        M.forward(dims, b, ws)
        ev = hip.create(2)
        hip.record(ev[0], stream.cuda_stream)
        for _ in range(K):
            M.forward(dims, b, ws)
        hip.record(ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        ms = hip.ms(ev[0], ev[1]) / K
        hip.destroy(ev)
        assert int(b["d_err"].item()) == 0
        return ms, b

    ms_id, b_id = step_ms(None, inp["w13"], inp["w2"])
    ms_lpt, b_lpt = step_ms(slot_t, w13p, w2p)
    same = bool(torch.equal(b_id["out"].view(torch.int16), b_lpt["out"].view(torch.int16)))

    def perm_ms(slot):
        b = M.alloc_forward_buffers(dims, dev)
        ws = M.alloc_workspace(dims, dev)
        args = (dims, b_id["topk_idx"], inp["x"], None, b["perm"], b["inv"], b["counts"],
                b["offsets"])
        M.permute(*args, workspace=ws, slot_of_expert=slot)
        ev = hip.create(2)
        hip.record(ev[0], stream.cuda_stream)
        for _ in range(K):
            M.permute(*args, workspace=ws, slot_of_expert=slot)
        hip.record(ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        ms = hip.ms(ev[0], ev[1]) / K
        hip.destroy(ev)
        return ms

    return {"ranks": P, "cv_identity": round(cv_id, 5), "cv_lpt": round(cv, 6),
            "rank_load_lpt": rank_load.tolist(), "plan_us_host": round(plan_us, 2),
            "step_ms_identity": round(ms_id, 5), "step_ms_lpt": round(ms_lpt, 5),
            "out_bitwise_equal": same, "permute_ms": round(perm_ms(None), 5),
            "permute_placed_ms": round(perm_ms(slot_t), 5)}


def copy_gbs(dev, mib=512, reps=10):
    """Measured device-to-device copy rate, (read + write bytes) / median time."""
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        c.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(c))
    return round(2 * (mib << 20) / (float(np.median(ts)) * 1e-3) / 1e9, 1)


def upload(L, dev):
    """Host (numpy) inputs of layer L -> device tensors (bf16 bit patterns as bfloat16)."""
    import torch

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    return {n: up(getattr(L, n)) for n in ("x", "w_router", "logit_bias", "idx_in", "w_in",
                                           "w13", "w2", "token_mult", "cu_seqlens")}


def decode_rows(Ts, steps, warmup, tile_m=0):
    """Decode-shaped layer: one timed moe_forward per batch size T, each after a read of
    another 512 MB buffer so that the expert weights come from HBM (a read evicts
    them from L2 and the 256 MB memory-attached cache without leaving dirty lines whose
    write-back would be charged to the timed step), reported in tokens/s and in
    effective HBM GB/s = algorithmic bytes / time, where the algorithmic bytes are the
    active experts' w13 and w2 (read once), the router weights, x and out, and the
    routing outputs. Returns (rows, layer)."""
    import torch

    import moe_layer_routing_amd as M
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = W.make_config("c5")
    inp = upload(L, dev)
    scrub = torch.ones(128 << 20, dtype=torch.int32, device=dev)      # 512 MB
    hip = HipEvents()
    stream = torch.cuda.current_stream()
    rows = []
    for T in Ts:
        dims = M.make_dims(T, L.d, L.E, L.k, L.I, M.MOE_BF16, tile_m)
        b = M.alloc_forward_buffers(dims, dev, router=True)
        del b["x_perm"]
        b.update(x=inp["x"][:T].contiguous(), w_router=inp["w_router"], w13=inp["w13"],
                 w2=inp["w2"])
        ws = M.alloc_workspace(dims, dev)
        for _ in range(warmup):
            M.forward(dims, b, ws)
        # the step as a caller runs it (events only around it), then the same step with the
        # library's profiling events between its launches, for the gate/up launch's duration
        # (each event recorded inside the step delays the launch after it by a few us)
        times, itimes, t13 = [], [], []
        for _ in range(steps):
            scrub.sum()
            ev = hip.create(2)
            hip.record(ev[0], stream.cuda_stream)
            M.forward(dims, b, ws)
            hip.record(ev[1], stream.cuda_stream)
            torch.cuda.synchronize()
            times.append(hip.ms(ev[0], ev[1]))
            hip.destroy(ev)
        for _ in range(steps):
            scrub.sum()
            ev = hip.create(5)
            hip.record(ev[0], stream.cuda_stream)
            M.forward(dims, b, ws, prof_events=ev[1:4])
            hip.record(ev[4], stream.cuda_stream)
            torch.cuda.synchronize()
            itimes.append(hip.ms(ev[0], ev[4]))
            t13.append(hip.ms(ev[1], ev[2]))
            hip.destroy(ev)
        # the same step captured once into a HIP graph and replayed (no launch overhead)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            M.forward(dims, b, ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            M.forward(dims, b, ws)
        gtimes = []
        for _ in range(steps):
            scrub.sum()
            ev = hip.create(2)
            hip.record(ev[0], stream.cuda_stream)
            graph.replay()
            hip.record(ev[1], stream.cuda_stream)
            torch.cuda.synchronize()
            gtimes.append(hip.ms(ev[0], ev[1]))
            hip.destroy(ev)
        del graph
        assert int(b["d_err"].item()) == 0
        t_ms = float(np.median(times))
        gr_ms = float(np.median(gtimes))
        g_ms = float(np.median(t13))
        active = int((b["counts"] > 0).sum().item())
        A = T * L.k
        nbytes = (active * 3 * L.d * L.I * 2 + L.E * L.d * 2 + 2 * T * L.d * 2 + 8 * T * L.k)
        g_bytes = active * 2 * L.I * L.d * 2 + A * L.d * 2 + A * L.I * 2
        rows.append({"T": T, "ms": round(t_ms, 4), "p10_ms": round(float(np.percentile(times, 10)), 4),
                     "p90_ms": round(float(np.percentile(times, 90)), 4),
                     "tokens_per_s": round(T / (t_ms * 1e-3), 1),
                     "graph_ms": round(gr_ms, 4),
                     "instrumented_ms": round(float(np.median(itimes)), 4),
                     "graph_hbm_gbs": None,
                     "active_experts": active, "hbm_gbs": round(nbytes / (t_ms * 1e-3) / 1e9, 1),
                     "gate_up_ms": round(g_ms, 4), "gate_up_bytes": g_bytes,
                     "gate_up_gbs": round(g_bytes / (g_ms * 1e-3) / 1e9, 1)})
        rows[-1]["graph_hbm_gbs"] = round(nbytes / (gr_ms * 1e-3) / 1e9, 1)
    del scrub
    return rows, L


def decode_sweep(args):
    """The decode-shaped sweep as its own JSON line (bench.py --config c5)."""
    rows, L = decode_rows([int(t) for t in args.decode_t.split(",")], args.steps, args.warmup,
                          args.tile_m)
    dev = "cuda:0"
    top = rows[-1]
    rec = {
        "metric": METRIC + " (decode-shaped layer, HBM GB/s)",
        "value": top["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": top["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS["c5"], "name": "c5", "T": top["T"], "d": L.d,
                   "E": L.E, "k": L.k, "inter": L.I, "mode": "router", "evict_read_mb": 512},
        "roofline": {"kernel": f"grouped gate/up GEMM + SwiGLU (decode tiles), T={top['T']}",
                     "bound": "hbm", "achieved": top["gate_up_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(top["gate_up_gbs"] / PEAK_HBM_GBS, 4),
                     "traffic": None,
                     "algorithmic": "active experts' w13 + gathered x rows + h, per launch",
                     "avg_launch_ms": top["gate_up_ms"]},
        "copy_gbs_read_plus_write": copy_gbs(dev),
        "sweep": rows,
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def copy_calibration(mib: int):
    """A plain copy of known size (read mib MiB, write mib MiB), five times: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch give the counters' scale."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_calibration_bytes": n, "read_kib": n // 1024, "write_kib": n // 1024,
                      "approx_ms": round(dt * 1e3, 4)}), flush=True)


def gemm_traffic(config: str):
    """HBM bytes per launch of the gate/up grouped GEMM as measured by the rocprofv3
    FETCH_SIZE + WRITE_SIZE passes recorded in profiles/, or None when that record is
    missing or was taken on a different grouped-GEMM source (its sha1 is stored with it)."""
    import hashlib
    rec = os.path.join(ROOT, "profiles", f"gemm_traffic_{config}.md")
    src = os.path.join(ROOT, "moe_layer_routing_amd", "csrc", "grouped_ffn.hip")
    if not os.path.exists(rec):
        return None
    fields = {}
    for line in open(rec):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    sha = hashlib.sha1(open(src, "rb").read()).hexdigest()
    if fields.get("grouped_ffn.hip sha1") != sha or "gate/up bytes per launch" not in fields:
        return None
    return int(fields["gate/up bytes per launch"])


def run_layer(cfg: str, args, hip, reports: bool, cpu_sample: int):
    """Times K whole moe_forward steps of workload ``cfg`` (inputs resident in HBM, the
    library's HIP events around both grouped GEMMs of every step) and, with ``reports``,
    the per-stage and NEXT-row reports. Returns the record fields of that workload."""
    import torch

    import moe_layer_routing_amd as M
    import workloads as W
    t0 = time.perf_counter()
    L = W.make_config(cfg)
    log(f"{cfg}: inputs generated ({time.perf_counter() - t0:.1f} s)")
    dev = torch.device("cuda:0")
    dims = M.make_dims(L.T, L.d, L.E, L.k, L.I, M.MOE_BF16 if L.dtype == "bf16" else M.MOE_F32,
                       args.tile_m)
    inp = upload(L, dev)
    S = 0 if L.cu_seqlens is None else len(L.cu_seqlens) - 1
    b = M.alloc_forward_buffers(dims, dev, router=(L.mode == "router"), num_seqs=S,
                                weighted=True)
    del b["x_perm"]          # the dispatch gather runs inside the gate/up GEMM
    for n in ("x", "w13", "w2"):
        b[n] = inp[n]
    if L.mode == "router":
        b["w_router"], b["logit_bias"] = inp["w_router"], inp["logit_bias"]
    else:
        b["idx_in"], b["w_in"] = inp["idx_in"], inp["w_in"]
    if S:
        b["cu_seqlens"] = inp["cu_seqlens"]
    ws = M.alloc_workspace(dims, dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        M.forward(dims, b, ws)
    torch.cuda.synchronize()
    assert int(b["d_err"].item()) == 0, "device error word set"
    host_counts = b["counts"].cpu().numpy()

    K = args.steps
    evs = hip.create(3 * K)
    bnd = hip.create(K + 1)                 # step boundaries
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        hip.record(bnd[i], stream.cuda_stream)
        M.forward(dims, b, ws, prof_events=evs[3 * i:3 * i + 3])
    hip.record(bnd[K], stream.cuda_stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = hip.ms(bnd[0], bnd[K])
    step_ms = np.array([hip.ms(bnd[i], bnd[i + 1]) for i in range(K)])
    t13 = np.array([hip.ms(evs[3 * i], evs[3 * i + 1]) for i in range(K)])
    t2 = np.array([hip.ms(evs[3 * i + 1], evs[3 * i + 2]) for i in range(K)])
    hip.destroy(evs)
    hip.destroy(bnd)
    log(f"{cfg}: {K} timed steps, median {float(np.median(step_ms)):.4f} ms")
    out = {}
    if reports:
        out["stages_hbm"] = stage_rates(L, dims, inp, K, hip, stream)
        if L.E % 8 == 0:
            out["placement"] = placement_report(L, dims, inp, host_counts, K, hip, stream)
        out["expert_parallel"] = ranks_report(L, dims, inp, K, hip, stream)
        if L.mode == "router":
            out["router_variants"] = variant_report(L, dims, inp, K, hip, stream)
            out["backward"] = backward_report(L, dims, inp, K, hip, stream)
            out["backward"]["forward_ms_for_reference"] = round(float(np.median(step_ms)), 5)
        log(f"{cfg}: stage and NEXT-row reports done")

    A = L.T * L.k
    med = float(np.median(step_ms))
    flops13 = 4.0 * A * L.d * L.I
    flops2 = 2.0 * A * L.I * L.d
    t13_avg = float(t13.mean())
    t2_avg = float(t2.mean())
    ach13 = flops13 / (t13_avg * 1e-3) / 1e12
    ach_ffn = (flops13 + flops2) / ((t13_avg + t2_avg) * 1e-3) / 1e12
    out.update({
        "tokens_per_s": round(L.T / (med * 1e-3), 1),
        "ms_per_step_mean": round(total_ms / K, 5),
        "step_ms": {"median": round(med, 5),
                    "p10": round(float(np.percentile(step_ms, 10)), 5),
                    "p90": round(float(np.percentile(step_ms, 90)), 5)},
        "config": {"workload": WORKLOADS[cfg], "name": cfg, "T": L.T, "d": L.d, "E": L.E,
                   "k": L.k, "inter": L.I, "mode": L.mode, "tile_m": args.tile_m or "auto",
                   "tile_height": M.tile_height(dims)},
        "dtype": "bf16" if L.dtype == "bf16" else "f32",
        "roofline": {
            "kernel": "grouped_gemm_dma128_kernel<gate/up + SwiGLU, fused gather>",
            "bound": "mfma",
            "achieved": round(ach13, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach13 / PEAK_BF16_TFLOPS, 4),
            "traffic": gemm_traffic(cfg) if not args.tile_m else None,
            "algorithmic": f"4*T*k*d*I = {flops13:.4g} FLOP per launch",
            "avg_launch_ms": round(t13_avg, 5),
        },
        "grouped_gemm": {
            "tflops": round(ach_ffn, 2),
            "frac_bf16_peak": round(ach_ffn / PEAK_BF16_TFLOPS, 4),
            "gate_up_ms": round(t13_avg, 5),
            "down_ms": round(t2_avg, 5),
            "down_tflops": round(flops2 / (t2_avg * 1e-3) / 1e12, 2),
        },
        "wall_s_timed": round(t_wall, 4),
    })
    if cpu_sample > 0:
        tps, secs, threads = cpu_baseline(L, cpu_sample)
        out["cpu_baseline"] = {
            "value": round(tps, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"first {min(cpu_sample, L.T)} of the {L.T} tokens, every stage "
                      f"({secs:.1f} s)",
        }
        log(f"{cfg}: oracle sample done ({secs:.1f} s)")
    del b, inp, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS),
                    help="headline workload (default: the packed-microbatch layer, the "
                         "largest that the metric is quoted on)")
    ap.add_argument("--extra", default="c2,c4,c5",
                    help="further workloads timed in the same run and reported under "
                         "'other_configs' (comma list, '' for none; c5: the decode-shaped "
                         "layer at T = 1 and 64, under 'decode')")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens of the workload the CPU oracle runs (0 = skip)")
    ap.add_argument("--tile-m", type=int, default=0)
    ap.add_argument("--decode-t", default="1,2,4,8,16,32,64",
                    help="batch sizes of the decode-shaped sweep (--config c5)")
    ap.add_argument("--no-reports", action="store_true",
                    help="time the layer steps only (no stage, placement, router-variant, "
                         "expert-parallel or backward reports, no extra workloads): for "
                         "counter passes, whose per-dispatch averages must see the step's "
                         "kernels alone")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(expert-parallel sharding is a design note only); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.config == "c5":
        decode_sweep(args)
        return

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()
    stream = torch.cuda.current_stream()
    head = run_layer(args.config, args, hip, not args.no_reports, args.cpu_sample)
    extra = {}
    decode = None
    if not args.no_reports:
        head["ep_share"] = ep_share_report(args.steps, hip, stream)
        log("expert-parallel share done")
        for cfg in [c for c in args.extra.split(",") if c and c != args.config]:
            if cfg == "c5":
                rows, _ = decode_rows([1, 64], min(args.steps, 20), min(args.warmup, 5))
                decode = {"workload": WORKLOADS["c5"], "sweep": rows}
                log("decode-shaped layer done")
                continue
            r = run_layer(cfg, args, hip, reports=(cfg == "c2"), cpu_sample=0)
            extra[cfg] = {n: r[n] for n in ("tokens_per_s", "step_ms", "grouped_gemm",
                                            "roofline", "router_variants", "backward",
                                            "placement", "stages_hbm", "expert_parallel")
                          if n in r}
            extra[cfg]["workload"] = r["config"]["workload"]

    rec = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"]["median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "peak": derived_peak(hip),
        "grouped_gemm": head["grouped_gemm"],
        "step_ms": head["step_ms"],
        "ms_per_step_mean": head["ms_per_step_mean"],
        "stages_hbm": head.get("stages_hbm"),
        "placement": head.get("placement"),
        "expert_parallel": head.get("expert_parallel"),
        "router_variants": head.get("router_variants"),
        "backward": head.get("backward"),
        "ep_share": head.get("ep_share"),
        "other_configs": extra or None,
        "decode": decode,
        "wall_s_timed": head["wall_s_timed"],
        "cpu_baseline": head.get("cpu_baseline"),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
