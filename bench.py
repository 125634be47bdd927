"""Benchmark of one full-attention layer decision on one MI355X.

A step = block scores -> Top-p select -> expand + compact -> compose, over one batch
of synthetic inputs already resident in HBM (default: the Llama-3.1-8B shape at 128K
tokens).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--p P]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/sec selected+compacted per layer at 128K; % MFMA peak, % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# Kernel instances the headline decision launches (d = 128, contiguous keys, 16-byte rows),
# as rocprofv3 names them.
SCORE_KERNEL = "up_score_partial_kernel<128, 2, 4, 8, false, false>"
GATHER_KERNEL = "up_gather_kernel<unsigned int __vector(4), 128, 2>"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, scaled by the plain-copy calibration; None
    if there is no summary or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    scale = None
    for line in open(path):
        if line.startswith("scale "):
            parts = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
            scale = float(parts["fetch"]), float(parts["write"])
            continue
        if not line.startswith("kernel=") or " | " not in line:
            continue
        name, rest = line[len("kernel="):].split(" | ", 1)
        parts = dict(kv.split("=", 1) for kv in rest.split() if "=" in kv)
        if name.strip() == kernel and scale:
            src = os.path.join(ROOT, parts["source"])
            if not os.path.exists(src):
                return None
            if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != parts["sha256"]:
                return None
            return (float(parts["fetch_kib"]) * scale[0] + float(parts["write_kib"]) * scale[1]) * 1024
    return None


def causal_pairs(L: int, W: int) -> int:
    """(query, key) pairs one head scores: W*(L-W) + W*(W+1)/2."""
    return W * (L - W) + W * (W + 1) // 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama31_8b_128k")
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline decision (no given-lse, two-stream or paged "
                         "legs): the mode the rocprofv3 summaries are taken in")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="BYTES",
                    help="only time a plain device-to-device copy of BYTES (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this build has no "
              "multi-GPU path; the per-GPU share is what one GPU measures.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_reference:
        copy_reference(torch, args.copy_reference, args.steps)
        return
    import block_wise_token_amd as up
    from workloads import synth

    cfg = synth.WORKLOADS[args.workload]
    p = cfg["p"] if args.p is None else args.p
    t0 = time.time()
    b = synth.make_batch(cfg)
    hidden = synth.gen_hidden(b.T, cfg["H"], cfg["seed"])
    pos = synth.positions(b.cu_seqlens)
    log(f"[bench] generated {args.workload}: T={b.T} in {time.time() - t0:.1f}s")

    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    qwin, k, hid = bf16(b.qwin), bf16(b.k), bf16(hidden)
    cu = torch.from_numpy(b.cu_seqlens).to(dev)
    posd = torch.from_numpy(pos).to(dev)
    dec = up.LayerDecision(qwin, k, cu, b.cu_seqlens, hid, posd, b.n, b.G, p)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0, "device error word set"
    log(f"[bench] warmup done ({args.warmup} steps)")

    # Timed region: K steps, nothing instrumented.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        dec.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})")

    # Same K steps again with the library's per-kernel HIP events on the launch stream.
    up.profile_reset()
    up.profile_enable(True)
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record(stream)
    for _ in range(args.steps):
        dec.run()
    ev3.record(stream)
    torch.cuda.synchronize()
    up.profile_enable(False)
    ms_step_instr = ev2.elapsed_time(ev3) / args.steps
    kern = {}
    for name in up.KERNEL_IDS:
        n, ms = up.profile_read(name)
        if n:
            kern[name] = {"launches": n, "avg_us": ms * 1e3 / n}
    up.profile_reset()
    assert up.device_error() == 0

    kept = int(dec.cu_out[-1].item())
    T = b.T
    row_bytes = cfg["H"] * 2
    # Algorithmic work per launch.
    pairs = sum(causal_pairs(int(L), min(b.n, int(L))) for L in np.diff(b.cu_seqlens))
    score_flops = 2.0 * b.d * b.Hq * pairs                          # one Q K^T over causal pairs
    # rows read + written, position read + written, index written, and the fused drop
    # composition: previous original index read + composed index written
    gather_bytes = kept * (2 * row_bytes + 12 + 8)
    s_us = kern["score_partial"]["avg_us"]
    g_us = kern["gather"]["avg_us"]
    # Score pass bytes: K and the window queries read once, 8 B per (row, block) and per
    # (row, key chunk) of softmax statistics written.  Below the ridge point (peak flops
    # over peak bandwidth) the pass is bounded by HBM, above it by the matrix cores.
    nb_tot = int(sum((int(L) + b.G - 1) // b.G for L in np.diff(b.cu_seqlens)))
    score_bytes = (2.0 * T * b.Hkv * b.d + 2.0 * b.qwin.shape[0] * b.Hq * b.d
                   + 8.0 * nb_tot * b.Hq * b.n)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    score_tflops = score_flops / (s_us * 1e-6) / 1e12
    gather_gbs = gather_bytes / (g_us * 1e-6) / 1e9
    if score_flops / score_bytes >= ridge:
        roof_score = {"bound": "mfma", "achieved": round(score_tflops, 2),
                      "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(score_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                      "work_per_launch": score_flops}
    else:
        score_gbs = score_bytes / (s_us * 1e-6) / 1e9
        roof_score = {"bound": "hbm", "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                      "work_per_launch": score_bytes,
                      "mfma_tflops": round(score_tflops, 2)}
    roof_score.update({"traffic": measured_traffic(args.workload, SCORE_KERNEL)
                       if b.d == 128 else None,
                       "kernel": "up_score_partial_kernel", "avg_us": round(s_us, 2),
                       "flop_per_byte": round(score_flops / score_bytes, 1),
                       "variant": "one pass: a single Q K^T over the causal keys keeps a "
                                  "per-(row, block) sum relative to its statistics chunk's "
                                  "reference; row statistics and block masses follow from "
                                  "them (no second Q K^T)"})
    roof_gather = {"bound": "hbm", "achieved": round(gather_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(args.workload, GATHER_KERNEL),
                   "kernel": "up_gather_kernel", "avg_us": round(g_us, 2),
                   "work_per_launch": gather_bytes}
    dominant = roof_gather if g_us >= s_us else roof_score

    result = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": b.B, "T": T, "Hq": b.Hq, "Hkv": b.Hkv,
                   "d": b.d, "n": b.n, "G": b.G, "p": p, "H": cfg["H"], "seed": cfg["seed"],
                   "kept_tokens": kept, "rho": kept / T},
        "roofline": dominant,
        "rooflines": {"score": roof_score, "gather": roof_gather},
        "kernels_avg_us": {k2: round(v["avg_us"], 2) for k2, v in kern.items()},
        "ms_per_step_instrumented": ms_step_instr,
    }

    # The scope's next row: the same decision given each window row's log-sum-exp (what
    # the layer's own attention keeps), here taken from the full pass's row_lse output.
    # Reported beside the headline, which runs every step of the path itself.
    if not args.headline_only:
        result["median_flushed"] = median_flushed_leg(torch, dec, stream, T)
        result["given_lse"] = given_lse_leg(up, torch, dec, qwin, k, cu, b, hid, posd, p, args,
                                            stream, score_flops)

    # Independent decisions (a stream of requests) on two HIP streams: one request's
    # HBM-bound compaction runs beside the next one's compute-bound scoring.
    if not args.headline_only:
        result["two_streams"] = two_streams_leg(up, torch, dec, qwin, k, cu, b, hid, posd, p,
                                                args)

    # Top-k instead of Top-p (scope: next), with k = the blocks the Top-p cut kept.
    if not args.headline_only:
        result["topk"] = topk_leg(up, torch, dec, qwin, k, cu, b, hid, posd, args, stream)

    # Keys read through a block table from a paged cache (scope: next), score pass only.
    if not args.headline_only:
        result["paged_keys"] = paged_keys_leg(up, torch, qwin, k, cu, b, args)

    # Every layer of a multi-layer workload, drops composed across layers.
    if not args.headline_only and cfg.get("layers", 1) > 1:
        result["stack"] = stack_leg(up, torch, cfg, b, hid, posd, p, args)

    # The other cut thresholds of the 128K configuration.
    if not args.headline_only and args.workload == "llama31_8b_128k" and args.p is None:
        result["p_sweep"] = p_sweep_leg(up, torch, qwin, k, cu, b, hid, posd, args, stream,
                                        row_bytes)

    # The decision captured once into a HIP graph and replayed.
    if not args.headline_only:
        result["graph"] = graph_leg(up, torch, dec, args, T)

    # One tensor-parallel rank's share of the heads (8 ranks), score pass only.
    if not args.headline_only:
        result["tp8_share"] = tp_share_leg(up, torch, qwin, k, cu, b, args, s_us)

    # What a plain device-to-device copy of the gather's row bytes reaches on this GPU:
    # the practical ceiling the gather's HBM fraction is read against.
    if not args.headline_only:
        result["copy_ceiling"] = copy_ceiling_leg(torch, kept * row_bytes, g_us, gather_bytes)

    # The layer that then runs on the survivors (scope: next), against the same layer on
    # every token.
    if not args.headline_only and b.d in (64, 128, 256):
        F = ffn_width(cfg["H"])
        if b.T * 2 * F >= 1 << 32:
            # the layer library refuses GEMM operands of 2^32 elements or more
            result["consumer"] = {"skipped": f"the FFN of {b.T} rows at width {F} has a "
                                             f"{b.T * 2 * F:.3g}-element operand; GEMMs of "
                                             "2^32 elements or more are refused"}
        else:
            result["consumer"] = consumer_leg(up, torch, dec, hid, b, cfg)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(b, hidden, pos, p, cfg)
    print(json.dumps(result), flush=True)


def ffn_width(H):
    """FFN width: Llama-3.1-8B's for H = 4096, Gemma-3-12B's for H = 3840."""
    return {4096: 14336, 3840: 15360}.get(H, int(round(3.5 * H / 256)) * 256)


def consumer_leg(up, torch, dec, hid, b, cfg, reps=2):
    """One decoder layer with random weights -- q, k, v projections, rotary attention at
    the carried positions, output projection plus residual, SwiGLU FFN plus residual --
    on the survivors of the headline decision and on every token (no drop, positions
    0..N-1).  Weights and inputs are seeded; nothing here is part of `value`."""
    import math
    H, Hq, Hkv, d = cfg["H"], b.Hq, b.Hkv, b.d
    F = ffn_width(H)
    dev = hid.device
    g = torch.Generator(device=dev).manual_seed(20260)

    def w(n, k_):
        return (torch.randn(n, k_, generator=g, device=dev) / math.sqrt(k_)).to(torch.bfloat16)

    Wq, Wk, Wv, Wo = w(Hq * d, H), w(Hkv * d, H), w(Hkv * d, H), w(H, Hq * d)
    Wgu, Wd = w(2 * F, H), w(H, F)
    N = b.T
    kept = int(dec.cu_out[-1].item())
    cu_all_h = b.cu_seqlens
    cu_kept_h = dec.cu_out.cpu().numpy()
    cu_all = torch.from_numpy(cu_all_h).to(dev)
    pos_all = torch.from_numpy(synth_positions(cu_all_h)).to(dev)
    buf = {name: torch.empty((N, cols), dtype=torch.bfloat16, device=dev)
           for name, cols in (("q", Hq * d), ("k", Hkv * d), ("v", Hkv * d), ("att", Hq * d),
                              ("h2", H), ("y", H))}
    ws_att = torch.empty(max(up.rope_attention_workspace_bytes(cu_all_h, Hq, Hkv, d),
                             up.rope_attention_workspace_bytes(cu_kept_h, Hq, Hkv, d)),
                         dtype=torch.uint8, device=dev)
    ws_ffn = torch.empty(up.swiglu_ffn_workspace_bytes(N, H, F), dtype=torch.uint8, device=dev)
    ws_gemm = torch.empty(32 << 20, dtype=torch.uint8, device=dev)

    def layer(x, pos, cu, cu_h, R):
        q = up.linear(x, Wq, out=buf["q"][:R], workspace=ws_gemm)
        k_ = up.linear(x, Wk, out=buf["k"][:R], workspace=ws_gemm)
        v = up.linear(x, Wv, out=buf["v"][:R], workspace=ws_gemm)
        att = up.rope_attention(q.view(R, Hq, d), k_.view(R, Hkv, d), v.view(R, Hkv, d), pos, cu,
                                cu_h, out=buf["att"][:R].view(R, Hq, d), workspace=ws_att)
        h2 = up.linear(att.view(R, Hq * d), Wo, residual=x, out=buf["h2"][:R], workspace=ws_gemm)
        return up.swiglu_ffn(h2, Wgu, Wd, residual=h2, out=buf["y"][:R], workspace=ws_ffn)

    stream = torch.cuda.current_stream()
    cases = {"survivors": (dec.hidden_out[:kept], dec.pos_out[:kept], dec.cu_out, cu_kept_h, kept),
             "all_tokens": (hid, pos_all, cu_all, cu_all_h, N)}
    out = {}
    for name, (x, pos, cu, cu_h, R) in cases.items():
        layer(x, pos, cu, cu_h, R)                       # warm-up (GEMM plans, caches)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            layer(x, pos, cu, cu_h, R)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        up.profile_reset()
        up.profile_enable(True)
        layer(x, pos, cu, cu_h, R)
        torch.cuda.synchronize()
        up.profile_enable(False)
        kt = {}
        for kname in ("attn_plan", "rope_layout", "attention", "swiglu"):
            n, tot = up.profile_read(kname)
            if n:
                kt[kname] = round(tot * 1e3, 1)          # microseconds per layer
        up.profile_reset()
        assert up.device_error() == 0
        # The GEMMs (libuniprefill_layer.so, hipBLASLt): the layer's six, timed together.
        a_ffn = torch.empty((R, F), dtype=torch.bfloat16, device=dev)
        gu = torch.empty((R, 2 * F), dtype=torch.bfloat16, device=dev)

        def gemms():
            up.linear(x, Wq, out=buf["q"][:R], workspace=ws_gemm)
            up.linear(x, Wk, out=buf["k"][:R], workspace=ws_gemm)
            up.linear(x, Wv, out=buf["v"][:R], workspace=ws_gemm)
            up.linear(buf["att"][:R], Wo, residual=x, out=buf["h2"][:R], workspace=ws_gemm)
            up.linear(buf["h2"][:R], Wgu, out=gu, workspace=ws_gemm)
            up.linear(a_ffn, Wd, out=buf["y"][:R], workspace=ws_gemm)
        gemms()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            gemms()
        g1.record(stream)
        torch.cuda.synchronize()
        kt["gemm"] = round(g0.elapsed_time(g1) / reps * 1e3, 1)
        del gu, a_ffn
        pairs = sum(int(L) * (int(L) + 1) // 2 for L in np.diff(cu_h))
        att_flops = 4.0 * d * Hq * pairs                  # Q K^T and P V over causal pairs
        gemm_flops = 2.0 * R * H * (Hq * d + 2 * Hkv * d + Hq * d + 3 * F)
        att_tf = att_flops / (kt["attention"] * 1e-6) / 1e12
        out[name] = {"rows": R, "ms": round(ms, 3), "kernel_us": kt,
                     "attention_tflops": round(att_tf, 1),
                     "attention_frac": round(att_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "gemm_tflops": round(gemm_flops / (kt["gemm"] * 1e-6) / 1e12, 1)}
        log(f"[bench] consumer {name}: {R} rows, {ms:.2f} ms/layer, attention {att_tf:.0f} TFLOP/s")
    out["scores_in_attention"] = scores_in_attention_leg(up, torch, buf, b, pos_all, cu_all,
                                                         cu_all_h, ws_att, reps)
    out["time_ratio"] = round(out["survivors"]["ms"] / out["all_tokens"]["ms"], 4)
    out["rho"] = round(kept / N, 4)
    out["note"] = ("one decoder layer (projections, rotary attention at the carried positions, "
                   "SwiGLU FFN width %d) with random weights; not the headline" % F)
    return out


def scores_in_attention_leg(up, torch, buf, b, pos_all, cu_all, cu_all_h, ws_att, reps):
    """The full-attention layer's attention on every token, alone and with the block
    scores of its window rows taken inside it (up_rope_attention_scores), against the
    separate score pass over the same q and k (up_block_scores); per-kernel HIP events,
    microseconds per call."""
    Hq, Hkv, d, n, G = b.Hq, b.Hkv, b.d, b.n, b.G
    R = b.T
    dev = buf["q"].device
    q = buf["q"][:R].view(R, Hq, d)
    k_ = buf["k"][:R].view(R, Hkv, d)
    v = buf["v"][:R].view(R, Hkv, d)
    att = buf["att"][:R].view(R, Hq, d)
    nb = int(sum((int(L) + G - 1) // G for L in np.diff(cu_all_h)))
    sc = torch.empty(nb, dtype=torch.float32, device=dev)
    ws_as = torch.empty(up.rope_attention_scores_workspace_bytes(cu_all_h, Hq, Hkv, d, n, G),
                        dtype=torch.uint8, device=dev)
    win = np.concatenate([np.arange(max(int(cu_all_h[i + 1]) - n, int(cu_all_h[i])),
                                    int(cu_all_h[i + 1]))
                          for i in range(len(cu_all_h) - 1)])
    qwin = q[torch.from_numpy(win).to(dev)].contiguous()
    ws_bs = torch.empty(up.block_scores_workspace_bytes(cu_all_h, Hq, Hkv, d, n, G),
                        dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()

    def timed(fn, names):
        """(microseconds per whole call on the caller's stream, per-kernel averages)."""
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        call_us = e0.elapsed_time(e1) * 1e3 / reps
        up.profile_reset()
        up.profile_enable(True)
        fn()
        torch.cuda.synchronize()
        up.profile_enable(False)
        res = {}
        for nm in names:
            cnt, ms = up.profile_read(nm)
            if cnt:
                res[nm] = round(ms * 1e3 / cnt, 2)
        up.profile_reset()
        assert up.device_error() == 0
        return call_us, res

    def plain_call():
        up.rope_attention(q, k_, v, pos_all, cu_all, cu_all_h, out=att, workspace=ws_att)

    def fused_call():
        up.rope_attention_scores(q, k_, v, pos_all, cu_all, cu_all_h, n, G, out=att, scores=sc,
                                 workspace=ws_as)

    plain_names = ("attn_plan", "rope_layout", "attention")
    fused_names = ("score_plan", "attn_plan", "rope_layout", "attention", "attention_window",
                   "block_mass", "normalize")
    runs = [(timed(plain_call, plain_names), timed(fused_call, fused_names)) for _ in range(2)]
    plain_us, plain = min((r[0] for r in runs), key=lambda x: x[0])   # alternated, best of two
    fused_us, fused = min((r[1] for r in runs), key=lambda x: x[0])
    sep_us, sep = timed(lambda: up.block_scores(qwin, k_, cu_all, cu_all_h, n, G, out=sc,
                                                workspace=ws_bs),
                        ("score_plan", "score_partial", "row_stats", "block_mass", "normalize"))
    return {"attention_call_us": round(plain_us, 1), "attention_with_scores_call_us":
            round(fused_us, 1), "extra_us": round(fused_us - plain_us, 1),
            "separate_score_pass_call_us": round(sep_us, 1),
            "kernels_us": {"attention": plain, "attention_with_scores": fused,
                           "separate_score_pass": sep},
            "note": "block scores of the window rows taken inside the layer's attention on "
                    "every token (the window tiles on a second stream beside the others): "
                    "extra_us is what the scores add to the attention call; the separate "
                    "pass re-reads K and recomputes the window's Q K^T"}


def synth_positions(cu_h):
    from workloads import synth
    return synth.positions(cu_h)


def median_flushed_leg(torch, dec, stream, T, reps=100, warmup=20, flush_bytes=1 << 30):
    """Median of individually timed decisions with a 1 GiB write between them, so
    that no input is left in the 256 MB Infinity Cache from the previous rep."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dec.run()
    times = []
    for _ in range(reps):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dec.run()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    med = float(np.median(times))
    del scratch
    return {"reps": reps, "median_ms": med, "p10_ms": float(np.percentile(times, 10)),
            "p90_ms": float(np.percentile(times, 90)), "tokens_per_s": T / (med * 1e-3),
            "note": "1 GiB written between reps (Infinity Cache flushed); not the headline"}


def given_lse_leg(up, torch, dec_full, qwin, k, cu, b, hid, posd, p, args, stream, score_flops):
    lse = torch.empty((qwin.shape[0], b.Hq), dtype=torch.float32, device=qwin.device)
    up.block_scores(qwin, k, cu, b.cu_seqlens, b.n, b.G, row_lse=lse)
    dec = up.LayerDecision(qwin, k, cu, b.cu_seqlens, hid, posd, b.n, b.G, p, row_lse=lse)
    for _ in range(args.warmup):
        dec.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        dec.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    up.profile_reset()
    up.profile_enable(True)
    for _ in range(args.steps):
        dec.run()
    torch.cuda.synchronize()
    up.profile_enable(False)
    kern = {}
    for name in ("score_plan", "score_partial_lse", "lse_finalize", "select", "block_dst", "gather"):
        n_, t_ = up.profile_read(name)
        if n_:
            kern[name] = round(t_ * 1e3 / n_, 2)
    up.profile_reset()
    assert up.device_error() == 0
    same = bool(torch.equal(dec.keep, dec_full.keep))
    s_us = kern.get("score_partial_lse", float("nan"))
    return {"ms_per_step": ms, "tokens_per_s": b.T / (ms * 1e-3), "kernels_avg_us": kern,
            "score_tflops": round(score_flops / (s_us * 1e-6) / 1e12, 2),
            "same_keep_as_full_pass": same,
            "note": "scores from given window-row log-sum-exp (up_block_scores_lse); not the "
                    "headline, which computes the row statistics itself"}


def topk_leg(up, torch, dec_p, qwin, k, cu, b, hid, posd, args, stream):
    """The decision with a Top-k cut (k = the number of blocks the headline's Top-p cut
    kept, so both keep the same number of blocks), timed like the headline."""
    if b.B != 1:
        return None
    kblocks = int(dec_p.keep.sum().item())
    dec = up.LayerDecision(qwin, k, cu, b.cu_seqlens, hid, posd, b.n, b.G, 1.0, topk=kblocks)
    for _ in range(args.warmup):
        dec.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        dec.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    up.profile_reset()
    up.profile_enable(True)
    dec.run()
    torch.cuda.synchronize()
    up.profile_enable(False)
    n_, t_ = up.profile_read("select")
    up.profile_reset()
    assert up.device_error() == 0
    same = bool(torch.equal(dec.keep, dec_p.keep))
    del dec
    return {"k_blocks": kblocks, "ms_per_step": ms, "tokens_per_s": b.T / (ms * 1e-3),
            "select_us": round(t_ * 1e3 / max(n_, 1), 2), "same_keep_as_top_p": same,
            "note": "Top-k cut with k = the Top-p cut's block count; not the headline"}


def two_streams_leg(up, torch, dec_a, qwin, k, cu, b, hid, posd, p, args):
    """Throughput of independent decisions issued alternately on two streams (each
    decision has its own buffers; both read the same resident inputs)."""
    dec_b = up.LayerDecision(qwin, k, cu, b.cu_seqlens, hid, posd, b.n, b.G, p)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for j in range(2 * args.warmup):
        (dec_a if j % 2 == 0 else dec_b).run(stream=sa if j % 2 == 0 else sb)
    torch.cuda.synchronize()
    n = 2 * args.steps
    t0 = time.perf_counter()
    for j in range(n):
        (dec_a if j % 2 == 0 else dec_b).run(stream=sa if j % 2 == 0 else sb)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert up.device_error() == 0
    same = bool(torch.equal(dec_a.keep, dec_b.keep))
    return {"decisions": n, "ms_per_decision": dt * 1e3 / n, "tokens_per_s": b.T * n / dt,
            "same_keep": same, "note": "two independent decisions in flight on two HIP "
                                       "streams; wall clock; not the headline"}


def paged_keys_leg(up, torch, qwin, k, cu, b, args, page_size=16):
    """Score pass with the keys scattered into shuffled pages of 16 tokens (the input
    layout built here with torch indexing), timed against the contiguous pass (best of
    three alternating rounds each)."""
    if b.B != 1 or b.T % page_size:
        return None
    npg = b.T // page_size
    g = torch.Generator(device="cpu").manual_seed(7)
    perm = torch.randperm(npg, generator=g).to(k.device)
    pages = torch.empty((npg, page_size) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    pages[perm] = k.view((npg, page_size) + tuple(k.shape[1:]))
    table = perm.to(torch.int32).view(1, npg).contiguous()
    lse = torch.empty((qwin.shape[0], b.Hq), dtype=torch.float32, device=qwin.device)
    up.block_scores(qwin, k, cu, b.cu_seqlens, b.n, b.G, row_lse=lse)
    out = {}
    legs = (
        ("contiguous", "score_partial",
         lambda: up.block_scores(qwin, k, cu, b.cu_seqlens, b.n, b.G)),
        ("paged", "score_partial",
         lambda: up.block_scores_paged(qwin, pages, table, cu, b.cu_seqlens, b.n, b.G)),
        ("lse_contiguous", "score_partial_lse",
         lambda: up.block_scores_lse(qwin, k, lse, cu, b.cu_seqlens, b.n, b.G)),
        ("lse_paged", "score_partial_lse",
         lambda: up.block_scores_lse_paged(qwin, pages, table, lse, cu, b.cu_seqlens, b.n, b.G)),
    )
    # The four passes alternate over three rounds and each keeps its best round, so
    # that none of them is favoured by the clock state it happens to start in.
    res, best = {}, {}
    for _ in range(3):
        for name, kname, fn in legs:
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            up.profile_reset()
            up.profile_enable(True)
            for _ in range(args.steps):
                res[name] = fn()
            torch.cuda.synchronize()
            up.profile_enable(False)
            n_, t_ = up.profile_read(kname)
            best[name] = min(best.get(name, float("inf")), t_ * 1e3 / n_)
            up.profile_reset()
    for name in best:
        out[name + "_score_us"] = round(best[name], 2)
    assert up.device_error() == 0
    out.update({"page_size": page_size,
                "bit_identical": bool(torch.equal(res["contiguous"], res["paged"])),
                "bit_identical_lse": bool(torch.equal(res["lse_contiguous"], res["lse_paged"]))})
    return out


def tp_share_leg(up, torch, qwin, k, cu, b, args, score_us_full, tp=8):
    """The score pass on one tensor-parallel rank's heads (Hq/tp query heads, Hkv/tp kv
    heads: what each of tp GPUs would run on its own, at its real shape), timed like the
    headline's score kernel; the all-gather of block masses that would follow is not
    built (one GPU)."""
    if b.Hq % tp or b.Hkv % tp:
        return None
    hq, hk = b.Hq // tp, b.Hkv // tp
    q_r, k_r = qwin[:, :hq].contiguous(), k[:, :hk].contiguous()
    pairs = sum(causal_pairs(int(L), min(b.n, int(L))) for L in np.diff(b.cu_seqlens))
    flops = 2.0 * b.d * hq * pairs
    out_s = torch.empty(int(sum((int(L) + b.G - 1) // b.G for L in np.diff(b.cu_seqlens))),
                        dtype=torch.float32, device=qwin.device)
    ws = torch.empty(max(1, up.block_scores_workspace_bytes(b.cu_seqlens, hq, hk, b.d, b.n, b.G)),
                     dtype=torch.uint8, device=qwin.device)

    def run():
        up.block_scores(q_r, k_r, cu, b.cu_seqlens, b.n, b.G, out=out_s, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1e3 / args.steps
    up.profile_reset()
    up.profile_enable(True)
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    up.profile_enable(False)
    n_, t_ = up.profile_read("score_partial")
    s_us = t_ * 1e3 / n_
    up.profile_reset()
    assert up.device_error() == 0
    tf = flops / (s_us * 1e-6) / 1e12
    return {"tp": tp, "Hq": hq, "Hkv": hk, "score_kernel_us": round(s_us, 2),
            "score_tflops": round(tf, 2), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "block_scores_call_us": round(call_us, 2),
            "full_heads_score_kernel_us": round(score_us_full, 2),
            "note": "one rank's share of the heads; the cross-rank exchange is not built"}


def p_sweep_leg(up, torch, qwin, k, cu, b, hid, posd, args, stream, row_bytes):
    """The same decision at the other cut thresholds of the 128K configuration: step
    time, kept fraction and the gather's rate (fewer kept rows, fewer bytes)."""
    out = {}
    for p in (0.95, 0.999):
        dec = up.LayerDecision(qwin, k, cu, b.cu_seqlens, hid, posd, b.n, b.G, p)
        for _ in range(args.warmup):
            dec.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            dec.run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        up.profile_reset()
        up.profile_enable(True)
        for _ in range(args.steps):
            dec.run()
        torch.cuda.synchronize()
        up.profile_enable(False)
        n_, t_ = up.profile_read("gather")
        g_us = t_ * 1e3 / n_
        up.profile_reset()
        assert up.device_error() == 0
        kept = int(dec.cu_out[-1].item())
        gbytes = kept * (2 * row_bytes + 12 + 8)
        out[str(p)] = {"ms_per_step": round(ms, 4), "tokens_per_s": b.T / (ms * 1e-3),
                       "rho": kept / b.T, "gather_us": round(g_us, 2),
                       "gather_GBps": round(gbytes / (g_us * 1e-6) / 1e9, 1)}
    return out


def stack_leg(up, torch, cfg, b0, hid, posd, p, args):
    """Every full-attention layer of a multi-layer workload: layer l scores fresh Q/K
    drawn over the survivors of layer l-1, compacts them and composes the drops (the
    original indices travel with the rows).  Each layer's decision is timed like the
    headline."""
    from workloads import synth
    dev = hid.device

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    T0 = b0.T
    orig = torch.arange(T0, dtype=torch.int32, device=dev)
    orig_np = np.arange(T0, dtype=np.int32)
    layers, total = [], 0.0
    for layer in range(cfg["layers"]):
        if layer == 0:
            b = b0
        else:
            req = synth.gen_layer(orig_np, T0, b0.needles[0], cfg["Hq"], cfg["Hkv"], cfg["d"],
                                  cfg["n"], cfg["G"], cfg["seed"], layer)
            b = synth.pack([req], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["n"], cfg["G"])
        L = b.T
        cu = torch.from_numpy(b.cu_seqlens).to(dev)
        dec = up.LayerDecision(bf16(b.qwin), bf16(b.k), cu, b.cu_seqlens, hid, posd, b.n, b.G, p,
                               prev_orig=orig)
        for _ in range(args.warmup):
            dec.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dec.run()
        e1.record()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        ms = e0.elapsed_time(e1) / args.steps
        kept = int(dec.cu_out[-1].item())
        layers.append({"layer": layer, "tokens": L, "kept": kept, "ms": round(ms, 4),
                       "tokens_per_s": L / (ms * 1e-3)})
        total += ms
        hid, posd = dec.hidden_out[:kept].clone(), dec.pos_out[:kept].clone()
        orig = dec.orig[:kept].clone()
        orig_np = orig.cpu().numpy()
        del dec
    last_kept_orig_ok = bool(np.array_equal(orig_np[-b0.n:], np.arange(T0 - b0.n, T0)))
    return {"layers": layers, "total_ms": round(total, 4), "final_tokens": int(orig_np.size),
            "window_survives": last_kept_orig_ok,
            "note": "each layer's decision timed on its own inputs; not the headline"}


def graph_leg(up, torch, dec_big, args, T_big, reps=50):
    """Decisions replayed from a HIP graph (torch.cuda.CUDAGraph) against the same calls
    launched one by one: at the bench's workload and at the small single-request size
    (4096 tokens, where the host's launch cost matters)."""
    from workloads import synth
    legs = [(args.workload, dec_big, T_big, args.steps)]
    small_name = "single_4k_h8_d64"
    if args.workload != small_name:
        cfg = synth.WORKLOADS[small_name]
        sb = synth.make_batch(cfg)
        dev = dec_big.qwin.device

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        hid = bf16(synth.gen_hidden(sb.T, cfg["H"], cfg["seed"]))
        small = up.LayerDecision(bf16(sb.qwin), bf16(sb.k), torch.from_numpy(sb.cu_seqlens).to(dev),
                                 sb.cu_seqlens, hid,
                                 torch.from_numpy(synth.positions(sb.cu_seqlens)).to(dev),
                                 sb.n, sb.G, cfg["p"])
        legs.append((small_name, small, sb.T, reps))
    else:
        legs = [(small_name, dec_big, T_big, reps)]
    out = {}
    for name, dec, T, n in legs:
        dec.run()
        torch.cuda.synchronize()
        want_keep = dec.keep.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dec.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dec.run()
        g10 = torch.cuda.CUDAGraph()   # ten decisions in one graph
        with torch.cuda.graph(g10):
            for _ in range(10):
                dec.run()
        torch.cuda.synchronize()
        n10 = max(n // 10, 1)
        res = {}
        for mode in ("eager", "graph", "graph10", "eager", "graph", "graph10"):
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            if mode == "graph10":
                for _ in range(n10):
                    g10.replay()
            else:
                for _ in range(n):
                    g.replay() if mode == "graph" else dec.run()
            e1.record(stream)
            torch.cuda.synchronize()
            k = 10 * n10 if mode == "graph10" else n
            wall = (time.perf_counter() - t0) * 1e3 / k
            res.setdefault(mode, []).append((e0.elapsed_time(e1) / k, wall))
        assert up.device_error() == 0
        same = bool(torch.equal(dec.keep, want_keep))
        out[name] = {"tokens": T, "decisions": n,
                     "eager_ms": round(min(x[0] for x in res["eager"]), 4),
                     "graph_ms": round(min(x[0] for x in res["graph"]), 4),
                     "graph10_ms": round(min(x[0] for x in res["graph10"]), 4),
                     "eager_wall_ms": round(min(x[1] for x in res["eager"]), 4),
                     "graph_wall_ms": round(min(x[1] for x in res["graph"]), 4),
                     "same_keep": same}
    out["note"] = ("graph: one decision per graph, replayed back to back; graph10: ten "
                   "decisions per graph (per-decision time); best of two rounds; "
                   "not the headline")
    return out


def copy_ceiling_leg(torch, nbytes, gather_us, gather_bytes, reps=20):
    """torch's device-to-device copy of `nbytes` (read + write), timed like the gather."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    gather_gbs = gather_bytes / (gather_us * 1e-6) / 1e9
    return {"bytes_read_plus_written": 2 * nbytes, "us": round(ms * 1e3, 1), "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gather_vs_copy": round(gather_gbs / gbs, 4),
            "note": "torch copy_ of the kept rows' bytes; the gather moves these plus indices"}


def copy_reference(torch, nbytes, steps):
    """Plain copy of a known number of bytes (torch's device-to-device copy kernel)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_reference_bytes": nbytes, "reads": nbytes, "writes": nbytes,
                      "ms": ms, "GB/s_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}))


def cpu_baseline(b, hidden, pos, p, cfg):
    """The oracle, untuned, timed on this host on whole decisions of the same workload,
    repeated until about ten seconds of CPU work have been done (at most 16)."""
    from oracle import uniprefill_oracle as O
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info] or [1])
        blas = ", ".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in info
                                 if d.get("user_api") == "blas"})) or blas
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    log("[bench] cpu baseline: oracle on full decisions ...")
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 10.0 and reps < 16):
        t0 = time.perf_counter()
        O.decide(b.qwin, b.k, b.cu_seqlens, hidden, pos, b.Hq, b.Hkv, b.d, b.n, b.G, p, fast=True)
        dt += time.perf_counter() - t0
        reps += 1
    log(f"[bench] cpu baseline: {reps} decisions in {dt:.1f}s")
    return {"value": reps * b.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full decisions of {cfg and 'the same workload'} "
                      f"({b.T} tokens each: scores, Top-p, expand, compact, compose), NumPy float64",
            "seconds": dt, "cpu": cpu, "blas": blas}


if __name__ == "__main__":
    main()
