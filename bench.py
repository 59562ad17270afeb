#!/usr/bin/env python3
"""Draft-round benchmark of the DSpark hot path on one MI355X.

One step = one draft round of the chosen head workload, every row of the hot
path, in order on one stream (dspark_draft_round): lm_head GEMV over all
drafted rows -> k-step on-device Markov loop, with the confidence probe on
every drafted row computed in the same launch; the drafted ids and probe
logits are stored by the kernels straight into pinned host memory. Inputs
are seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line (stdout). Progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--config qwen3_8b_head]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft rounds/s + achieved HBM GB/s (% of peak), V=151936 r=256 B=7"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


COUNTERS = os.path.join(ROOT, "profiles", "counters_{workload}.json")


def _sha256(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(workload):
    """HBM bytes per dispatch of each kernel of the round, from the committed
    rocprofv3 counter runs (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    same counter reads for a device-to-device copy of known size). A kernel
    whose source file changed since its counters were taken is reported as
    None. Returns {role: bytes or None} for the roles recorded."""
    path = COUNTERS.format(workload=workload)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    out = {}
    for role, k in rec.get("kernels", {}).items():
        fresh = all(_sha256(src) == sha for src, sha in k.get("sources", {}).items())
        out[role] = k["traffic_bytes_per_dispatch"] if fresh else None
    return out


def round_bytes(cfg):
    """Algorithmic HBM bytes of one round (each weight once per use; W2 once
    per step). A bf16 weight is 2 bytes, a Q8_0 one 34/32 (a binary16 scale
    per 32 int8 quants)."""
    R, B, k, d, V, r = cfg["num_reqs"], cfg["B"], cfg["k"], cfg["d"], cfg["V"], cfg["r"]
    wb = 34 / 32 if cfg.get("weights") == "q8_0" else 2
    rows = R * B
    lm = int(V * d * wb) + rows * d * 4 + rows * V * 4
    mk = int(k * (V * r * wb + R * r * wb) + k * R * V * 4) + R * k * 8 + R * 8
    pr = rows * d * 4 + d * 2 + rows * 8
    return lm, mk, pr


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, seconds, gpu):
    """The fp64 oracle, as it stands, timed on this host on a bounded sample
    of one round of the same workload, scaled to rounds/s:
      * lm_head on the first V/slices vocabulary rows (time x slices),
      * the full k-step Markov loop over all V, run on the base logits the
        GPU produced in the timed rounds (the same fp32 tensor the GPU loop
        read) and teacher-forced along the GPU's drafted tokens,
      * the probe on every drafted row.
    Repeated until about `seconds` of CPU work has been spent.

    The same oracle calls also check the GPU's round: the sampled logits
    against the oracle's within 1e-3 + 1e-3 |o|, every drafted id against
    the oracle's greedy pick at that step, the probe logits within
    1e-4 max(|o|, 1). Positions where the oracle's top-2 margin is below
    1e-3 are near-ties: listed (request, step, GPU token, oracle token,
    runner-up, margin, and whether the GPU's pick is a valid greedy pick),
    whether or not they match."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = [x.get("num_threads", 1) for x in threadpool_info() if x.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # pragma: no cover
        threadpool_limits, threads = None, 1
    R, B, k, V = inp["num_reqs"], inp["B"], inp["k"], inp["V"]
    slices = max(1, V // 16384)
    rows = np.arange(V // slices)
    q8 = inp.get("weights") == "q8_0"
    base, g_ids, g_logit = gpu["base"], gpu["ids"], gpu["logit"]
    t_lm, t_mk, t_pr, n = 0.0, 0.0, 0.0, 0
    check = None
    while True:
        a = time.perf_counter()
        if q8:
            ref_rows = oracle.gemv_q8_rows(inp["Wq_lm"], inp["Wd_lm"], inp["H"], rows)
        else:
            ref_rows = oracle.gemv_rows(inp["W_lm"], inp["H"], rows)
        b = time.perf_counter()
        if q8:
            W1, W2 = oracle.q8_0_to_f64(inp["w1q"], inp["w1d"]), oracle.q8_0_to_f64(inp["w2q"], inp["w2d"])
        else:
            W1, W2 = oracle.bf16_to_f64(inp["w1"]), oracle.bf16_to_f64(inp["w2"])
        steps = []
        for q in range(R):
            prev = int(inp["prev0"][q])
            for i in range(k):
                st = oracle.markov_step(base[q, i], W1, W2, prev)
                g = int(g_ids[q, i])  # identity d2t: the drafted id is the token
                steps.append((q, i, g, st.tok, st.runner_up, st.margin,
                              bool(0 <= g < V and float(st.s.max() - st.s[g]) <= oracle.NEAR_TIE)))
                if not (0 <= g < V):
                    break
                prev = g  # teacher-forced along the GPU's tokens
        c = time.perf_counter()
        ref_logit, _ = oracle.conf_probe(inp["H"], inp["probe_w"], float(inp["probe_bias"]),
                                         float(inp["probe_threshold"]))
        d = time.perf_counter()
        t_lm, t_mk, t_pr, n = t_lm + (b - a), t_mk + (c - b), t_pr + (d - c), n + 1
        log(f"  oracle sample {n}: lm_head slice {b - a:.2f} s, markov {c - b:.2f} s, probe {d - c:.3f} s")
        if check is None:
            lg = gpu["logits"][:, rows].astype(np.float64)
            err = np.abs(lg - ref_rows)
            near = [dict(request=q, step=i, gpu_token=g, oracle_token=o, runner_up=ru, margin=m, gpu_pick_valid=v)
                    for q, i, g, o, ru, m, v in steps if m < oracle.NEAR_TIE]
            bad = [(q, i, g, o) for q, i, g, o, ru, m, v in steps if m >= oracle.NEAR_TIE and g != o]
            perr = np.abs(g_logit.astype(np.float64) - ref_logit) / np.maximum(np.abs(ref_logit), 1.0)
            check = {
                "mode": "component: the oracle's loop reads the GPU's fp32 base logits, teacher-forced",
                "lm_head_rows_checked": int(len(rows)), "lm_head_max_abs_err": float(err.max()),
                "lm_head_within_tol": bool(np.all(err <= 1e-3 + 1e-3 * np.abs(ref_rows))),
                "ids_checked": len(steps), "ids_mismatched_outside_near_ties": len(bad), "mismatches": bad[:16],
                "near_tie_threshold": oracle.NEAR_TIE, "near_ties": len(near), "near_tie_records": near,
                "probe_max_rel_err": float(perr.max()), "probe_within_tol": bool(np.all(perr <= 1e-4)),
            }
        if t_lm + t_mk + t_pr >= seconds:
            break
    per_round = (t_lm * slices + t_mk + t_pr) / n
    # The small workload end to end on one thread (the oracle's own round function).
    single = None
    if threadpool_limits is not None:
        from gemv_markov_argmax_amd import synth
        tiny = synth.round_inputs("tiny")
        with threadpool_limits(limits=1):
            m, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 2.0:
                oracle.draft_round(tiny["W_lm"], tiny["H"], tiny["w1"], tiny["w2"], tiny["prev0"], tiny["num_reqs"],
                                   tiny["B"], tiny["k"], tiny["probe_w"], 0.0, 0.0)
                m += 1
            single = dict(workload="tiny", threads=1, rounds_per_s=m / (time.perf_counter() - t0))
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return dict(value=1.0 / per_round, unit="rounds/s", cores=int(threads), kind="oracle",
                sample=(f"{n} x [lm_head on {len(rows)} of {V} vocab rows (scaled x{slices}) + full {k}-step "
                        f"Markov loop over V={V} on the GPU's base logits + probe on {R * B} rows] of the "
                        f"{inp['name']} workload; fp64 numpy oracle (a correctness oracle, not a tuned CPU "
                        f"implementation), BLAS threads={threads}"),
                cpu_model=_cpu_model(), affinity_cores=affinity, single_thread=single), check


def bench_layer(args, dev):
    """One step = one draft layer at M = 7 plus the 7424-wide probe on the 7
    drafted rows. The layer's projections run as a transformer layer runs
    them: q, k and v share their input and go as one GEMV over the
    concatenated [3 * 4096, 4096] weight, gate and up likewise over
    [2 * 12288, 4096]; o and down on their own (4 launches, every weight byte
    read once, as with 7 separate GEMVs). The seven separate GEMVs are timed
    too. Steps cycle through --layer-copies distinct weight sets, like a
    multi-layer drafter, so no weight is served from the Infinity Cache."""
    import numpy as np
    import torch

    from gemv_markov_argmax_amd import ops, synth

    log(f"[bench] generating draft_layer inputs ({args.layer_copies} weight copies)")
    inp = synth.layer_inputs(copies=args.layer_copies)
    names = list(inp["layers"][0].keys())
    Ws = [{nm: ops.bf16_from_bits(lw[nm], dev) for nm in names} for lw in inp["layers"]]
    fnames = list(synth.FUSED_INPUT.keys())
    Wf = [{nm: ops.bf16_from_bits(w, dev) for nm, w in synth.fused_layer(lw).items()} for lw in inp["layers"]]
    Xs = {nm: torch.from_numpy(inp["X"][nm]).to(dev) for nm in names}
    Xf = {nm: Xs[synth.FUSED_INPUT[nm]] for nm in fnames}
    Ys = {nm: torch.empty(inp["M"], Ws[0][nm].shape[0], device=dev) for nm in names}
    Yf = {nm: torch.empty(inp["M"], Wf[0][nm].shape[0], device=dev) for nm in fnames}
    px = torch.from_numpy(inp["probe_x"]).to(dev)
    pw = ops.bf16_from_bits(inp["probe_w"], dev)
    plog = torch.empty(inp["M"], device=dev)
    ppass = torch.empty(inp["M"], dtype=torch.int32, device=dev)
    M = inp["M"]

    def gbytes(W):
        return W.numel() * 2 + M * W.shape[1] * 4 + M * W.shape[0] * 4

    gemv_bytes = {nm: gbytes(Ws[0][nm]) for nm in names}
    fused_bytes = {nm: gbytes(Wf[0][nm]) for nm in fnames}
    probe_bytes = M * inp["probe_width"] * 4 + inp["probe_width"] * 2 + M * 8
    layer_bytes = sum(fused_bytes.values()) + probe_bytes

    def step_fused(c):
        for nm in fnames:
            ops.proj_smallm(Wf[c][nm], Xf[nm], out=Yf[nm])
        ops.conf_probe(px, pw, 0.0, 0.0, logit_out=plog, pass_out=ppass)

    def step_separate(c):
        for nm in names:
            ops.proj_smallm(Ws[c][nm], Xs[nm], out=Ys[nm])
        ops.conf_probe(px, pw, 0.0, 0.0, logit_out=plog, pass_out=ppass)

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_layers(step):
        for s_ in range(args.warmup):
            step(s_ % args.layer_copies)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record()
        for s_ in range(args.steps):
            step(s_ % args.layer_copies)
        b.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(b) * 1e3 / args.steps

    # Timed region: whole layers back to back, one pair of events around all.
    elapsed, layer_us = timed_layers(step_fused)
    elapsed_sep, layer_us_sep = timed_layers(step_separate)

    # Per projection (outside the timed region): the same GEMV launched back to
    # back over the weight copies, one pair of events around the batch.
    def per_gemv(Wsets, Xd, Yd, nms):
        per = {}
        for nm in nms:
            n = 8 * args.layer_copies
            a.record()
            for j in range(n):
                ops.proj_smallm(Wsets[j % args.layer_copies][nm], Xd[nm], out=Yd[nm])
            b.record()
            torch.cuda.synchronize()
            per[nm] = a.elapsed_time(b) * 1e3 / n
        return per

    per_f = per_gemv(Wf, Xf, Yf, fnames)
    per_s = per_gemv(Ws, Xs, Ys, names)
    gbs_f = {nm: fused_bytes[nm] / (per_f[nm] * 1e-6) / 1e9 for nm in fnames}
    gbs_s = {nm: gemv_bytes[nm] / (per_s[nm] * 1e-6) / 1e9 for nm in names}
    tot_f, tot_s = sum(per_f.values()), sum(per_s.values())
    agg = sum(fused_bytes.values()) / (tot_f * 1e-6) / 1e9
    agg_s = sum(gemv_bytes.values()) / (tot_s * 1e-6) / 1e9
    log(f"[bench] draft_layer: {args.steps / elapsed:.1f} layers/s ({layer_us:.1f} us per layer incl. probe); "
        f"GEMV sum {tot_f:.1f} us = {agg:.0f} GB/s; "
        + ", ".join(f"{nm} {per_f[nm]:.1f} us ({gbs_f[nm]:.0f} GB/s)" for nm in fnames))
    log(f"[bench] seven separate GEMVs: {args.steps / elapsed_sep:.1f} layers/s ({layer_us_sep:.1f} us per layer); "
        f"GEMV sum {tot_s:.1f} us = {agg_s:.0f} GB/s; "
        + ", ".join(f"{nm} {per_s[nm]:.1f} us ({gbs_s[nm]:.0f} GB/s)" for nm in names))
    out = {
        "metric": "draft layers/s + achieved HBM GB/s of the M=7 projections",
        "value": args.steps / elapsed, "unit": "layers/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "draft_layer", "M": M, "d": inp["d"], "ffn": inp["ffn"],
                   "probe_width": inp["probe_width"], "weight_copies": args.layer_copies,
                   "projections": "qkv [12288,4096], o [4096,4096], gate_up [24576,4096], down [4096,12288]"},
        "roofline": {"bound": "hbm", "kernel": "proj_smallm GEMVs (4 per layer)", "achieved": agg,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": agg / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_layer": sum(fused_bytes.values()), "gemv_us_per_layer": tot_f},
        "per_gemv": {nm: {"us": per_f[nm], "GB/s": gbs_f[nm], "bytes": fused_bytes[nm]} for nm in fnames},
        "step_hbm": {"achieved": layer_bytes / (layer_us * 1e-6) / 1e9, "unit": "GB/s", "layer_us": layer_us},
        "separate_gemvs": {"layers_per_s": args.steps / elapsed_sep, "layer_us": layer_us_sep, "gemv_us": tot_s,
                           "GB/s": agg_s,
                           "per_gemv": {nm: {"us": per_s[nm], "GB/s": gbs_s[nm]} for nm in names}},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_block(args, dev, layers: int, with_head: bool):
    """draft_block: one step = one draft block forward (rmsnorm, fused qkv,
    attention over 512 context positions, o + residual, rmsnorm, fused
    gate/up, SiLU gate, down + residual) at M = 7, d = 4096, 32 heads of 128,
    F = 12288, cycling over 4 weight copies so that no weight is served from
    the Infinity Cache.
    draft_round_8l: one step = a whole draft round: the fc projection
    ([4096, 4096]), 8 blocks (8 x 436 MB of layer weights, each block with
    its own context cache), the final norm, then the Qwen3-8B head round
    (dspark_draft_round: lm_head, Markov loop, probe): 4.8 GB of weights,
    about the ~4.7 GB SharpInference #441 says its drafter streams per round.
    Each block is one dspark_draft_block call."""
    import numpy as np
    import torch

    from gemv_markov_argmax_amd import ops, synth

    R, B, H, Dh, F, L = 1, 7, 32, 128, 12288, 512
    M, d = R * B, H * Dh
    n_w = layers if with_head else 4
    log(f"[bench] generating {n_w} draft blocks (d={d}, F={F}, context {L})")
    blocks = []
    for c in range(n_w):
        inp = synth.block_inputs(R, B, H, Dh, F, L, [L], synth.config_seed("draft_layer") + 100 * c)
        blocks.append(dict(w={k: ops.bf16_from_bits(v, dev) for k, v in inp["layers"][0].items()},
                           kc=ops.bf16_from_bits(inp["k_ctx"], dev).view(R, L, d),
                           vc=ops.bf16_from_bits(inp["v_ctx"], dev).view(R, L, d)))
        if c == 0:
            h0 = torch.from_numpy(inp["h"]).to(dev)
            eps = float(inp["eps"])
        del inp
    ctx_len = torch.tensor([L], dtype=torch.int32, device=dev)
    scratch = {}
    h = h0.clone()
    hb = torch.empty_like(h0)
    block_bytes = (3 * d * d + d * d + 2 * F * d + d * F) * 2 + 2 * d * 2 + 2 * R * L * d * 2 + M * d * 4 * 2

    head = None
    if with_head:
        fcw = ops.bf16_from_bits(synth.normal_bf16(synth.config_seed("draft_layer"), 7001, (d, d)), dev)
        x_in = torch.from_numpy(synth.normal_f32(synth.config_seed("draft_layer"), 7002, (M, d))).to(dev)
        fnorm = ops.bf16_from_bits(synth.bf16_bits_rne(
            1.0 + synth.normal_f32(synth.config_seed("draft_layer"), 7003, (d,), 0.1)), dev)
        hid = torch.empty(M, d, device=dev)
        hinp = synth.round_inputs("qwen3_8b_head")
        V, k, r = hinp["V"], hinp["k"], hinp["r"]
        head = dict(W=ops.bf16_from_bits(hinp["W_lm"], dev), w1=ops.bf16_from_bits(hinp["w1"], dev),
                    w2=ops.bf16_from_bits(hinp["w2"], dev), prev0=torch.from_numpy(hinp["prev0"]).to(dev),
                    pw=ops.bf16_from_bits(hinp["probe_w"], dev), base=torch.empty(R, B, V, device=dev),
                    ws=ops.draft_round_workspace(R, B, k, V, d, dev), k=k)
        out_host = torch.empty(R * k * 8 + M * 8, dtype=torch.uint8, pin_memory=True)
        ids = out_host[: R * k * 8].view(torch.int64).view(R, k)
        plog = out_host[R * k * 8: R * k * 8 + M * 4].view(torch.float32)
        ppass = out_host[R * k * 8 + M * 4:].view(torch.int32)
        lm_b, mk_b, pr_b = round_bytes(hinp)
        del hinp

    def step(s_):
        if not with_head:
            blk = blocks[s_ % n_w]
            ops.draft_block_forward(h, blk["w"], R, B, H, Dh, blk["kc"], blk["vc"], ctx_len, eps, scratch=scratch,
                                    out=hb)
            return
        ops.draft_forward(x_in, fcw, [b_["w"] for b_ in blocks], [b_["kc"] for b_ in blocks],
                          [b_["vc"] for b_ in blocks], R, B, H, Dh, ctx_len, fnorm, eps, scratch=scratch, out=hid)
        ops.draft_round(head["W"], hid, head["w1"], head["w2"], head["prev0"], B, head["k"], probe_w=head["pw"],
                        base_out=head["base"], ids_out=ids, logit_out=plog, pass_out=ppass, workspace=head["ws"])

    for s_ in range(args.warmup):
        step(s_)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    a.record()
    for s_ in range(args.steps):
        step(s_)
    b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_us = a.elapsed_time(b) * 1e3 / args.steps
    n_blocks = layers if with_head else 1
    fc_bytes = (d * d * 2 + 2 * M * d * 4 + d * 2 + 2 * M * d * 4) if with_head else 0  # fc and the final norm
    step_bytes = n_blocks * block_bytes + fc_bytes + ((lm_b + mk_b + pr_b) if with_head else 0)
    gbs = step_bytes / (step_us * 1e-6) / 1e9
    name = "draft_round_8l" if with_head else "draft_block"
    log(f"[bench] {name}: {args.steps / elapsed:.1f} steps/s, {step_us:.1f} us per step, "
        f"{step_bytes / 1e9:.3f} GB algorithmic -> {gbs:.0f} GB/s")
    out = {
        "metric": ("draft rounds/s of an 8-layer drafter (fc, blocks, norm) + Qwen3-8B head round" if with_head
                   else "draft blocks/s (one full layer at M=7) + achieved HBM GB/s"),
        "value": args.steps / elapsed, "unit": "rounds/s" if with_head else "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "layers": n_blocks, "M": M, "d": d, "heads": H, "head_dim": Dh, "ffn": F,
                   "context": L},
        "roofline": {"bound": "hbm", "kernel": "whole step (its GEMVs carry 98% of the bytes)", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_step": step_bytes, "step_us": step_us},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_8b_head",
                    choices=["tiny", "qwen3_8b_head", "lane27b", "reduced_vocab_batched", "draft_layer",
                             "qwen3_8b_head_q8", "lane27b_q8", "draft_block", "draft_round_8l"])
    ap.add_argument("--layer-copies", type=int, default=4,
                    help="draft_layer: distinct weight copies cycled through (defeats the 256 MB Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle timing budget (0 disables)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one untimed device-to-device copy of this many MiB (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X and no multi-GPU "
              "path is built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from gemv_markov_argmax_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.lib()
    if args.copy_calibration_mib > 0:
        nflt = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(nflt, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.config == "draft_layer":
        return bench_layer(args, dev)
    if args.config == "draft_block":
        return bench_block(args, dev, 1, False)
    if args.config == "draft_round_8l":
        return bench_block(args, dev, 8, True)
    log(f"[bench] generating {args.config} inputs")
    inp = synth.round_inputs(args.config)
    R, B, k, d, V, r = (inp[x] for x in ("num_reqs", "B", "k", "d", "V", "r"))
    rows = R * B

    q8 = inp.get("weights") == "q8_0"
    if q8:  # Q8_0 lm_head and markov weights: (quants, scales) pairs
        W = ops.q8_from_numpy(inp["Wq_lm"], inp["Wd_lm"], dev)
        # the lm_head's scale rows padded to whole 128-byte lines, a layout
        # made once when the weights are packed (same values, same products)
        W = (W[0], ops.q8_pad_scales(W[1]))
        w1 = ops.q8_from_numpy(inp["w1q"], inp["w1d"], dev)
        w2 = ops.q8_from_numpy(inp["w2q"], inp["w2d"], dev)
    else:
        W = ops.bf16_from_bits(inp["W_lm"], dev)
        w1 = ops.bf16_from_bits(inp["w1"], dev)
        w2 = ops.bf16_from_bits(inp["w2"], dev)
    H = torch.from_numpy(inp["H"]).to(dev)
    prev0 = torch.from_numpy(inp["prev0"]).to(dev)
    pw = ops.bf16_from_bits(inp["probe_w"], dev)
    logits = torch.empty(rows, V, device=dev)
    # The round's workspace: the Markov loop's, then (more than 16 rows, bf16)
    # the split lm_head's, which starts at the next 256-byte boundary.
    ws = ops.markov_workspace(R, k, V, dev) if q8 else ops.draft_round_workspace(R, B, k, V, d, dev)
    split_at = (ops.markov_workspace_bytes(R, k, V) + 255) // 256 * 256
    split = not q8 and ops.lm_head_split_workspace_bytes(V, d, rows) > 0
    # The round's results (drafted ids, probe logits and gates) are stored by
    # the kernels straight into pinned host memory mapped for the device: no
    # copy follows the round.
    out_host = torch.empty(R * k * 8 + rows * 8, dtype=torch.uint8, pin_memory=True)
    ids = out_host[: R * k * 8].view(torch.int64).view(R, k)
    plog = out_host[R * k * 8: R * k * 8 + rows * 4].view(torch.float32)
    ppass = out_host[R * k * 8 + rows * 4:].view(torch.int32)
    bias, thr = float(inp["probe_bias"]), float(inp["probe_threshold"])
    torch.cuda.synchronize()

    def lm():  # the round's own lm_head: rows handed out by the workspace's counter word, or K split
        if q8:
            ops.lm_head_q8(*W, H, out=logits)
        elif split:
            ops.lm_head_split(W, H, ws[split_at:], out=logits)
        else:
            ops.lm_head_sched(W, H, ws, out=logits, counter_offset=ops.markov_lm_counter_offset())

    probe = dict(x=H, w=pw, bias=bias, threshold=thr, logit_out=plog, pass_out=ppass)

    def mk():  # the Markov loop with the probe in the same launch
        if q8:
            ops.markov_sample_q8(logits.view(R, B, V), *w1, *w2, prev0, k, out=ids, workspace=ws, probe=probe)
        else:
            ops.markov_sample(logits.view(R, B, V), w1, w2, prev0, k, out=ids, workspace=ws, probe=probe)

    def mk_alone():
        if q8:
            ops.markov_sample_q8(logits.view(R, B, V), *w1, *w2, prev0, k, out=ids, workspace=ws)
        else:
            ops.markov_sample(logits.view(R, B, V), w1, w2, prev0, k, out=ids, workspace=ws)

    def pr():
        ops.conf_probe(H, pw, bias, thr, logit_out=plog, pass_out=ppass)

    # A round is dspark_draft_round: the lm_head launch, then the Markov loop
    # with the probe on its idle waves, in order on one stream, the results
    # landing in host memory. In the rounds that carry HIP events around the
    # lm_head, the same two launches are issued by their own entry points
    # (dspark_lm_head_sched on the workspace's counter word,
    # dspark_lm_head_split on the workspace's split part, or
    # dspark_lm_head_q8; dspark_markov_sample_probe), so that the events can
    # sit between them.
    main_stream = torch.cuda.current_stream()

    def one_round(ev=None):
        if ev is None and q8:
            ops.draft_round_q8(*W, H, *w1, *w2, prev0, B, k, probe_w=pw, probe_bias=bias, probe_threshold=thr,
                               base_out=logits.view(R, B, V), ids_out=ids, logit_out=plog, pass_out=ppass,
                               workspace=ws)
        elif ev is None:
            ops.draft_round(W, H, w1, w2, prev0, B, k, probe_w=pw, probe_bias=bias, probe_threshold=thr,
                            base_out=logits.view(R, B, V), ids_out=ids, logit_out=plog, pass_out=ppass,
                            workspace=ws)
        else:
            ev[0].record(main_stream)
            lm()
            ev[1].record(main_stream)
            mk()
            ev[2].record(main_stream)

    log(f"[bench] warmup {args.warmup} rounds")
    for _ in range(args.warmup):
        one_round()
    torch.cuda.synchronize()

    # Timed region: K whole rounds. HIP events on the stream the kernels run
    # on bracket the lm_head launch (the kernel the roofline entry is about)
    # and the Markov launch in every EVERY-th round; a pair of event records
    # costs the round ~20 us of idle time, so only a sample of the rounds
    # carries them.
    EVERY = 10
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(0, args.steps, EVERY)]
    log(f"[bench] timing {args.steps} rounds")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_round(evs[s // EVERY] if s % EVERY == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    lm_avg = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    mk_round_avg = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    gpu_out = dict(ids=ids.numpy().copy(), logit=plog.numpy().copy(),
                   logits=logits.cpu().numpy(), base=logits.view(R, B, V).cpu().numpy())

    # Outside the timed region: each component launched back to back,
    # bracketed by one pair of events.
    def per_call_ms(fn, n=max(20, args.steps // 4), before=None):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        if before is None:
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n
        tot = 0.0
        for _ in range(n):
            before()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        return tot / n
    def per_call_graph_ms(fn, n=50, reps=5):
        """GPU time per launch of a short kernel: n launches recorded in a HIP
        graph, replayed, one pair of events around each replay (back-to-back
        launches from the host would measure the host's issue rate)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = []
        for _ in range(reps):
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            best.append(a.elapsed_time(b) / n)
        del g
        return float(np.median(best))

    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    mk_ms, mka_ms = per_call_ms(mk), per_call_ms(mk_alone)
    # The round's lm_head back to back, and (when the round splits K) the
    # one-pass kernel of dspark_lm_head on the same tensors beside it.
    lm_b2b_ms = per_call_ms(lm)
    one_pass_ms = per_call_ms(lambda: ops.lm_head(W, H, out=logits)) if split else None
    pr_ms = per_call_graph_ms(pr)
    empty_ms = per_call_graph_ms(lambda: ops.stream_read(sink, 1, 256, sink=sink, nbytes=0))

    # The Markov loop split into its prologue (markov_w2 onto the chip) and
    # steps: the same call with one step, against k steps.
    ids1 = torch.empty(R, 1, dtype=torch.int64, device=dev)

    def mk_one():
        if q8:
            ops.markov_sample_q8(logits.view(R, B, V), *w1, *w2, prev0, 1, out=ids1, workspace=ws)
        else:
            ops.markov_sample(logits.view(R, B, V), w1, w2, prev0, 1, out=ids1, workspace=ws)
    mk1_ms = per_call_ms(mk_one)
    step_us = (mka_ms - mk1_ms) * 1e3 / (k - 1) if k > 1 else None
    # Cold: a 1 GiB read with plain loads before each call evicts markov_w2
    # from L2 and from the Infinity Cache (outside the events). A
    # non-temporal read, like the lm_head's weight stream, would leave it in
    # the Infinity Cache; a pass that writes would add its write-backs.
    flush = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    mk_cold_ms = per_call_ms(mk_alone, n=20, before=lambda: flush.sum())
    del flush

    # The streaming-read ceiling of this device in this run: 4 GiB read at
    # the lm_head's launch shape (one workgroup of 1024 threads per CU, a
    # contiguous share each), at a finer shape (8192 workgroups of 256), and
    # with the scheduled lm_head's schedule (a contiguous run per workgroup,
    # the rest handed out by a counter).
    big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    cnt = ops.lm_head_counter(dev)
    ceil = {}
    for label, g, t, fn in (("lm_head_shape", cus, 1024, lambda: ops.stream_read(big, cus, 1024, sink=sink)),
                            ("fine_grid", 8192, 256, lambda: ops.stream_read(big, 8192, 256, sink=sink)),
                            ("lm_head_schedule", cus, 1024,
                             lambda: ops.stream_read_sched(big, cus, 1024, cnt, sink=sink))):
        ms = per_call_ms(fn, n=10)
        ceil[label] = dict(groups=g, threads=t, us=ms * 1e3, gbs=big.numel() / (ms * 1e-3) / 1e9)
    del big
    torch.cuda.synchronize()
    # the ceiling of the lm_head's own schedule: scheduled rows where the
    # round's lm_head takes them (bf16, rows <= 8, d <= 4096, more than 16
    # tiles of 16 rows per CU)
    sched_lm = (not q8) and rows <= 8 and inp["d"] <= 4096 and inp["V"] > 16 * 16 * cus
    ceil_ref = "lm_head_schedule" if sched_lm else "lm_head_shape"
    lm_label = ("lm_head GEMV (dspark_lm_head_q8)" if q8 else "lm_head GEMV (dspark_lm_head_split)" if split
                else "lm_head GEMV (dspark_lm_head_sched)" if sched_lm
                else "lm_head GEMV (dspark_lm_head_sched, running dspark_lm_head's kernel at this shape)")

    rounds_per_s = args.steps / elapsed
    round_us = 1e6 * elapsed / args.steps
    lm_b, mk_b, pr_b = round_bytes(inp)
    lm_gbs = lm_b / (lm_avg * 1e-3) / 1e9
    traffic = counter_traffic(args.config)
    tr_lm, tr_mk = traffic.get("lm_head"), traffic.get("markov_loop_probe")
    hbm_round = (tr_lm + tr_mk) if (tr_lm is not None and tr_mk is not None) else None
    log(f"[bench] {rounds_per_s:.1f} rounds/s; lm_head {lm_avg * 1e3:.1f} us = {lm_gbs:.0f} GB/s; "
        f"markov+probe {mk_round_avg * 1e3:.1f} us in the round ({mk_ms * 1e3:.1f} back to back; loop alone "
        f"{mka_ms * 1e3:.1f}, cold {mk_cold_ms * 1e3:.1f}, one step {mk1_ms * 1e3:.1f}); standalone probe "
        f"{pr_ms * 1e3:.1f} us, empty launch {empty_ms * 1e3:.1f} us; stream ceiling "
        + ", ".join(f"{kk} {v['gbs']:.0f} GB/s" for kk, v in ceil.items()))

    cpu, check = None, None
    if args.cpu_seconds > 0:
        log("[bench] timing the fp64 oracle on the host (and checking the GPU's round against it)")
        cpu, check = cpu_baseline(inp, args.cpu_seconds, gpu_out)

    def frac(gbs):
        return None if gbs is None else gbs / HBM_PEAK_GBS

    mk_hbm_gbs = tr_mk / (mk_round_avg * 1e-3) / 1e9 if tr_mk is not None else None
    out = {
        "metric": METRIC,
        "value": rounds_per_s,
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q8_0" if q8 else "bf16",
        "data": "synthetic",
        "config": {"workload": args.config, "num_reqs": R, "B": B, "k": k, "d": d, "V": V, "r": r,
                   "weights": "q8_0" if q8 else "bf16"},
        "roofline": {"bound": "hbm", "kernel": lm_label,
                     "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lm_gbs / HBM_PEAK_GBS,
                     "traffic": tr_lm, "algorithmic_bytes_per_launch": lm_b, "avg_launch_us": lm_avg * 1e3,
                     "frac_of_stream_ceiling": lm_gbs / ceil[ceil_ref]["gbs"], "stream_ceiling_ref": ceil_ref,
                     "back_to_back_us": lm_b2b_ms * 1e3,
                     "one_pass_back_to_back_us": one_pass_ms * 1e3 if one_pass_ms is not None else None,
                     # The same launch against the matrix cores: the bf16 MFMA
                     # work of the exact hi/lo split of the activations (2M
                     # bf16 rows of A), 2 * 2M * V * d flops, against the dense
                     # bf16 peak. Not the binding limit of any lm_head here.
                     "mfma": None if q8 else {
                         "flops_per_launch": 2 * 2 * rows * inp["V"] * inp["d"],
                         "tflops": 2 * 2 * rows * inp["V"] * inp["d"] / (lm_avg * 1e-3) / 1e12,
                         "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                         "frac": 2 * 2 * rows * inp["V"] * inp["d"] / (lm_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}},
        # Whole round. HBM bytes are the counters' (markov_w2 is read from
        # memory once per call and served on chip for every step); the
        # algorithmic figure counts markov_w2 once per step, as the method
        # does, so its rate is an equivalent, not an HBM rate.
        "round": {"us": round_us,
                  "hbm_bytes_counters": hbm_round,
                  "hbm_gbs": hbm_round / (round_us * 1e-6) / 1e9 if hbm_round else None,
                  "hbm_frac": frac(hbm_round / (round_us * 1e-6) / 1e9) if hbm_round else None,
                  "algorithmic_bytes": lm_b + mk_b + pr_b,
                  "algorithmic_equivalent_gbs": (lm_b + mk_b + pr_b) / (round_us * 1e-6) / 1e9},
        # The Markov loop (with the probe on its idle waves) is bound by the
        # latency of its k steps (on-chip compute plus a grid-wide key
        # exchange per step), not by HBM: its bandwidth fraction is reported
        # beside its prologue/step split.
        "markov_loop": {"bound": "step latency", "steps": k,
                        "us_in_round": mk_round_avg * 1e3, "us_back_to_back": mk_ms * 1e3,
                        "us_loop_alone": mka_ms * 1e3, "us_cold": mk_cold_ms * 1e3,
                        "us_one_step_call": mk1_ms * 1e3, "us_per_step": step_us,
                        "hbm_bytes_counters": tr_mk, "hbm_gbs_in_round": mk_hbm_gbs, "hbm_frac": frac(mk_hbm_gbs),
                        "algorithmic_bytes": mk_b,
                        "algorithmic_equivalent_gbs": mk_b / (mka_ms * 1e-3) / 1e9},
        # Standalone probe and empty launch: GPU time per launch inside a
        # replayed HIP graph of 50 launches.
        "probe": {"bound": "launch latency", "us_standalone": pr_ms * 1e3, "us_empty_launch": empty_ms * 1e3,
                  "us_added_to_the_loop_launch": (mk_ms - mka_ms) * 1e3, "algorithmic_bytes": pr_b,
                  "hbm_frac_standalone": frac(pr_b / (pr_ms * 1e-3) / 1e9)},
        "stream_ceiling": {"bytes": 4 << 30, **ceil},
        "oracle_check": check,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
