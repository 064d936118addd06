#!/usr/bin/env python3
"""Benchmark: one decode step of the Qwen3-8B-shaped DFLARE drafter on one GPU.

A step is the whole hot path over one batch: append the 8 newly accepted
context rows (fusion over T=9 target layers + context K/V for 7 layers),
draft a 16-token block in one pass over a 4096-token context, and verify it
greedily against synthetic target logits. Inputs are seeded and synthetic
(weights ~N(0, 0.02) in bf16, target hidden states ~N(0, 1)); they stand in
for the trained drafters and benchmark prompts the method is evaluated on.

Prints one JSON line: draft tokens/s (B*(N-1) per step), the roofline of the
dominant kernel (gate/up projection + SwiGLU, each launch timed with HIP
events on its launch stream over a second run of the same steps, since a
timed launch idles the stream for a few microseconds), the whole step
against the HBM roofline, and the oracle's CPU throughput on a bounded
sample.

`--workload qwen3_8b_batched` (32 sequences, ragged contexts from 512 to
8192, ragged appends, temperature-1 verify), `--workload gpt_oss_20b`
(8 sequences at context 8192, greedy) and the Qwen3-4B shapes time their
steps the same way; their `roofline` is whichever of the block attention,
the gate/up projection and the LM head has the largest roofline time per
step (the attention for the 32-sequence batch, the LM head for GPT-OSS and
Qwen3-4B), and the step is set against a roofline that adds, per phase, the
larger of the HBM time and the dense-bf16 MFMA time.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
WORKLOAD = "qwen3_8b"
METRIC = "draft tokens/sec per GPU (block=16, Qwen3-8B-shape drafter+verify); % roofline"


def step_bytes(cfg, L, n_new):
    """Algorithmic HBM bytes of one step (bf16 weights, KV, logits)."""
    D, H, I, V, T, N = (cfg[k] for k in ("n_layers", "hidden", "intermediate", "vocab", "n_target_layers",
                                         "block_size"))
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    append = n_new * T * H * 2 + (D * 2 * kvd * H * 2) + D * n_new * 2 * kvd * 2
    layer_w = (qd * H + 2 * kvd * H + H * qd + 2 * I * H + H * I) * 2
    draft = D * layer_w + V * H * 2 + N * H * 2 + D * L * 2 * kvd * 2
    verify = N * V * 2
    return dict(append=append, draft=draft, verify=verify, total=append + draft + verify)


def gate_up_bytes(cfg, M):
    """Gate and up weights (bf16) + the normed input rows and the SwiGLU
    output rows (fp32-accurate activations: 4 bytes per value)."""
    H, I = cfg["hidden"], cfg["intermediate"]
    return 2 * I * H * 2 + M * H * 4 + M * I * 4


def traffic_from_profile(name="gate_up_qwen3_8b", kernel="gate_up"):
    """HBM bytes per launch of a kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary profiles/<name>_traffic.json, if it was
    taken on the kernel's current sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    sys.path.insert(0, ROOT)
    from profiling import KERNEL_SOURCES, source_hash
    d = json.load(open(p))
    if d.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return d.get("bytes_per_launch")


def host_info():
    """The host the oracle is timed on: CPU model, CPUs, BLAS pool size."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = 1
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas_threads": int(blas)}


def cpu_baseline(cfg, w, hidden_pre, hidden_step, anchor, logits_bits, min_seconds=10.0, max_steps=8):
    """The oracle, as it stands, on a bounded sample: the same decode step
    (append 8 rows, draft, verify) repeated after an untimed prefill until
    `min_seconds` of CPU work (at most `max_steps` steps), the cache set
    back to its pre-step state between steps outside the timed region.
    The oracle computes in float64 numpy (stricter than fp32); `cores` is
    the BLAS pool's thread count, the threads its matrix products use."""
    import oracle as O
    info = host_info()
    model = O.OracleModel(cfg, w)
    cache = O.OracleCache(cfg["n_layers"])
    for r0 in range(0, len(hidden_pre), 1024):  # untimed prefill, in row chunks
        O.ctx_append(model, cache, 0, O.bf16_bits_to_f64(hidden_pre[r0: r0 + 1024]))
    saved = ([dict(k) for k in cache.k], [dict(v) for v in cache.v], dict(cache.ctx_len))  # the append rebinds
    dt, steps = 0.0, 0
    while steps < max_steps and (steps == 0 or dt < min_seconds):
        cache.k, cache.v = [dict(k) for k in saved[0]], [dict(v) for v in saved[1]]
        cache.ctx_len = dict(saved[2])
        t0 = time.perf_counter()
        O.ctx_append(model, cache, 0, O.bf16_bits_to_f64(hidden_step))
        out = O.draft_block(model, cache, 0, int(anchor))
        O.verify_greedy(out["draft"], O.bf16_bits_to_f64(logits_bits))
        dt += time.perf_counter() - t0
        steps += 1
    return {"value": (cfg["block_size"] - 1) * steps / dt, "unit": "draft tokens/s", "cores": info["blas_threads"],
            "kind": "oracle",
            "sample": f"{steps} repeats of one decode step of the same workload (append 8 rows, draft a "
                      f"16-block over a {len(hidden_pre) + len(hidden_step)}-token context, greedy verify) "
                      "after an untimed prefill; float64 numpy",
            "precision": "float64", "seconds": dt, **info}


def accept_model(dr, cfg, seq, draft, seed, draws, temperature=0.0):
    """Accept lengths of the timed step's draft under the synthetic
    agreement model, over `draws` independent logits draws (one verify
    call each, outside the timed region): mean accepted draft tokens and
    mean committed tokens (accepted + the correction or bonus token)."""
    import torch
    from block_diffusion_drafter_softmax_amd import synth
    dev = draft.device
    d_host = draft.cpu().numpy()
    Bn = d_host.shape[0]
    acc = torch.zeros(Bn, dtype=torch.int32, device=dev)
    nxt = torch.zeros_like(acc)
    com = torch.zeros_like(acc)
    a_sum = c_sum = 0
    for s in range(draws):
        bits = synth.make_logits(cfg, d_host, seed, step=1000 + s)
        z = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16) if bits.dtype == np.uint16 \
            else torch.from_numpy(bits).to(dev)
        dr.verify(seq, draft, z, acc, nxt, com, temperature=temperature, seed=1, step=1000 + s)
        torch.cuda.synchronize()
        a_sum += int(acc.sum())
        c_sum += int(com.sum())
    return a_sum / (draws * Bn), c_sum / (draws * Bn)


def agreement_expectation(p, n_draft):
    """E[accepted] under the agreement model: leading successes of n_draft
    Bernoulli(p) trials, sum_{k=1..n} p^k."""
    return sum(p ** k for k in range(1, n_draft + 1))


MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def batched_roofline(cfg, ctx, n_new, K=0):
    """Per-phase algorithmic bytes and flops of one batched step, and
    t_roof = sum over phases of max(bytes / 8 TB/s, flops / 2.5 PF).
    K > 0 adds the dual-pass drafter's second pass (B*K blocks of N against
    each sequence's shared context: the context counts once per sequence,
    the weights once more) and the verification of K+1 candidates."""
    D, H, I, V, T, N = (cfg[k] for k in ("n_layers", "hidden", "intermediate", "vocab", "n_target_layers",
                                         "block_size"))
    d, nq, nkv = cfg["head_dim"], cfg["n_q_heads"], cfg["n_kv_heads"]
    qd, kvd = nq * d, nkv * d
    B = len(ctx)
    M, rows = B * N, int(np.sum(n_new))
    layer_w = qd * H + 2 * kvd * H + H * qd + 2 * I * H + H * I
    wt = 0 if cfg.get("tied_kv") else D * 2 * kvd * H
    wfc = T * H * H if cfg.get("fusion") == "fc" else 0  # DFlash's FC fusion layer
    gemm_bytes = (D * layer_w + V * H + wt + wfc) * 2
    gemm_flops = 2.0 * M * (D * layer_w + V * H) + 2.0 * rows * (D * 2 * kvd * H + wfc)
    keys = int(np.sum(ctx)) + B * N
    attn_bytes = D * keys * 2 * kvd * 2
    attn_flops = 4.0 * D * nq * N * keys * d
    rest_bytes = rows * T * H * 2 + D * rows * 2 * kvd * 2 + M * V * 2
    phases = {"gemm": (gemm_bytes, gemm_flops), "attention": (attn_bytes, attn_flops), "rest": (rest_bytes, 0.0)}
    if K:
        M2 = B * K * N
        phases["gemm_pass2"] = ((D * layer_w + V * H) * 2, 2.0 * M2 * (D * layer_w + V * H))
        phases["attention_pass2"] = (D * (int(np.sum(ctx)) + B * K * N) * 2 * kvd * 2,
                                     4.0 * D * nq * K * N * (int(np.sum(ctx)) + B * N) * d)
        phases["verify_candidates"] = (B * (K + 1) * N * V * 2 - M * V * 2, 0.0)
    t = {k: max(b / (HBM_PEAK_GBS * 1e9), f / (MFMA_PEAK_TFS * 1e12)) for k, (b, f) in phases.items()}
    return {"phases": {k: {"bytes": int(b), "flops": f, "t_us": round(t[k] * 1e6, 1)} for k, (b, f) in phases.items()},
            "t_roof_us": round(sum(t.values()) * 1e6, 1), "attn_bytes_per_layer": attn_bytes // D}


def dominant_kernel(cfg, ctx):
    """Among the first pass's block attention, gate/up projection (one
    launch each per layer) and LM head, the one with the largest roofline
    time per step: max(bytes / 8 TB/s, flops / 2.5 PF) times its units per
    step (a layer, or the whole LM head). Algorithmic bytes: the weights or
    the context K/V once, activations in (split, 4 bytes a value) and
    out; flops: the method's 2 per multiply-add (not the split
    activation's second product)."""
    from block_diffusion_drafter_softmax_amd import _binding as B
    D, H, I, V, N = (cfg[k] for k in ("n_layers", "hidden", "intermediate", "vocab", "block_size"))
    d, nq, nkv = cfg["head_dim"], cfg["n_q_heads"], cfg["n_kv_heads"]
    Bn = len(ctx)
    M, keys = Bn * N, int(np.sum(ctx))  # the chunk kernel takes the context keys (the merge the block's)
    cands = {
        "attention": ("block attention over the context K/V (one layer)", B.K_ATTN, D,
                      keys * 2 * nkv * d * 2 + M * nq * d * 4, 4.0 * nq * N * keys * d),
        "gate_up": ("gate/up projection + SwiGLU (one layer)", B.K_GATE_UP, D,
                    2 * I * H * 2 + M * H * 4 + M * I * 4, 2.0 * M * 2 * I * H),
        "lm_head": ("LM head + per-tile top-2 (draft rows)", B.K_LM_HEAD, 1,
                    V * H * 2 + Bn * (N - 1) * H * 4, 2.0 * Bn * (N - 1) * V * H),
    }

    def t_unit(c):
        return max(c[3] / (HBM_PEAK_GBS * 1e9), c[4] / (MFMA_PEAK_TFS * 1e12))

    key = max(cands, key=lambda k: cands[k][2] * t_unit(cands[k]))
    label, kind, units, nbytes, flops = cands[key]
    bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_PEAK_TFS * 1e12) else "mfma"
    return {"name": key, "label": label, "kind": kind, "units": units, "bytes": nbytes, "flops": flops,
            "bound": bound}


def run_batched(args, name):
    """A batched workload: prefill (device-generated hidden states; their
    values do not change the work), then timed steps as in the default
    workload, then the dominant kernel's launches timed in a second pass."""
    import torch
    from block_diffusion_drafter_softmax_amd import synth
    from block_diffusion_drafter_softmax_amd import _binding as B
    from block_diffusion_drafter_softmax_amd.drafter import Drafter

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = synth.config(name)
    Bn, N, T, H, V = cfg["batch"], cfg["block_size"], cfg["n_target_layers"], cfg["hidden"], cfg["vocab"]
    ctx = synth.context_lengths(cfg, 0)
    n_new = synth.appended_rows(cfg, 0)
    temp = 1.0 if cfg["verify"] == "temp1" else 0.0
    dev = torch.device("cuda")
    K = int(cfg.get("d2sd_k", 0))
    w = synth.make_weights(cfg, 0)
    chunk = 512
    dr = Drafter(cfg, w, max_batch=Bn * (K + 1), max_new=chunk, max_seqs=Bn,
                 pages_per_seq=(int(ctx.max()) + N + 15) // 16 + 1, page_order="shuffled")
    seq = torch.arange(Bn, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    hid = torch.randn((Bn, chunk, T, H), generator=gen, device=dev).to(torch.bfloat16)
    pre, done = ctx - n_new, np.zeros(Bn, dtype=np.int64)
    while (done < pre).any():
        n = np.minimum(pre - done, chunk).astype(np.int32)
        dr.ctx_append(seq, torch.from_numpy(n).to(dev), hid, chunk)
        done += n
    del hid
    torch.cuda.synchronize()
    assert dr.read_error() == 0
    log(f"prefill done: {Bn} sequences, contexts {ctx.min()}..{ctx.max()}, appends {int(n_new.sum())} rows")

    max_new = int(n_new.max())
    step_hid = torch.randn((Bn, max_new, T, H), generator=gen, device=dev).to(torch.bfloat16)
    n_new_t = torch.from_numpy(n_new.astype(np.int32)).to(dev)
    anchor = torch.from_numpy(synth.make_anchor(cfg, Bn, 0)).to(dev)
    draft = torch.zeros((Bn, N - 1), dtype=torch.int32, device=dev)
    acc = torch.zeros(Bn, dtype=torch.int32, device=dev)
    nxt = torch.zeros(Bn, dtype=torch.int32, device=dev)
    com = torch.zeros(Bn, dtype=torch.int32, device=dev)
    ctx0 = dr.ctx_len.clone()
    dr.ctx_append(seq, n_new_t, step_hid, max_new)
    dr.draft_block(seq, anchor, draft)
    torch.cuda.synchronize()
    logits_bits = synth.make_logits(cfg, draft.cpu().numpy(), 0)
    logits = torch.from_numpy(logits_bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def step_first():
        dr.ctx_len.copy_(ctx0)
        if args.separate_append:
            dr.ctx_append(seq, n_new_t, step_hid, max_new)
            dr.draft_block(seq, anchor, draft)
        else:
            dr.append_draft(seq, n_new_t, step_hid, anchor, draft, max_new=max_new)
        dr.verify(seq, draft, logits, acc, nxt, com, temperature=temp, seed=1, step=0)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        assert dr.read_error() == 0
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    step, first_ms = step_first, None
    if K:
        # dual-pass step: first draft, K lowest-confidence cut points, one
        # batched second pass, greedy verification of all K+1 candidates
        # (target logits built around the GPU's own candidates)
        C = K + 1
        drafts = torch.zeros((Bn, C, N - 1), dtype=torch.int32, device=dev)
        chosen = torch.zeros(Bn, dtype=torch.int32, device=dev)
        dr.ctx_len.copy_(ctx0)
        dr.ctx_append(seq, n_new_t, step_hid, max_new)
        dr.d2sd_draft(seq, anchor, K, drafts)
        torch.cuda.synchronize()
        z = synth.make_logits(cfg, drafts.cpu().numpy().reshape(Bn * C, N - 1), 0)
        logits_c = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16).view(Bn, C, N, V)
        del z
        first_ms = timed(step_first)

        def step():
            dr.ctx_len.copy_(ctx0)
            dr.ctx_append(seq, n_new_t, step_hid, max_new)
            dr.d2sd_draft(seq, anchor, K, drafts)
            dr.verify_multi(seq, drafts, logits_c, acc, nxt, com, chosen)

    ms_step = timed(step)
    acc_main, com_main = acc.clone(), com.clone()  # the timed step's outcome (the timer pass below reruns pass one)

    dk = dominant_kernel(cfg, ctx)
    B.check(B.dflash_kernel_timer(dr.handle, dk["kind"], 1), "timer")
    for _ in range(args.steps):
        step_first()  # the first pass's launches of the dominant kernel: the units below
    torch.cuda.synchronize()
    rc, k_ms, k_n = B.dflash_kernel_timer_read(dr.handle, dk["kind"])
    B.check(rc, "timer read")
    B.dflash_kernel_timer(dr.handle, dk["kind"], 0)
    assert dr.read_error() == 0

    rl = batched_roofline(cfg, ctx, n_new, K)
    rl1 = batched_roofline(cfg, ctx, n_new) if K else rl
    unit_s = k_ms / (args.steps * dk["units"]) / 1e3  # all launches of the kind per unit (a k split adds one)
    if dk["bound"] == "hbm":
        achieved, peak, unit = dk["bytes"] / unit_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = dk["flops"] / unit_s / 1e12, MFMA_PEAK_TFS, "TFLOP/s"
    accepted = float(acc_main.float().mean())
    committed = float(com_main.float().sum())
    accept_src = f"the timed step's verification over its {Bn} sequences (one agreement-model draw each)"
    if not K:  # more agreement-model draws around the timed draft: at least --accept-draws sequence samples
        n_draws = -(-args.accept_draws // Bn)
        ma, mc = accept_model(dr, cfg, seq, draft, 0, n_draws, temperature=temp)
        accepted, committed = ma, mc * Bn
        accept_src = (f"{'temperature-1' if temp else 'greedy'} verify of the timed draft ({Bn} sequences) "
                      f"against {n_draws} draws of the synthetic agreement model (p = {cfg['agreement']})")
    res = {
        "metric": "draft tokens/sec per GPU (block=16, batched drafter+verify); % roofline",
        "value": round(Bn * (N - 1) / (ms_step / 1e3), 1), "unit": "draft tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {Bn} sequences x block {N}, contexts {int(ctx.min())}..{int(ctx.max())} "
                               f"(sum {int(ctx.sum())}), {int(n_new.sum())} rows appended, "
                               f"{'temperature-1' if temp else 'greedy'} verify"
                               f"{f' of {K + 1} dual-pass candidates (K={K} cut points, one batched second pass)' if K else ''}"
                               f"; D {cfg['n_layers']}, H {H}, "
                               f"{cfg['n_q_heads']}/{cfg['n_kv_heads']} heads of {cfg['head_dim']}, "
                               f"I {cfg['intermediate']}, V {V}",
                   "global_batch": Bn, "block": N, "launch": "eager"},
        "roofline": {"bound": dk["bound"], "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic_from_profile(f"{dk['name']}_{name}", dk["name"]),
                     "kernel": dk["label"],
                     "bytes_per_unit": int(dk["bytes"]), "flops_per_unit": dk["flops"],
                     "us_per_unit": round(unit_s * 1e6, 2), "launches_timed": k_n},
        "step_roofline": {"bound": "mixed", "t_roof_us": rl["t_roof_us"], "phases": rl["phases"],
                          "frac": round(rl["t_roof_us"] / (ms_step * 1e3), 4)},
        "mean_accept": round(accepted, 3),
        "committed_tok_s": round(committed / (ms_step / 1e3), 1),
        "accept_source": accept_src,
        "first_pass_only": None if not K else {
            "ms_per_step": round(first_ms, 4), "draft_tok_s": round(Bn * (N - 1) / (first_ms / 1e3), 1),
            "t_roof_us": rl1["t_roof_us"], "frac": round(rl1["t_roof_us"] / (first_ms * 1e3), 4)},
        "cpu_baseline": None,
    }
    log(f"{ms_step:.3f} ms/step, {res['value']:.0f} draft tok/s, step roofline {res['step_roofline']['frac']:.3f}")
    print(json.dumps(res), flush=True)


def run_rollout(args):
    """S decode steps of the Qwen3-8B-shaped workload captured as one graph:
    each step appends the previous step's committed rows and drafts from its
    next token (device-resident, no host round trip); synthetic target
    logits by the agreement model (p = 0.8) are built on the device around
    each step's draft. Timed over replays of the whole graph."""
    import torch
    from block_diffusion_drafter_softmax_amd import synth
    from block_diffusion_drafter_softmax_amd.drafter import Drafter
    from block_diffusion_drafter_softmax_amd.rollout import Rollout

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = synth.config(WORKLOAD)
    S = args.rollout
    N, L, n_new, T, H, V = (cfg[k] for k in ("block_size", "context", "n_new", "n_target_layers", "hidden", "vocab"))
    dev = torch.device("cuda")
    w = synth.make_weights(cfg, 0)
    chunk = 512
    dr = Drafter(cfg, w, max_batch=1, max_new=chunk, max_seqs=1, pages_per_seq=(L + S * N + N + 15) // 16 + 1)
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    hid = torch.randn((1, chunk, T, H), generator=gen, device=dev).to(torch.bfloat16)
    done = 0
    while done < L - n_new:
        n = min(chunk, L - n_new - done)
        dr.ctx_append(seq, torch.tensor([n], dtype=torch.int32, device=dev), hid, chunk)
        done += n
    del hid
    # per-step target stand-in: hidden rows, noise logits, agreement coins
    hidden = torch.randn((S, 1, N, T, H), generator=gen, device=dev).to(torch.bfloat16)
    noise = torch.randn((S, 1, N, V), generator=gen, device=dev).to(torch.bfloat16)
    top1 = (noise[:, :, : N - 1].float().amax(-1) + 1.0).to(torch.bfloat16)
    agree = torch.rand((S, 1, N - 1), generator=gen, device=dev) < cfg["agreement"]
    anchor = torch.from_numpy(synth.make_anchor(cfg, 1, 0)).to(dev)
    rl = Rollout(dr, seq, anchor, torch.tensor([n_new], dtype=torch.int32, device=dev), hidden, noise, agree, top1)
    rl.run()
    torch.cuda.synchronize()
    assert dr.read_error() == 0
    graph = rl.capture()
    reps = max(1, args.steps // S)
    for _ in range(max(1, args.warmup // S)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert dr.read_error() == 0
    com = rl.commit.cpu().numpy()[:, 0]
    acc = rl.accept.cpu().numpy()[:, 0]
    ms_step = elapsed * 1e3 / (reps * S)
    ctx_steps = L + np.concatenate([[0], np.cumsum(com[:-1])])  # context of each step (after its append)
    appended = np.concatenate([[n_new], com[:-1]])
    t_roof = float(np.mean([step_bytes(cfg, int(c), int(a))["total"] for c, a in zip(ctx_steps, appended)])) \
        / (HBM_PEAK_GBS * 1e9) * 1e6
    res = {
        "metric": METRIC, "value": round((N - 1) / (ms_step / 1e3), 1), "unit": "draft tokens/s", "n_gpus": 1,
        "steps": reps * S, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Qwen3-8B-shaped roll-out: {S} device-resident decode steps in one graph "
                               f"(append the previous commit, draft, target stand-in, greedy verify), context "
                               f"{int(ctx_steps[0])}..{int(ctx_steps[-1])}",
                   "global_batch": 1, "block": N, "launch": "graph", "rollout_steps": S},
        "committed_tok_s": round(float(com.sum()) / (ms_step * S / 1e3), 1),
        "mean_accept": round(float(acc.mean()), 3),
        "step_roofline": {"bound": "hbm", "t_roof_us": round(t_roof, 1), "frac": round(t_roof / (ms_step * 1e3), 4)},
        "roofline": None, "cpu_baseline": None,
    }
    log(f"roll-out: {ms_step:.3f} ms/step over {S} steps, {res['value']:.0f} draft tok/s, "
        f"{res['committed_tok_s']:.0f} committed tok/s, mean accept {res['mean_accept']}")
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--accept-draws", type=int, default=32,
                    help="logits draws of the agreement model behind mean_accept / committed_tok_s")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--separate-append", action="store_true",
                    help="append and draft as two calls (dflash_ctx_append, dflash_draft_block) instead of "
                         "dflash_append_draft")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "qwen3_8b_batched", "gpt_oss_20b", "qwen3_4b", "qwen3_4b_fc"])
    ap.add_argument("--sampled", type=float, default=0.0,
                    help="tau > 0: drafts sampled at temperature tau, lossless verification at temperature 1")
    ap.add_argument("--context", type=int, default=0,
                    help="L > 0: the default workload at context length L instead of 4096 (a sweep, not the headline)")
    ap.add_argument("--rollout", type=int, default=0,
                    help="S > 0: S device-resident steps of the default workload captured as one graph")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the drafter's hot path runs on a single MI355X here; "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.rollout > 0:
        return run_rollout(args)
    if args.workload != WORKLOAD:
        return run_batched(args, args.workload)

    import torch
    from block_diffusion_drafter_softmax_amd import synth
    from block_diffusion_drafter_softmax_amd import _binding as B
    from block_diffusion_drafter_softmax_amd.drafter import Drafter

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = synth.config(WORKLOAD)
    if args.context:
        if args.context < cfg["n_new"]:
            raise SystemExit("--context must be at least the 8 appended rows")
        cfg["context"] = args.context
    N, L, n_new, T, H = cfg["block_size"], cfg["context"], cfg["n_new"], cfg["n_target_layers"], cfg["hidden"]
    seed = 0
    t0 = time.perf_counter()
    w = synth.make_weights(cfg, seed)
    hidden_pre = synth.make_hidden(cfg, L - n_new, seed, "pre/0")
    hidden_step = synth.make_hidden(cfg, n_new, seed, "step/0")
    anchor = synth.make_anchor(cfg, 1, seed)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")

    dev = torch.device("cuda")
    chunk = 512
    dr = Drafter(cfg, w, max_batch=1, max_new=chunk, max_seqs=1, pages_per_seq=(L + N + 15) // 16 + 1)
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    for r0 in range(0, L - n_new, chunk):
        rows = hidden_pre[r0: r0 + chunk]
        buf = np.zeros((1, chunk, T, H), dtype=np.uint16)
        buf[0, : len(rows)] = rows
        hid = torch.from_numpy(buf.view(np.int16)).to(dev).view(torch.bfloat16)
        dr.ctx_append(seq, torch.tensor([len(rows)], dtype=torch.int32, device=dev), hid, chunk)
    torch.cuda.synchronize()
    assert int(dr.ctx_len[0]) == L - n_new
    log("prefill done")

    ctx0 = dr.ctx_len.clone()
    step_hidden = torch.from_numpy(hidden_step.reshape(1, n_new, T, H).view(np.int16)).to(dev).view(torch.bfloat16)
    n_new_t = torch.tensor([n_new], dtype=torch.int32, device=dev)
    anchor_t = torch.from_numpy(anchor).to(dev)
    draft = torch.zeros((1, N - 1), dtype=torch.int32, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    com = torch.zeros(1, dtype=torch.int32, device=dev)

    # target logits built around the GPU's own draft (timing input only)
    dr.ctx_append(seq, n_new_t, step_hidden, n_new)
    dr.draft_block(seq, anchor_t, draft)
    torch.cuda.synchronize()
    logits_bits = synth.make_logits(cfg, draft.cpu().numpy(), seed)[0]
    logits = torch.from_numpy(logits_bits.view(np.int16)).to(dev).view(torch.bfloat16).unsqueeze(0)
    dr.ctx_len.copy_(ctx0)

    # The same workload every step: the context goes back to L - 8 before the
    # append. A fill kernel, not a copy: a copy is a memcpy node in a graph
    # capture, which the runtime may run on a copy engine and synchronise
    # with the kernels around it.
    def rewind():
        dr.ctx_len.fill_(L - n_new)

    def step():
        rewind()
        if args.separate_append:
            dr.ctx_append(seq, n_new_t, step_hidden, n_new)
            dr.draft_block(seq, anchor_t, draft)
        else:  # the same two calls as one (fewer launches, the same results)
            dr.append_draft(seq, n_new_t, step_hidden, anchor_t, draft, max_new=n_new)
        dr.verify(seq, draft, logits, acc, nxt, com)

    tau = args.sampled
    if tau > 0:  # sampled drafts; the drafter's logits go to HBM for the verification
        draft_logits = torch.zeros((1, N - 1, cfg["vocab"]), dtype=torch.float32, device=dev)

        def step():
            rewind()
            dr.ctx_append(seq, n_new_t, step_hidden, n_new)
            dr.draft_sample(seq, anchor_t, tau, draft, draft_logits, seed=1, step=0)
            dr.verify_sample(seq, draft, draft_logits, tau, logits, acc, nxt, com, seed=1, step=0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert dr.read_error() == 0

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    # The dominant kernel's launch duration, from HIP events, over a second
    # run of the same eager steps: a timed launch costs the stream a few
    # microseconds of idle time, so the steps above run without the timer.
    B.check(B.dflash_kernel_timer(dr.handle, B.K_GATE_UP, 1), "timer")
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rc, gu_ms, gu_n = B.dflash_kernel_timer_read(dr.handle, B.K_GATE_UP)
    B.check(rc, "timer read")
    B.dflash_kernel_timer(dr.handle, B.K_GATE_UP, 0)
    assert dr.read_error() == 0

    ms_step = elapsed * 1e3 / args.steps
    tok_s = (N - 1) / (ms_step / 1e3)
    sb = step_bytes(cfg, L, n_new)
    if tau > 0:  # the drafter's fp32 logits, written once and read by the verification
        sb["total"] += 2 * (N - 1) * cfg["vocab"] * 4
    M = N
    roof = None
    if gu_n:
        gu_avg_s = gu_ms / gu_n / 1e3
        gbytes = gate_up_bytes(cfg, M)
        achieved = gbytes / gu_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(),
                "kernel": "gate_up (gate/up projection + SwiGLU)", "bytes_per_launch": gbytes,
                "avg_launch_us": round(gu_avg_s * 1e6, 2), "launches_timed": gu_n}
    t_roof_us = sb["total"] / (HBM_PEAK_GBS * 1e9) * 1e6
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "draft tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped DFLARE drafter decode step: append 8 context rows "
                               f"(T=9 fusion), draft block 16 over ctx {L} (7 layers, H 4096, 32/8 heads, "
                               "I 12288, V 151936), "
                               + (f"drafts sampled at temperature {tau}, lossless temperature-1 verify"
                                  if tau > 0 else "greedy verify") + "; batch 1",
                   "global_batch": 1, "seq_len": L, "block": N, "launch": "graph" if graph else "eager",
                   "calls": ("dflash_ctx_append + dflash_draft_block" if args.separate_append
                             else "dflash_append_draft") + " + dflash_verify"},
        "roofline": roof,
        "step_roofline": {"bound": "hbm", "bytes": sb["total"], "t_roof_us": round(t_roof_us, 1),
                          "achieved_GBs": round(sb["total"] / (ms_step / 1e3) / 1e9, 1),
                          "frac": round(t_roof_us / (ms_step * 1e3), 4)},
    }
    if tau <= 0:
        ma, mc = accept_model(dr, cfg, seq, draft, seed, args.accept_draws)
        res["mean_accept"] = round(ma, 3)
        res["committed_tok_s"] = round(mc / (ms_step / 1e3), 1)
        res["accept_source"] = (f"greedy verify of the timed draft against {args.accept_draws} draws of the "
                                f"synthetic agreement model (p = {cfg['agreement']}; expectation "
                                f"{agreement_expectation(cfg['agreement'], N - 1):.2f} accepted)")
    else:
        res["mean_accept"] = int(acc[0])
        res["committed_tok_s"] = round(int(com[0]) / (ms_step / 1e3), 1)
        res["accept_source"] = "the timed step's own verification (one draw of the agreement model)"
    log(f"{ms_step:.3f} ms/step, {tok_s:.0f} draft tok/s, step roofline {res['step_roofline']['frac']:.3f}")
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (one step)")
        del graph
        res["cpu_baseline"] = cpu_baseline(cfg, w, hidden_pre, hidden_step, anchor[0], logits_bits)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
