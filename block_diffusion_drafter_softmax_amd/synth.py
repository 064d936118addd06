"""Seeded synthetic workloads: drafter shapes and input generators.

Harness code shared by the HIP path's tests/bench and by the oracle's
callers. It holds no arithmetic of the method: it only draws numbers
(weights, target hidden states, anchors, context lengths, target logits)
and rounds them once to bfloat16.

The drafter shapes are those the pages name (Qwen3-4B, Qwen3-8B and
GPT-OSS-20B targets with DFlash/DFLARE drafters; DFLARE summary, section 4
and section 3 for depth 7 and T = 9), plus a tiny CPU-seconds shape. The
pages evaluate on public benchmarks (GSM8K, MATH-500, AIME25, HumanEval,
MBPP, MT-Bench) with trained drafters; none of that is used here: these
seeded inputs stand in for them by shape, context length and acceptance
behaviour only.

Every tensor gets its own numpy PCG64 stream keyed by (seed, tensor name,
chunk index), so results do not depend on thread count or call order.
"""
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_BASE = dict(rope_theta=1e6, rms_eps=1e-6, use_rope=1, page_size=16)

CONFIGS = {
    # CPU-seconds shape; logits fp32 with the draft token boosted by +3 w.p. 0.7
    "tiny": dict(_BASE, hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 intermediate=704, vocab=4096, n_target_layers=3, block_size=8, tied_kv=0,
                 context=128, batch=1, n_new=8, verify="greedy", logits_dtype="f32",
                 agreement=0.7, logit_model="boost3"),
    # Qwen3-4B-shaped drafter, DFlash style: T=5, one K/V projection for context and block
    "qwen3_4b": dict(_BASE, hidden=2560, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     intermediate=9728, vocab=151936, n_target_layers=5, block_size=16, tied_kv=1,
                     context=2048, batch=1, n_new=8, verify="greedy", logits_dtype="bf16",
                     agreement=0.8, logit_model="top_plus1"),
    # the same shape with DFlash's own conditioning: one FC layer fuses the
    # T states into a single context shared by all layers
    "qwen3_4b_fc": dict(_BASE, hidden=2560, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        intermediate=9728, vocab=151936, n_target_layers=5, block_size=16, tied_kv=1,
                        context=2048, batch=1, n_new=8, verify="greedy", logits_dtype="bf16",
                        agreement=0.8, logit_model="top_plus1", fusion="fc"),
    # Qwen3-8B-shaped drafter with DFLARE fusion over T=9 and separate W^t / W^d
    "qwen3_8b": dict(_BASE, hidden=4096, n_layers=7, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     intermediate=12288, vocab=151936, n_target_layers=9, block_size=16, tied_kv=0,
                     context=4096, batch=1, n_new=8, verify="greedy", logits_dtype="bf16",
                     agreement=0.8, logit_model="top_plus1"),
    # batched serving at the Qwen3-8B shape: 32 ragged contexts, temperature-1 verify
    "qwen3_8b_batched": dict(_BASE, hidden=4096, n_layers=7, n_q_heads=32, n_kv_heads=8, head_dim=128,
                             intermediate=12288, vocab=151936, n_target_layers=9, block_size=16,
                             tied_kv=0, context=(512, 8192), batch=32, n_new=16, verify="temp1",
                             logits_dtype="bf16", agreement=0.75, logit_model="accept_p"),
    # GPT-OSS-20B-shaped drafter, batch 8, context 8192, with the dual-pass
    # drafter's second pass over K = 4 cut points and multi-candidate verify
    "gpt_oss_20b": dict(_BASE, hidden=2880, n_layers=5, n_q_heads=64, n_kv_heads=8, head_dim=64,
                        intermediate=2880, vocab=201088, n_target_layers=9, block_size=16, tied_kv=0,
                        context=8192, batch=8, n_new=8, verify="greedy", logits_dtype="bf16",
                        agreement=0.8, logit_model="top_plus1", d2sd_k=4),
}


def config(name, **overrides):
    c = dict(CONFIGS[name])
    c["name"] = name
    c["mask_token_id"] = c["vocab"] - 1
    c.update(overrides)
    return c


def _rng(seed, name, chunk=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode()), chunk])))


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 24
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import os
        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def normal_bf16(shape, std, seed, name):
    """N(0, std^2) draws rounded to bf16 bits, generated in fixed chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def work(ci):
        lo, hi = ci * _CHUNK, min(n, (ci + 1) * _CHUNK)
        x = _rng(seed, name, ci).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)

    list(_pool().map(work, range((n + _CHUNK - 1) // _CHUNK)))
    return out.reshape(shape)


def make_weights(cfg, seed=0, std=0.02):
    """Drafter weights as bf16 bits (nn.Linear layout, stacked over layers).

    Linear and embedding weights ~N(0, std^2); norm gains 1.0; W_fuse
    ~N(0, 1) in float32. With tied_kv the context projections are omitted.

    ``cfg["qk_score_var"]`` (optional, parity inputs only) draws the query
    and key projections (wq, wk_d, wk_t) with std sqrt(v / H) instead, so
    that the attention logits q.k / sqrt(d_h) of unit-RMS rows have variance
    about v whatever the width. At small widths std 0.02 makes the scores
    nearly zero: the attention is uniform, every mask position of a block
    then carries the same state and the whole block drafts one token. With
    v ~ 2.5 (what std 0.02 gives at H = 4096) the RoPE positions separate
    the rows and the drafted tokens differ from position to position.
    """
    D, H, I, V, T = cfg["n_layers"], cfg["hidden"], cfg["intermediate"], cfg["vocab"], cfg["n_target_layers"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    shapes = dict(wq=(D, qd, H), wk_d=(D, kd, H), wv_d=(D, kd, H), wo=(D, H, qd),
                  wg=(D, I, H), wu=(D, I, H), wd=(D, H, I), embed=(V, H), lm_head=(V, H))
    if not cfg.get("tied_kv"):
        shapes.update(wk_t=(D, kd, H), wv_t=(D, kd, H))
    qk_std = float(np.sqrt(cfg["qk_score_var"] / H)) if cfg.get("qk_score_var") else std
    w = {k: normal_bf16(s, qk_std if k in ("wq", "wk_d", "wk_t") else std, seed, k) for k, s in shapes.items()}
    one = np.uint16(0x3F80)
    for k, s in dict(g_fuse=(D, H), g_attn=(D, H), g_mlp=(D, H), g_final=(H,)).items():
        w[k] = np.full(s, one, dtype=np.uint16)
    w["w_fuse"] = _rng(seed, "w_fuse").standard_normal((D, T), dtype=np.float32)
    if cfg.get("fusion", "softmax") == "fc":  # DFlash's FC fusion: W_fc [H, T*H], gain [H]
        w["w_fc"] = normal_bf16((H, T * H), std, seed, "w_fc")
        w["g_fc"] = np.full(H, one, dtype=np.uint16)
    return w


def make_hidden(cfg, n_rows, seed, tag):
    """Target hidden states ~N(0,1) as bf16 bits, [n_rows, T, H]."""
    return normal_bf16((n_rows, cfg["n_target_layers"], cfg["hidden"]), 1.0, seed, "hidden/" + tag)


def make_anchor(cfg, batch, seed, tag="anchor"):
    """Anchor tokens ~U[0, V-1) (the mask id V-1 excluded)."""
    return _rng(seed, tag).integers(0, cfg["vocab"] - 1, size=batch).astype(np.int32)


def context_lengths(cfg, seed):
    """Context length per sequence after this step's append."""
    B, ctx = cfg["batch"], cfg["context"]
    if isinstance(ctx, tuple):
        return _rng(seed, "ctx_len").integers(ctx[0], ctx[1] + 1, size=B).astype(np.int64)
    return np.full(B, ctx, dtype=np.int64)


def appended_rows(cfg, seed):
    """Rows appended this step per sequence: fixed n_new, or (ragged
    batches) 1 + leading successes of N-1 Bernoulli(agreement) trials."""
    B = cfg["batch"]
    if not isinstance(cfg["context"], tuple):
        return np.full(B, cfg["n_new"], dtype=np.int64)
    ok = _rng(seed, "n_new").random((B, cfg["block_size"] - 1)) < cfg["agreement"]
    lead = np.argmin(np.concatenate([ok, np.zeros((B, 1), bool)], axis=1), axis=1)
    return (1 + lead).astype(np.int64)


def make_logits(cfg, draft, seed, step=0):
    """Synthetic target logits [B, N, V] built around the given draft tokens.

    tiny ("boost3"): z ~ N(0,1) float32; rows r < N-1 get +3 on d_{r+1}
      with probability `agreement`.
    greedy shapes ("top_plus1"): z ~ N(0,1) -> bf16; rows r < N-1 get
      z[r, d_{r+1}] = max_k z[r, k] + 1 with probability `agreement`.
    temperature 1 ("accept_p"): z ~ N(0,1) -> bf16; rows r < N-1 get
      z[r, d] = ln(p/(1-p)) + logsumexp_{k != d} z[r, k], so that d has
      probability p = `agreement` under softmax(z[r]) (before rounding).
    Returns float32 (the "boost3" model, or any model with
    ``cfg["logits_f32"]`` set: no bf16 rounding anywhere) or bf16 bits
    (uint16).
    """
    draft = np.asarray(draft)
    B, N, V = draft.shape[0], cfg["block_size"], cfg["vocab"]
    r = _rng(seed, f"logits/{step}")
    z = r.standard_normal((B, N, V), dtype=np.float32)
    coin = r.random((B, N - 1)) < cfg["agreement"]
    model = cfg["logit_model"]
    f32 = model == "boost3" or bool(cfg.get("logits_f32"))
    if not f32:
        z = f32_to_bf16_bits(z).astype(np.uint32) << 16
        z = z.view(np.float32)
    for b in range(B):
        for row in range(N - 1):
            d = int(draft[b, row])
            if model == "boost3":
                if coin[b, row]:
                    z[b, row, d] += 3.0
            elif model == "top_plus1":
                if coin[b, row]:
                    z[b, row, d] = z[b, row].max() + 1.0
            elif model == "accept_p":
                p = cfg["agreement"]
                rest = np.delete(z[b, row].astype(np.float64), d)
                m = rest.max()
                z[b, row, d] = np.log(p / (1 - p)) + m + np.log(np.exp(rest - m).sum())
    if f32:
        return z
    return f32_to_bf16_bits(z)
