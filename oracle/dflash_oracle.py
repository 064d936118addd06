"""Plain float64 oracle of one block-diffusion decode step: fuse, append, draft, verify.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library or its binding and imports nothing from them.

What it follows (the pages are three web summaries; sections, not lines):
  * "DFLARE - scaling draft capacity of block-diffusion speculative decoding"
    (gist.science technical summary), section 2.1 "Adaptive layer fusion":
    per-draft-layer softmax weights alpha^(i) over the T target layers, a
    weighted sum of the T target hidden states, then RMSNorm.
  * same page, section 1 (first limitation): DFlash's own conditioning, one
    fully-connected layer fusing the T target states into a single context
    shared by every draft layer (the ``fusion == "fc"`` variant).
  * same page, section 2.2 "Heterogeneous KV projections": the fused
    context goes through its own W^t_K / W^t_V, the draft block (the
    target-decoded token plus mask positions) through W^d_K / W^d_V.
  * same page, section 1 and "DFlash: Block Diffusion for Flash Speculative
    Decoding" (euno.news), Overview and Methodology step 2: the whole block
    is drafted in one non-autoregressive forward pass; the context enters
    every draft layer as keys/values only.
  * DFlash page, Methodology step 3: parallel verification with the
    standard speculative acceptance test; a rejected position is replaced
    by the target's own token. Key contributions: the result is lossless.
  * DFlash page, Methodology step 4: the window advances by the number of
    accepted tokens.
  * DFlash page, Methodology step 3 with a sampled draft: the same standard
    acceptance test with a general drafter distribution (accept with
    probability min(1, p/q), resample from max(0, p - q)).
  * "D^2SD: Accelerating Speculative Decoding with Dual Diffusion Draft
    Models" (euno.news), Methodology steps 1-4: per-position confidence of
    the first draft, K prefixes cut where a rejection is most likely, a
    second batched drafting pass re-anchored on each prefix, and one
    verification of all candidates that keeps the longest accepted prefix.

Where the pages are silent the readings are (each also listed in the
design notes): one pass, no noise; mask positions are an embedding row
``mask_token_id``; rotate-half RoPE with theta from the config; every block
query sees all context keys and all block keys; GQA by contiguous groups;
scale 1/sqrt(d_h); RMSNorm eps from the config with a gain at each of the
four norms (fusion, pre-attention, pre-MLP, final); no biases; argmax ties
go to the lowest index; target row r predicts the token after block
position r.

Arithmetic is float64 throughout. The stated precision of the path is bf16
storage with fp32 accumulation; what is stored in bf16 is the weights (given
as bf16 values) and the keys/values: the rotated context K and the context V
in the cache, and the rotated block K and block V the draft attends to. Those
four are rounded to bf16 (round to nearest even, 8 significant bits) here;
transient activations (fused context, normed rows, queries, attention output,
SwiGLU output) are not storage and stay exact. Passing ``storage=False``
turns the K/V rounding off too (exact float64), which the pins use. Logits
are rounded to float32 before the argmax, the precision in which the kernel
takes that decision.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, invariants, library routines (torch's RMSNorm,
scaled-dot-product attention and SiLU; numpy's Philox) or brute force. The
composition of the whole step has no printed example on the pages: parity
unpinned beyond its parts.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits_to_f64", "fusion_weights", "rmsnorm", "rope",
    "fuse_context", "fuse_context_fc", "attention", "silu", "argmax_first", "top2_gap",
    "OracleModel", "OracleCache", "ctx_append", "draft_block",
    "verify_greedy", "verify_temp1", "philox4x64_10", "philox4x64_10_vec",
    "rng_uniform", "rng_gumbel_row", "draft_confidence", "d2sd_cut_points",
    "d2sd_candidate_tokens", "d2sd_candidates", "verify_greedy_multi",
    "draft_sample", "verify_sampled", "rng_gumbel_row_words",
]


# ---------------------------------------------------------------- precision
def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits. With x = m * 2**e, 0.5 <= |m| < 1,
    the quantum is 2**(e-8); ``np.round`` rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    scaled = np.ldexp(x, 8 - e)
    return np.ldexp(np.round(scaled), e - 8)


def bf16_bits_to_f64(bits):
    """Widen raw bfloat16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _store(x, storage):
    return bf16_round(x) if storage else np.asarray(x, dtype=np.float64)


# ------------------------------------------------- DFLARE 2.1: layer fusion
def fusion_weights(w_fuse):
    """alpha^(i) = softmax over the T entries of row i of W_fuse [D, T].

    DFLARE summary, section 2.1: a learnable fusion matrix W_fuse gives,
    through a softmax, per-draft-layer weights alpha^(i) (D x T scalars).
    Max-subtracted; entries of -inf get weight exactly 0.
    """
    w = np.asarray(w_fuse, dtype=np.float64)
    m = np.max(w, axis=1, keepdims=True)
    e = np.exp(w - m)
    return e / np.sum(e, axis=1, keepdims=True)


def rmsnorm(x, g, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def fuse_context(alpha_i, h, g, eps):
    """f^(i)_t = RMSNorm(sum_j alpha^(i)_j h^(j)_t) * g_fuse^(i).

    DFLARE summary, section 2.1. ``h`` is [n, T, H] (the T selected target
    layers per appended token); the sum runs in ascending j.
    """
    h = np.asarray(h, dtype=np.float64)
    s = np.zeros((h.shape[0], h.shape[2]), dtype=np.float64)
    for j in range(h.shape[1]):
        s = s + alpha_i[j] * h[:, j, :]
    return rmsnorm(s, g, eps)


def fuse_context_fc(w_fc, h, g, eps):
    """c_t = RMSNorm(W_fc [h^(0)_t; ...; h^(T-1)_t]) * g_fc.

    DFlash's conditioning as the DFLARE summary describes it (section 1,
    first limitation): one fully-connected layer merges the hidden states of
    the selected target layers into a single shared representation, and that
    same signal feeds every draft layer. ``h`` is [n, T, H]; the T states of
    a token are concatenated along the feature axis in layer order; W_fc is
    [H, T*H] (nn.Linear, no bias). The RMSNorm with gain after the layer is
    the reading taken here, as in DFLARE's own fusion (section 2.1).
    """
    h = np.asarray(h, dtype=np.float64)
    n, T, H = h.shape
    return rmsnorm(h.reshape(n, T * H) @ np.asarray(w_fc, dtype=np.float64).T, g, eps)


# ------------------------------------------------------------------- RoPE
def rope(x, pos, theta):
    """Rotate-half rotary embedding of x [n, heads, d] at positions pos [n].

    Dimension pairs (j, j + d/2) are rotated by the angle pos * theta^(-2j/d),
    angles in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# -------------------------------------------------------------- attention
def attention(q, k, v):
    """Unmasked GQA attention of block queries over [context ; block] keys.

    q [N, n_q, d]; k, v [Lk, n_kv, d]. Query head hq reads kv head
    hq // (n_q / n_kv). Scale 1/sqrt(d); max-subtracted softmax over all
    Lk keys: every block position sees every context key and every block
    key (the draft is not autoregressive: DFlash page, Methodology; DFLARE
    summary, section 1).
    """
    n, n_q, d = q.shape
    n_kv = k.shape[1]
    group = n_q // n_kv
    out = np.zeros((n, n_q, d), dtype=np.float64)
    for hq in range(n_q):
        g = hq // group
        s = (q[:, hq, :] @ k[:, g, :].T) / math.sqrt(d)
        s = s - np.max(s, axis=1, keepdims=True)
        a = np.exp(s)
        a = a / np.sum(a, axis=1, keepdims=True)
        out[:, hq, :] = a @ v[:, g, :]
    return out


def silu(z):
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------- argmax
def argmax_first(z):
    """Index of the maximum of each row; the lowest index wins ties."""
    return np.argmax(np.asarray(z), axis=-1)


def top2_gap(z):
    """Largest minus second-largest value of each row (float64)."""
    z = np.asarray(z, dtype=np.float64)
    part = np.partition(z, -2, axis=-1)
    return part[..., -1] - part[..., -2]


# ----------------------------------------------------------- model, cache
@dataclass
class OracleModel:
    """Drafter weights as raw bf16 bits (uint16) plus float32 W_fuse.

    Shapes follow nn.Linear ([out, in]), stacked over the D draft layers:
    wq [D, n_q*d, H]; wk_d, wv_d, wk_t, wv_t [D, n_kv*d, H]; wo [D, H, n_q*d];
    wg, wu [D, I, H]; wd [D, H, I]; embed, lm_head [V, H]; g_fuse, g_attn,
    g_mlp [D, H]; g_final [H]; w_fuse [D, T] float32. With ``tied_kv`` the
    context projections are the block ones (DFlash's shared projection).
    With ``fusion == "fc"`` the context is DFlash's FC fusion instead, from
    w_fc [H, T*H] and g_fc [H].
    """
    cfg: dict
    w: dict
    alpha: np.ndarray = field(init=False)

    def __post_init__(self):
        self.alpha = fusion_weights(self.w["w_fuse"])

    def rows(self, name, idx):
        """Selected rows of a 2-D table (embedding), widened to float64."""
        a = self.w[name][np.asarray(idx)]
        return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    def f64(self, name, layer=None):
        if self.cfg.get("tied_kv") and name in ("wk_t", "wv_t"):
            name = {"wk_t": "wk_d", "wv_t": "wv_d"}[name]
        a = self.w[name] if layer is None else self.w[name][layer]
        if a.dtype == np.uint16:
            return bf16_bits_to_f64(a)
        return np.asarray(a, dtype=np.float64)


class OracleCache:
    """Per-layer, per-sequence context keys (rotated) and values, float64."""

    def __init__(self, n_layers):
        self.k = [dict() for _ in range(n_layers)]
        self.v = [dict() for _ in range(n_layers)]
        self.ctx_len = {}

    def length(self, seq):
        return self.ctx_len.get(seq, 0)


# --------------------------------------------- DFLARE 2.2: context append
def ctx_append(model, cache, seq, hidden, storage=True):
    """Append n context rows of sequence ``seq`` to every layer's cache.

    hidden [n, T, H]: the T target-layer states of each appended token.
    Per layer i: f = fuse_context(alpha^(i), ...); K = RoPE(f W^t_K^T) at
    positions ctx_len .. ctx_len+n-1; V = f W^t_V^T (DFLARE summary,
    section 2.2: the target context gets its own W^t_K, W^t_V). With
    ``fusion == "fc"`` every layer takes the one shared f = fuse_context_fc
    (DFlash, as in section 1 of that summary). Then ctx_len += n.
    """
    c = model.cfg
    n_kv, d = c["n_kv_heads"], c["head_dim"]
    hidden = np.asarray(hidden, dtype=np.float64)
    n = hidden.shape[0]
    p0 = cache.length(seq)
    pos = p0 + np.arange(n)
    shared = None
    if c.get("fusion", "softmax") == "fc":
        shared = fuse_context_fc(model.f64("w_fc"), hidden, model.f64("g_fc"), c["rms_eps"])
    for i in range(c["n_layers"]):
        if shared is not None:
            f = shared
        else:
            f = fuse_context(model.alpha[i], hidden, model.f64("g_fuse", i), c["rms_eps"])
        k = (f @ model.f64("wk_t", i).T).reshape(n, n_kv, d)
        v = (f @ model.f64("wv_t", i).T).reshape(n, n_kv, d)
        if c.get("use_rope", 1):
            k = rope(k, pos, c["rope_theta"])
        k = _store(k, storage)
        v = _store(v, storage)
        old_k = cache.k[i].get(seq, np.zeros((0, n_kv, d)))
        old_v = cache.v[i].get(seq, np.zeros((0, n_kv, d)))
        cache.k[i][seq] = np.concatenate([old_k, k], axis=0)
        cache.v[i][seq] = np.concatenate([old_v, v], axis=0)
    cache.ctx_len[seq] = p0 + n


# ------------------------------------------------------- one-pass draft
def draft_block(model, cache, seq, anchor, storage=True, tokens=None):
    """Draft N-1 tokens for sequence ``seq`` in one forward pass.

    Block = [anchor, mask, ..., mask] at positions L .. L+N-1 (L = ctx_len;
    DFLARE summary, section 2.2: the draft's own states are the
    target-decoded token and the masked positions). Each draft layer:
    pre-norm GQA attention with RoPE over [context K/V ; block K/V], then a
    SwiGLU MLP, both residual. Final norm and LM head on block rows
    1..N-1, argmax (lowest index on ties) gives the draft tokens.

    ``tokens`` overrides the block token ids (tests use it). Returns a dict:
    draft [N-1] int, gap [N-1] (top-1 minus top-2 logit), logits [N-1, V]
    (float32 values, float64 dtype), hidden [D+1, N, H] residual stream
    (the embeddings, then the stream after each layer), block_k / block_v
    (per layer, [N, n_kv, d], K rotated).
    """
    c = model.cfg
    N, H = c["block_size"], c["hidden"]
    n_q, n_kv, d = c["n_q_heads"], c["n_kv_heads"], c["head_dim"]
    eps, theta = c["rms_eps"], c["rope_theta"]
    use_rope = c.get("use_rope", 1)
    L = cache.length(seq)
    if tokens is None:
        tokens = [anchor] + [c["mask_token_id"]] * (N - 1)
    tokens = np.asarray(tokens)
    pos = L + np.arange(N)
    x = model.rows("embed", tokens)
    hidden = [x.copy()]
    block_k, block_v = [], []
    for i in range(c["n_layers"]):
        h = rmsnorm(x, model.f64("g_attn", i), eps)
        q = (h @ model.f64("wq", i).T).reshape(N, n_q, d)
        kb = (h @ model.f64("wk_d", i).T).reshape(N, n_kv, d)
        vb = (h @ model.f64("wv_d", i).T).reshape(N, n_kv, d)
        if use_rope:
            q = rope(q, pos, theta)
            kb = rope(kb, pos, theta)
        kb, vb = _store(kb, storage), _store(vb, storage)
        block_k.append(kb)
        block_v.append(vb)
        kc = cache.k[i].get(seq, np.zeros((0, n_kv, d)))
        vc = cache.v[i].get(seq, np.zeros((0, n_kv, d)))
        o = attention(q, np.concatenate([kc, kb]), np.concatenate([vc, vb]))
        o = o.reshape(N, n_q * d)
        x = x + o @ model.f64("wo", i).T
        h2 = rmsnorm(x, model.f64("g_mlp", i), eps)
        a = h2 @ model.f64("wg", i).T
        b = h2 @ model.f64("wu", i).T
        m = silu(a) * b
        x = x + m @ model.f64("wd", i).T
        hidden.append(x.copy())
    y = rmsnorm(x[1:], model.f64("g_final"), eps)
    # Output columns are computed a slice of the vocabulary at a time only
    # to bound memory; each logit is the same full dot product.
    vocab = model.w["lm_head"].shape[0]
    z = np.empty((N - 1, vocab), dtype=np.float64)
    for v0 in range(0, vocab, 16384):
        z[:, v0:v0 + 16384] = y @ model.rows("lm_head", np.arange(v0, min(vocab, v0 + 16384))).T
    z = z.astype(np.float32).astype(np.float64)
    return {
        "draft": argmax_first(z),
        "gap": top2_gap(z),
        "logits": z,
        "hidden": np.stack(hidden),
        "block_k": block_k,
        "block_v": block_v,
    }


# ----------------------------------------------------------- verification
def verify_greedy(draft, z):
    """Greedy verification of one sequence's block.

    draft [N-1]: d_1 .. d_{N-1}; z [N, V]: target logits, row r predicting
    the token after block position r. t_r = argmax z[r] (lowest index on
    ties). a = the largest k with d_j = t_{j-1} for every j <= k; the
    target's own token t_a replaces the first rejected position, or is the
    bonus token when all N-1 are accepted (DFlash page, Methodology step 3).
    Returns (accept_len a, next_token t_a, commit_len a+1).
    """
    t = argmax_first(z)
    n_draft = len(draft)
    a = 0
    while a < n_draft and int(draft[a]) == int(t[a]):
        a += 1
    return a, int(t[a]), a + 1


# ------------------------------------------------- dual-pass drafting (D2SD)
def draft_confidence(z):
    """Confidence of each draft position: the drafter's largest softmax
    probability, max_k softmax(z[r])_k = 1 / sum_k exp(z[r,k] - max z[r])
    (D2SD page, Methodology step 1: a score per position for how likely the
    target accepts it; reading: the drafter's own top probability).
    z [R, V] -> [R] float64."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    return 1.0 / np.exp(z - m).sum(axis=1)


def d2sd_cut_points(conf, K):
    """Where to cut the first draft (D2SD page, Methodology step 2: the
    likeliest rejection points). conf[j-1] is the confidence of draft
    position j = 1 .. N-1. Reading: the min(K, N-1) positions of lowest
    confidence, ties to the lower position, returned in ascending position
    order (the order of the candidates)."""
    ranked = sorted(range(len(conf)), key=lambda j: (float(conf[j]), j))
    return sorted(j + 1 for j in ranked[:min(K, len(conf))])


def d2sd_candidate_tokens(anchor, draft, c, N, mask_id):
    """Input block of the candidate re-anchored at cut point c (D2SD page,
    Methodology step 3): the anchor, the first draft's d_1 .. d_{c-1} kept
    as real tokens, masks from position c on."""
    return [int(anchor)] + [int(t) for t in draft[:c - 1]] + [int(mask_id)] * (N - c)


def d2sd_candidates(model, cache, seq, anchor, K, storage=True):
    """First draft, its confidences and cut points, and the K re-anchored
    candidates (the second pass uses the same weights and the same context
    cache; D2SD page, Methodology steps 1-3). Candidate 0 is the first
    draft; candidate k >= 1 keeps d_1 .. d_{c_k - 1} and takes the second
    pass's argmax tokens from position c_k on.
    Returns dict: first (draft_block output), conf [N-1], cuts [K'],
    drafts [K'+1, N-1], second (draft_block outputs of the second pass)."""
    c = model.cfg
    N = c["block_size"]
    first = draft_block(model, cache, seq, anchor, storage)
    conf = draft_confidence(first["logits"])
    cuts = d2sd_cut_points(conf, K)
    drafts = [np.asarray(first["draft"])]
    second = []
    for cp in cuts:
        toks = d2sd_candidate_tokens(anchor, first["draft"], cp, N, c["mask_token_id"])
        out = draft_block(model, cache, seq, anchor, storage, tokens=toks)
        drafts.append(np.concatenate([np.asarray(first["draft"])[:cp - 1], np.asarray(out["draft"])[cp - 1:]]))
        second.append(out)
    return {"first": first, "conf": conf, "cuts": cuts, "drafts": np.stack(drafts), "second": second}


def verify_greedy_multi(drafts, z):
    """Greedy verification of C candidate blocks of one sequence (D2SD page,
    Methodology step 4: the longest prefix the target agrees with is kept,
    the rest discarded). drafts [C, N-1]; z [C, N, V]: the target's logits
    for each candidate block. Each candidate is verified as in
    ``verify_greedy``; the longest accept wins, the lowest candidate index
    on ties. Returns (accept_len, next_token, commit_len, chosen)."""
    best = None
    for ci in range(len(drafts)):
        a, nxt, cm = verify_greedy(drafts[ci], z[ci])
        if best is None or a > best[0]:
            best = (a, nxt, cm, ci)
    return best


# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC 2011): the multipliers and Weyl key increments are
# the published ones.
_PHILOX_M0 = 0xD2E7470EE14C6C93
_PHILOX_M1 = 0xCA5A826395121157
_PHILOX_W0 = 0x9E3779B97F4A7C15
_PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds on Python integers: 4 words out."""
    c0, c1, c2, c3 = (int(w) & _MASK64 for w in counter)
    k0, k1 = (int(w) & _MASK64 for w in key)
    for r in range(10):
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0) & _MASK64, p1 & _MASK64, \
                         ((p0 >> 64) ^ c3 ^ k1) & _MASK64, p0 & _MASK64
        if r < 9:
            k0 = (k0 + _PHILOX_W0) & _MASK64
            k1 = (k1 + _PHILOX_W1) & _MASK64
    return [c0, c1, c2, c3]


def _mulhilo64(a, m):
    """Full 64x64 -> 128-bit product of uint64 arrays by a constant."""
    a = np.asarray(a, dtype=np.uint64)
    lo32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a_lo, a_hi = a & lo32, a >> s32
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> s32) + (lh & lo32) + (hl & lo32)
    lo = (ll & lo32) | ((mid & lo32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def philox4x64_10_vec(c0, c1, c2, c3, k0, k1):
    """Philox4x64-10 over uint64 arrays (same rounds as ``philox4x64_10``)."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(w, dtype=np.uint64) for w in (c0, c1, c2, c3))
        c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
        k0, k1 = np.uint64(k0 & _MASK64), np.uint64(k1 & _MASK64)
        for r in range(10):
            hi0, lo0 = _mulhilo64(c0, _PHILOX_M0)
            hi1, lo1 = _mulhilo64(c2, _PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            if r < 9:
                k0 = k0 + np.uint64(_PHILOX_W0)
                k1 = k1 + np.uint64(_PHILOX_W1)
        return c0, c1, c2, c3


def _counter(step, seq, row, k, stream):
    """Counter words (k, row | stream << 32, seq, step); key (seed, 0)."""
    return (k, (int(row) & 0xFFFFFFFF) | (int(stream) << 32), seq, step)


def rng_uniform(seed, step, seq, row, k=0, stream=0):
    """Uniform in [0, 1): the top 24 bits of Philox word 0, times 2^-24."""
    w0 = philox4x64_10(_counter(step, seq, row, k, stream), (seed, 0))[0]
    return float(w0 >> 40) * 2.0 ** -24


def rng_gumbel_row(seed, step, seq, row, vocab, stream=1):
    """Standard Gumbel noise for every k < vocab of one row, float32.

    u' = (top 23 bits of Philox word 0 + 1/2) * 2^-23 lies strictly in
    (0, 1) and is exact in float32; G = -log(-log u'), evaluated in float32.
    Stream 1 serves the verification's samples, stream 2 the sampled draft.
    """
    k = np.arange(vocab, dtype=np.uint64)
    c1 = np.uint64((int(row) & 0xFFFFFFFF) | (int(stream) << 32))
    w0, _, _, _ = philox4x64_10_vec(k, c1, np.uint64(seq), np.uint64(step), seed, 0)
    u = ((w0 >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23
    u = u.astype(np.float32)
    return (-np.log(-np.log(u))).astype(np.float32)


def verify_temp1(draft, z, seed, step, seq):
    """Temperature-1 verification by rejection sampling (lossless).

    The drafter emits argmax tokens, so its proposal is one-hot on d_j. The
    standard speculative test (DFlash page, Methodology step 3; lossless per
    its key contributions) then reads: accept d_{a+1} iff u_a < p_a(d_{a+1})
    with p_r = softmax(z[r]) and u_a uniform; at the first rejection sample
    from p_a with d_{a+1} removed and renormalised (the residual
    max(0, p - q) for one-hot q); if all N-1 are accepted, sample the bonus
    token from p_{N-1}. Samples are drawn by Gumbel-max: argmax_k of
    z[row, k] + G_k in float32, lowest index on ties.

    Returns (a, next_token, commit_len, info) where info holds p, u and the
    Gumbel top-2 gap of the sampled row (tests use them for the exclusion
    rule).
    """
    z = np.asarray(z, dtype=np.float64)
    n_rows, vocab = z.shape
    mx = np.max(z, axis=1, keepdims=True)
    lse = (mx + np.log(np.sum(np.exp(z - mx), axis=1, keepdims=True)))[:, 0]
    a = 0
    ps, us = [], []
    while a < n_rows - 1:
        u = rng_uniform(seed, step, seq, a, 0, 0)
        p = math.exp(z[a, int(draft[a])] - lse[a])
        ps.append(p)
        us.append(u)
        if u < p:
            a += 1
        else:
            break
    row = a
    key = z[row].astype(np.float32) + rng_gumbel_row(seed, step, seq, row, vocab)
    if a < n_rows - 1:
        key[int(draft[a])] = -np.inf
    nxt = int(argmax_first(key))
    finite = key[np.isfinite(key)].astype(np.float64)
    info = {"p": ps, "u": us, "gumbel_gap": float(top2_gap(finite)), "row": row}
    return a, nxt, a + 1, info


def rng_gumbel_row_words(seed, step, seq, row, vocab, stream=2):
    """Standard Gumbel noise for every k < vocab of one row, float32, from all
    four Philox words: entry k takes word k % 4 of the block at counter
    (k // 4, row | stream << 32, seq, step); u' and G as in rng_gumbel_row.
    The sampled draft's noise (stream 2)."""
    n4 = (vocab + 3) // 4
    k4 = np.arange(n4, dtype=np.uint64)
    c1 = np.uint64((int(row) & 0xFFFFFFFF) | (int(stream) << 32))
    words = philox4x64_10_vec(k4, c1, np.uint64(seq), np.uint64(step), seed, 0)
    w = np.stack(words, axis=1).reshape(-1)[:vocab]  # entry 4i + j <- word j of block i
    u = ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23
    u = u.astype(np.float32)
    return (-np.log(-np.log(u))).astype(np.float32)


# ------------------------------------------ sampled drafts (temperature tau)
def _row_lse(z):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


def draft_sample(z, tau, seed, step, seq):
    """Draft tokens sampled from the drafter at temperature tau > 0.

    z [N-1, V]: the drafter's logits of block rows 1 .. N-1 (LM-head row r
    gives draft position r + 1). Its proposal for that position is
    q_r = softmax(z[r] / tau); the token is drawn by Gumbel-max,
    argmax_k (z[r, k] / tau + G_k), in float32 with the Gumbel noise of
    rng_gumbel_row_words (stream 2), lowest index on ties. Returns
    (draft [N-1], key top-2 gap per row).
    """
    z = np.asarray(z, dtype=np.float64)
    n_rows, vocab = z.shape
    draft = np.zeros(n_rows, dtype=np.int64)
    gaps = np.zeros(n_rows)
    for r in range(n_rows):
        key = z[r].astype(np.float32) / np.float32(tau) + rng_gumbel_row_words(seed, step, seq, r, vocab, stream=2)
        draft[r] = int(argmax_first(key))
        gaps[r] = float(top2_gap(key.astype(np.float64)))
    return draft, gaps


def verify_sampled(draft, zq, tau, z, seed, step, seq):
    """Lossless verification of a sampled draft at target temperature 1.

    The standard speculative acceptance test (DFlash page, Methodology step
    3; lossless per its key contributions) with a general proposal: target
    p_r = softmax(z[r]) and drafter q_r = softmax(zq[r] / tau) for the token
    d_{r+1} proposed at row r. Accept d_{a+1} iff u_a * q_a(d) < p_a(d),
    i.e. with probability min(1, p/q), u_a the stream-0 uniform of row a; at
    the first rejection draw from the residual max(0, p_a - q_a)
    renormalised, by Gumbel-max over log(p_k - q_k) + G_k (stream 1) on the
    entries with p_k > q_k; if all N-1 are accepted, draw the bonus token
    from p_{N-1} (argmax of z + G, as for the one-hot draft). The keys are
    float32, lowest index on ties.

    Returns (a, next_token, commit_len, info): info holds per tested row p,
    q, u, and the Gumbel top-2 gap of the sampled row (exclusion rule).
    """
    z = np.asarray(z, dtype=np.float64)
    zq = np.asarray(zq, dtype=np.float64) / float(tau)
    n_rows, vocab = z.shape
    lse_p, lse_q = _row_lse(z), _row_lse(zq)
    a = 0
    ps, qs, us = [], [], []
    while a < n_rows - 1:
        d = int(draft[a])
        u = rng_uniform(seed, step, seq, a, 0, 0)
        p = math.exp(z[a, d] - lse_p[a])
        q = math.exp(zq[a, d] - lse_q[a])
        ps.append(p)
        qs.append(q)
        us.append(u)
        if u * q < p:
            a += 1
        else:
            break
    g = rng_gumbel_row(seed, step, seq, a, vocab, stream=1)
    if a < n_rows - 1:
        w = np.exp(z[a] - lse_p[a]) - np.exp(zq[a] - lse_q[a])
        key = np.full(vocab, -np.inf, dtype=np.float32)
        pos = w > 0
        key[pos] = np.log(w[pos]).astype(np.float32) + g[pos]
    else:
        key = z[a].astype(np.float32) + g
    nxt = int(argmax_first(key))
    finite = key[np.isfinite(key)].astype(np.float64)
    info = {"p": ps, "q": qs, "u": us, "row": a,
            "gumbel_gap": float(top2_gap(finite)) if finite.size > 1 else float("inf")}
    return a, nxt, a + 1, info
