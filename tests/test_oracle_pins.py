"""Pins of the oracle against what the pages and the mathematics fix.

Each test checks one oracle function against something other than itself:
a closed form, an invariant, a library routine (torch's RMSNorm, SDPA and
SiLU; scipy's softmax; numpy's Philox), a published known-answer vector, or
brute force on tiny inputs. The composition of a whole decode step has no
worked example on the pages; it is pinned only through these parts.
"""
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    c = dict(hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
             intermediate=48, vocab=64, n_target_layers=3, block_size=6,
             rope_theta=1e4, rms_eps=1e-6, mask_token_id=63, tied_kv=0, use_rope=1)
    c.update(kw)
    return c


def tiny_weights(c, seed=0, scale=0.3):
    r = np.random.default_rng(seed)
    D, H, I, V, T = c["n_layers"], c["hidden"], c["intermediate"], c["vocab"], c["n_target_layers"]
    qd, kd = c["n_q_heads"] * c["head_dim"], c["n_kv_heads"] * c["head_dim"]
    n = lambda *s: r.standard_normal(s) * scale
    w = dict(wq=n(D, qd, H), wk_d=n(D, kd, H), wv_d=n(D, kd, H), wk_t=n(D, kd, H),
             wv_t=n(D, kd, H), wo=n(D, H, qd), wg=n(D, I, H), wu=n(D, I, H),
             wd=n(D, H, I), embed=r.standard_normal((V, H)), lm_head=n(V, H),
             g_fuse=1 + 0.1 * r.standard_normal((D, H)), g_attn=1 + 0.1 * r.standard_normal((D, H)),
             g_mlp=1 + 0.1 * r.standard_normal((D, H)), g_final=1 + 0.1 * r.standard_normal(H),
             w_fuse=r.standard_normal((D, T)))
    return w


# ------------------------------------------------------------ bf16 storage
def test_bf16_round_matches_torch_rne():
    r = np.random.default_rng(1)
    x = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    ours = O.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even is 1.
    assert O.bf16_round(1 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert O.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert O.bf16_round(-(1 + 2.0 ** -8)) == -1.0
    assert O.bf16_round(0.0) == 0.0


def test_bf16_bits_widen():
    got = O.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x4049], dtype=np.uint16))
    assert list(got) == [1.0, -2.0, 0.25, 0.0, 3.140625]


# ------------------------------------------------------- fusion (DFLARE 2.1)
def test_fusion_weights_simplex_and_library_softmax():
    w = np.random.default_rng(2).standard_normal((7, 9)) * 3
    a = O.fusion_weights(w)
    assert np.all(a >= 0)
    assert np.allclose(a.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(a, scipy.special.softmax(w, axis=1), rtol=1e-13, atol=0)
    # softmax is shift invariant per row
    assert np.allclose(O.fusion_weights(w + 123.0), a, rtol=1e-12, atol=0)


def test_fusion_weights_special_rows():
    w = np.zeros((2, 5))
    w[1] = -np.inf
    w[1, 3] = 0.7
    a = O.fusion_weights(w)
    assert np.all(a[0] == 0.2)
    assert list(a[1]) == [0, 0, 0, 1.0, 0]


def test_one_hot_fusion_is_rmsnorm_of_that_layer():
    r = np.random.default_rng(3)
    h = r.standard_normal((5, 4, 32))
    g = 1 + 0.1 * r.standard_normal(32)
    alpha = np.array([0.0, 0.0, 1.0, 0.0])
    f = O.fuse_context(alpha, h, g, 1e-6)
    ref = F.rms_norm(torch.from_numpy(h[:, 2, :]), (32,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(f, ref, rtol=1e-12, atol=1e-14)


def test_fusion_of_two_layers_matches_library_norm_of_mean():
    r = np.random.default_rng(4)
    h = r.standard_normal((3, 2, 16))
    g = np.ones(16)
    f = O.fuse_context(np.array([0.5, 0.5]), h, g, 1e-6)
    mean = torch.from_numpy(h.mean(axis=1))
    ref = F.rms_norm(mean, (16,), eps=1e-6).numpy()
    assert np.allclose(f, ref, rtol=1e-12, atol=1e-14)


def test_fusion_constant_vector_closed_form():
    # s = c * 1  ->  f = c / sqrt(c^2 + eps) * g  (eps matters for small c)
    g = np.linspace(0.5, 1.5, 8)
    for c in (1e-3, -2e-3, 0.7):
        h = np.full((1, 1, 8), c)
        f = O.fuse_context(np.array([1.0]), h, g, 1e-6)
        assert np.allclose(f[0], c / math.sqrt(c * c + 1e-6) * g, rtol=1e-13, atol=0)


def test_rmsnorm_scale_invariance():
    x = np.random.default_rng(5).standard_normal((4, 64))
    g = np.ones(64)
    assert np.allclose(O.rmsnorm(37.0 * x, g, 1e-6), O.rmsnorm(x, g, 1e-6), rtol=1e-6, atol=0)


# ------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = np.random.default_rng(6).standard_normal((3, 2, 16))
    assert np.array_equal(O.rope(x, np.zeros(3), 1e6), x)


def test_rope_is_complex_rotation_of_half_pairs():
    # rotate-half RoPE == multiplying z_j = x_j + i x_{j+d/2} by exp(i p theta^(-2j/d))
    r = np.random.default_rng(7)
    d, theta = 16, 1e6
    x = r.standard_normal((5, 3, d))
    pos = np.array([0, 1, 7, 4096, 8191])
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    j = np.arange(d // 2)
    rot = np.exp(1j * pos[:, None, None] * np.power(theta, -2.0 * j / d)[None, None, :])
    w = z * rot
    ref = np.concatenate([w.real, w.imag], axis=-1)
    assert np.allclose(O.rope(x, pos, theta), ref, rtol=0, atol=1e-12)


def test_rope_relative_position_and_norm():
    r = np.random.default_rng(8)
    q = r.standard_normal((1, 1, 32))
    k = r.standard_normal((1, 1, 32))
    s1 = np.sum(O.rope(q, np.array([100]), 1e4) * O.rope(k, np.array([37]), 1e4))
    s2 = np.sum(O.rope(q, np.array([100 + 999]), 1e4) * O.rope(k, np.array([37 + 999]), 1e4))
    assert abs(s1 - s2) < 1e-10
    assert np.isclose(np.linalg.norm(O.rope(q, np.array([12345]), 1e6)), np.linalg.norm(q), rtol=1e-13)


# -------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa_with_gqa():
    r = np.random.default_rng(9)
    N, n_q, n_kv, d, L = 6, 8, 2, 16, 37
    q = r.standard_normal((N, n_q, d))
    k = r.standard_normal((L, n_kv, d))
    v = r.standard_normal((L, n_kv, d))
    got = O.attention(q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)                      # [n_q, N, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_zero_queries_average_values():
    r = np.random.default_rng(10)
    k = r.standard_normal((11, 2, 8))
    v = r.standard_normal((11, 2, 8))
    out = O.attention(np.zeros((4, 4, 8)), k, v)
    for hq in range(4):
        assert np.allclose(out[:, hq, :], v[:, hq // 2, :].mean(axis=0), atol=1e-13)


def test_attention_block_permutation_equivariance_without_rope():
    r = np.random.default_rng(11)
    N, L = 6, 9
    q = r.standard_normal((N, 4, 8))
    kb, vb = r.standard_normal((N, 2, 8)), r.standard_normal((N, 2, 8))
    kc, vc = r.standard_normal((L, 2, 8)), r.standard_normal((L, 2, 8))
    perm = r.permutation(N)
    base = O.attention(q, np.concatenate([kc, kb]), np.concatenate([vc, vb]))
    permuted = O.attention(q[perm], np.concatenate([kc, kb[perm]]), np.concatenate([vc, vb[perm]]))
    assert np.allclose(permuted, base[perm], atol=1e-12)


def test_softmax_over_concatenation_equals_lse_merge_of_parts():
    r = np.random.default_rng(12)
    q = r.standard_normal((3, 1, 8))
    k = r.standard_normal((20, 1, 8))
    v = r.standard_normal((20, 1, 8))
    full = O.attention(q, k, v)
    parts = []
    for sl in (slice(0, 13), slice(13, 20)):
        s = q[:, 0, :] @ k[sl, 0, :].T / math.sqrt(8)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        parts.append((m, p.sum(axis=1), p @ v[sl, 0, :]))
    M = np.maximum(parts[0][0], parts[1][0])
    num = sum(np.exp(m - M)[:, None] * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    assert np.allclose(full[:, 0, :], num / den[:, None], atol=1e-13)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)


# ---------------------------------------------------------- argmax helpers
def test_argmax_first_and_gap_brute_force():
    r = np.random.default_rng(13)
    z = r.integers(0, 4, size=(200, 9)).astype(np.float64)   # many ties
    idx = O.argmax_first(z)
    gap = O.top2_gap(z)
    for row, i, gp in zip(z, idx, gap):
        best = 0
        for j in range(len(row)):
            if row[j] > row[best]:
                best = j
        assert i == best
        srt = sorted(row, reverse=True)
        assert gp == srt[0] - srt[1]


# ------------------------------------------ draft block special cases
def _model(c, w):
    return O.OracleModel(c, w)


def _prefill(model, c, L, seed=20, seq=0):
    cache = O.OracleCache(c["n_layers"])
    h = np.random.default_rng(seed).standard_normal((L, c["n_target_layers"], c["hidden"]))
    O.ctx_append(model, cache, seq, h, storage=False)
    return cache, h


def test_zero_output_projections_predict_mask_row_closed_form():
    c = tiny_cfg()
    w = tiny_weights(c)
    w["wo"][:] = 0
    w["wd"][:] = 0
    m = _model(c, w)
    cache, _ = _prefill(m, c, 10)
    out = O.draft_block(m, cache, 0, anchor=5, storage=False)
    # the residual stream never changes, so every mask row is E[mask]
    assert np.array_equal(out["hidden"][-1], out["hidden"][0])
    e = torch.from_numpy(w["embed"][c["mask_token_id"]][None, :])
    y = F.rms_norm(e, (c["hidden"],), torch.from_numpy(w["g_final"]), eps=c["rms_eps"])
    expect = int(torch.argmax((y @ torch.from_numpy(w["lm_head"]).T)[0]))
    assert list(out["draft"]) == [expect] * (c["block_size"] - 1)


def test_zero_gate_mlp_adds_nothing():
    c = tiny_cfg(n_layers=1)
    w = tiny_weights(c)
    w["wg"][:] = 0
    w["wo"][:] = 0
    m = _model(c, w)
    cache, _ = _prefill(m, c, 4)
    out = O.draft_block(m, cache, 0, anchor=1, storage=False)
    assert np.array_equal(out["hidden"][1], out["hidden"][0])


def test_one_layer_draft_matches_torch_composition():
    """One draft layer plus LM head against torch's own RMSNorm, linear,
    SDPA and SiLU, with the context K/V built the same way."""
    c = tiny_cfg(n_layers=1)
    w = tiny_weights(c, seed=21)
    m = _model(c, w)
    L = 7
    cache, h = _prefill(m, c, L)
    anchor = 9
    out = O.draft_block(m, cache, 0, anchor, storage=False)

    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    H, N, d = c["hidden"], c["block_size"], c["head_dim"]
    n_q, n_kv = c["n_q_heads"], c["n_kv_heads"]
    eps, theta = c["rms_eps"], c["rope_theta"]

    def rot(x, pos):  # complex-number RoPE, independent of the oracle's
        xc = torch.complex(x[..., : d // 2], x[..., d // 2:])
        fr = theta ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
        ph = torch.polar(torch.ones(len(pos), d // 2, dtype=torch.float64),
                         t(pos)[:, None] * fr[None, :])[:, None, :]
        y = xc * ph
        return torch.cat([y.real, y.imag], dim=-1)

    alpha = torch.softmax(t(w["w_fuse"][0]), dim=0)
    fused = F.rms_norm((t(h) * alpha[None, :, None]).sum(dim=1), (H,), t(w["g_fuse"][0]), eps=eps)
    kc = rot(F.linear(fused, t(w["wk_t"][0])).view(L, n_kv, d), np.arange(L))
    vc = F.linear(fused, t(w["wv_t"][0])).view(L, n_kv, d)
    tokens = [anchor] + [c["mask_token_id"]] * (N - 1)
    x = t(w["embed"][tokens])
    pos = np.arange(L, L + N)
    hn = F.rms_norm(x, (H,), t(w["g_attn"][0]), eps=eps)
    q = rot(F.linear(hn, t(w["wq"][0])).view(N, n_q, d), pos)
    kb = rot(F.linear(hn, t(w["wk_d"][0])).view(N, n_kv, d), pos)
    vb = F.linear(hn, t(w["wv_d"][0])).view(N, n_kv, d)
    K = torch.cat([kc, kb]).permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)
    V = torch.cat([vc, vb]).permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), K, V).permute(1, 0, 2).reshape(N, -1)
    x = x + F.linear(o, t(w["wo"][0]))
    h2 = F.rms_norm(x, (H,), t(w["g_mlp"][0]), eps=eps)
    x = x + F.linear(F.silu(F.linear(h2, t(w["wg"][0]))) * F.linear(h2, t(w["wu"][0])), t(w["wd"][0]))
    assert np.allclose(out["hidden"][1], x.numpy(), rtol=1e-10, atol=1e-10)
    y = F.rms_norm(x[1:], (H,), t(w["g_final"]), eps=eps)
    z = F.linear(y, t(w["lm_head"])).numpy()
    assert np.allclose(out["logits"], z.astype(np.float32), rtol=1e-6, atol=1e-6)
    assert list(out["draft"]) == list(np.argmax(z.astype(np.float32), axis=1))


def test_tied_kv_is_dflash_shared_projection():
    """W^t = W^d: context and block K/V are one projection of concat[f; h]
    (DFlash's shared KV projection, DFLARE summary section 2.2)."""
    c = tiny_cfg(n_layers=1, tied_kv=1)
    w = tiny_weights(c, seed=22)
    del w["wk_t"], w["wv_t"]
    m = _model(c, w)
    L = 5
    cache, h = _prefill(m, c, L)
    out = O.draft_block(m, cache, 0, 3, storage=False)
    f = O.fuse_context(m.alpha[0], h, w["g_fuse"][0], c["rms_eps"])
    tokens = [3] + [c["mask_token_id"]] * (c["block_size"] - 1)
    hb = O.rmsnorm(w["embed"][tokens], w["g_attn"][0], c["rms_eps"])
    both = np.concatenate([f, hb])
    n_all = both.shape[0]
    k_shared = O.rope((both @ w["wk_d"][0].T).reshape(n_all, c["n_kv_heads"], -1), np.arange(n_all), c["rope_theta"])
    v_shared = (both @ w["wv_d"][0].T).reshape(n_all, c["n_kv_heads"], -1)
    assert np.allclose(np.concatenate([cache.k[0][0], out["block_k"][0]]), k_shared, rtol=1e-12, atol=1e-12)
    assert np.allclose(np.concatenate([cache.v[0][0], out["block_v"][0]]), v_shared, rtol=1e-12, atol=1e-12)


def test_untied_context_uses_its_own_projection():
    c = tiny_cfg(n_layers=1)
    w = tiny_weights(c, seed=23)
    m = _model(c, w)
    cache, h = _prefill(m, c, 4)
    f = O.fuse_context(m.alpha[0], h, w["g_fuse"][0], c["rms_eps"])
    v_t = (f @ w["wv_t"][0].T).reshape(4, c["n_kv_heads"], -1)
    v_d = (f @ w["wv_d"][0].T).reshape(4, c["n_kv_heads"], -1)
    assert np.allclose(cache.v[0][0], v_t, atol=1e-12)
    assert not np.allclose(cache.v[0][0], v_d, atol=1e-3)


# ----------------------------------------- DFlash FC fusion (shared context)
def _selector(T, H, j, scale=1.0):
    """W_fc [H, T*H] that reads layer j's state times `scale`."""
    w = np.zeros((H, T * H))
    w[:, j * H:(j + 1) * H] = np.eye(H) * scale
    return w


def test_fc_fusion_selector_is_one_hot_layer_fusion():
    r = np.random.default_rng(40)
    T, H, eps = 4, 32, 1e-6
    h = r.standard_normal((7, T, H))
    g = 1 + 0.1 * r.standard_normal(H)
    for j in range(T):
        fc = O.fuse_context_fc(_selector(T, H, j), h, g, eps)
        alpha = np.where(np.arange(T) == j, 1.0, 0.0)
        assert np.allclose(fc, O.fuse_context(alpha, h, g, eps), rtol=1e-15, atol=0)
        ref = F.rms_norm(torch.from_numpy(h[:, j]), (H,), weight=torch.from_numpy(g), eps=eps).numpy()
        assert np.allclose(fc, ref, rtol=1e-12, atol=1e-12)


def test_fc_fusion_with_scaled_identities_is_the_weighted_sum_fusion():
    r = np.random.default_rng(41)
    T, H, eps = 5, 24, 1e-6
    h = r.standard_normal((6, T, H))
    g = 1 + 0.1 * r.standard_normal(H)
    alpha = O.fusion_weights(r.standard_normal((1, T)))[0]
    w_fc = sum(_selector(T, H, j, alpha[j]) for j in range(T))
    assert np.allclose(O.fuse_context_fc(w_fc, h, g, eps), O.fuse_context(alpha, h, g, eps), rtol=1e-12, atol=1e-12)


def test_fc_fusion_matches_torch_linear_then_rmsnorm():
    r = np.random.default_rng(42)
    T, H, eps = 3, 40, 1e-6
    h = r.standard_normal((5, T, H))
    w_fc = r.standard_normal((H, T * H)) * 0.1
    g = 1 + 0.1 * r.standard_normal(H)
    cat = torch.cat([torch.from_numpy(h[:, j]) for j in range(T)], dim=1)  # [n, T*H], layer order
    ref = F.rms_norm(F.linear(cat, torch.from_numpy(w_fc)), (H,), weight=torch.from_numpy(g), eps=eps)
    assert np.allclose(O.fuse_context_fc(w_fc, h, g, eps), ref.numpy(), rtol=1e-12, atol=1e-12)
    # the norm comes after the layer: scaling W_fc leaves the context unchanged (up to eps)
    assert np.allclose(O.fuse_context_fc(3.0 * w_fc, h, g, eps), O.fuse_context_fc(w_fc, h, g, eps), rtol=1e-5)


def _fc_model(c, w, r):
    H, T = c["hidden"], c["n_target_layers"]
    w = dict(w, w_fc=r.standard_normal((H, T * H)) * 0.1, g_fc=1 + 0.1 * r.standard_normal(H))
    return O.OracleModel(dict(c, fusion="fc"), w), w


def test_fc_append_feeds_one_shared_context_to_every_layer():
    c = tiny_cfg(n_layers=3)
    r = np.random.default_rng(43)
    w = tiny_weights(c, seed=43)
    for k in ("wk_t", "wv_t"):
        w[k] = np.repeat(w[k][:1], 3, axis=0)  # the same context projection in every layer
    m, w = _fc_model(c, w, r)
    cache, h = _prefill(m, c, 6)
    for i in (1, 2):
        assert np.array_equal(cache.k[i][0], cache.k[0][0]) and np.array_equal(cache.v[i][0], cache.v[0][0])
    f = O.fuse_context_fc(w["w_fc"], h, w["g_fc"], c["rms_eps"])
    v = (f @ w["wv_t"][0].T).reshape(6, c["n_kv_heads"], -1)
    assert np.allclose(cache.v[0][0], v, rtol=1e-12, atol=1e-12)


def test_fc_append_with_a_selector_equals_one_hot_softmax_fusion():
    c = tiny_cfg(n_layers=2)
    r = np.random.default_rng(44)
    w = tiny_weights(c, seed=44)
    T, H, j = c["n_target_layers"], c["hidden"], 1
    g = 1 + 0.1 * r.standard_normal(H)
    w_fc = dict(w, w_fc=_selector(T, H, j), g_fc=g)
    w_sm = dict(w, w_fuse=np.where(np.arange(T) == j, 0.0, -np.inf)[None].repeat(2, 0), g_fuse=np.stack([g, g]))
    h = r.standard_normal((5, T, H))
    a, b = O.OracleCache(2), O.OracleCache(2)
    O.ctx_append(O.OracleModel(dict(c, fusion="fc"), w_fc), a, 0, h, storage=False)
    O.ctx_append(O.OracleModel(c, w_sm), b, 0, h, storage=False)
    for i in range(2):
        assert np.allclose(a.k[i][0], b.k[i][0], rtol=1e-13, atol=1e-13)
        assert np.allclose(a.v[i][0], b.v[i][0], rtol=1e-13, atol=1e-13)


def test_append_in_chunks_equals_one_append():
    c = tiny_cfg()
    m = _model(c, tiny_weights(c, seed=24))
    h = np.random.default_rng(25).standard_normal((9, 3, 32))
    a, b = O.OracleCache(2), O.OracleCache(2)
    O.ctx_append(m, a, 0, h)
    O.ctx_append(m, b, 0, h[:4])
    O.ctx_append(m, b, 0, h[4:])
    for i in range(2):
        assert np.array_equal(a.k[i][0], b.k[i][0])
        assert np.array_equal(a.v[i][0], b.v[i][0])
    assert a.ctx_len[0] == b.ctx_len[0] == 9


def test_identical_mask_rows_without_rope_give_identical_outputs():
    c = tiny_cfg(use_rope=0)
    m = _model(c, tiny_weights(c, seed=26))
    cache, _ = _prefill(m, c, 6)
    out = O.draft_block(m, cache, 0, 2)
    hid = out["hidden"][-1]
    for j in range(2, c["block_size"]):
        assert np.array_equal(hid[j], hid[1])


def test_storage_rounding_lands_on_bf16_grid():
    """K/V (context cache and block) are bf16 storage; the residual stream
    and the other activations are not rounded."""
    c = tiny_cfg()
    m = _model(c, tiny_weights(c, seed=27))
    cache = O.OracleCache(2)
    O.ctx_append(m, cache, 0, np.random.default_rng(28).standard_normal((5, 3, 32)))
    for i in range(2):
        for t in (cache.k[i][0], cache.v[i][0]):
            assert np.array_equal(O.bf16_round(t), t)
    out = O.draft_block(m, cache, 0, 3)
    for i in range(2):
        assert np.array_equal(O.bf16_round(out["block_k"][i]), out["block_k"][i])
        assert np.array_equal(O.bf16_round(out["block_v"][i]), out["block_v"][i])
    assert not np.array_equal(O.bf16_round(out["hidden"][-1]), out["hidden"][-1])


# ---------------------------------------------------- greedy verification
def _brute_accept(draft, t):
    n = len(draft)
    for k in range(n, -1, -1):
        if all(draft[j - 1] == t[j - 1] for j in range(1, k + 1)):
            return k
    return 0


def test_verify_greedy_brute_force():
    r = np.random.default_rng(30)
    for _ in range(500):
        N, V = 6, 4
        z = r.integers(0, 3, size=(N, V)).astype(np.float64)
        t = [int(np.argmax(row)) for row in z]
        draft = np.array([t[j] if r.random() < 0.7 else r.integers(0, V) for j in range(N - 1)])
        a, nxt, commit = O.verify_greedy(draft, z)
        assert a == _brute_accept(list(draft), t)
        assert nxt == t[a] and commit == a + 1


def test_verify_greedy_all_agree_and_first_disagrees():
    z = np.eye(5)[[1, 2, 3, 4, 0]] * 3.0     # argmax of row r is (r+1) % 5
    a, nxt, _ = O.verify_greedy(np.array([1, 2, 3, 4]), z)
    assert (a, nxt) == (4, 0)
    a, nxt, _ = O.verify_greedy(np.array([0, 2, 3, 4]), z)
    assert (a, nxt) == (0, 1)


# ------------------------------------------------------------------ RNG
def test_philox_known_answer_vectors():
    path = os.path.join(GOLDEN, "philox4x64_10_kat.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for row in rows:
        vals = [int(x, 16) for x in row]
        assert O.philox4x64_10(vals[0:4], vals[4:6]) == vals[6:10]
        v = O.philox4x64_10_vec(*[np.uint64(x) for x in vals[0:4]], vals[4], vals[5])
        assert [int(x) for x in v] == vals[6:10]


def test_philox_matches_numpy_library():
    # numpy's Philox (4x64-10) increments its counter before each block.
    r = np.random.default_rng(31)
    for _ in range(20):
        ctr = [int(x) for x in r.integers(0, 2 ** 63, size=4)]
        key = [int(x) for x in r.integers(0, 2 ** 63, size=2)]
        bg = np.random.Philox(counter=ctr, key=key)
        got = [int(x) for x in bg.random_raw(4)]
        nxt = [ctr[0] + 1] + ctr[1:]
        assert O.philox4x64_10(nxt, key) == got


def test_uniforms_are_exact_fp32_and_in_range():
    us = [O.rng_uniform(7, 3, 1, row) for row in range(200)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(np.float32(u)) == u for u in us)
    g = O.rng_gumbel_row(7, 3, 1, 2, 5000)
    assert np.all(np.isfinite(g)) and g.dtype == np.float32
    # Gumbel(0,1): mean = Euler-Mascheroni constant, variance pi^2/6
    assert abs(float(g.mean()) - 0.5772) < 0.05
    assert abs(float(g.var()) - math.pi ** 2 / 6) < 0.15


# -------------------------------------------- temperature-1 verification
def test_temp1_certain_accept_and_certain_reject():
    r = np.random.default_rng(40)
    N, V = 5, 16
    for s in range(50):
        z = r.standard_normal((N, V))
        draft = r.integers(0, V, size=N - 1)
        zz = z.copy()
        zz[np.arange(N - 1), draft] += 1e4
        a, nxt, _, _ = O.verify_temp1(draft, zz, seed=s, step=0, seq=0)
        assert a == N - 1
        zz = z.copy()
        zz[0, draft[0]] -= 1e4
        a, nxt, _, _ = O.verify_temp1(draft, zz, seed=s, step=0, seq=0)
        assert a == 0 and nxt != draft[0]


def test_temp1_residual_never_returns_rejected_token():
    r = np.random.default_rng(41)
    z = r.standard_normal((3, 6))
    draft = np.array([2, 4])
    for s in range(400):
        a, nxt, _, _ = O.verify_temp1(draft, z, seed=s, step=1, seq=2)
        if a < 2:
            assert nxt != draft[a]


def test_temp1_first_token_is_lossless_chi_square():
    """The first committed token must follow softmax(z[0]) whatever the draft
    (the lossless guarantee, DFlash page, key contributions)."""
    r = np.random.default_rng(42)
    V, n = 8, 20000
    z = r.standard_normal((2, V)) * 1.2
    draft = np.array([int(np.argsort(z[0])[-2])])          # a plausible but not top draft
    counts = np.zeros(V)
    accepted = 0
    for s in range(n):
        a, nxt, _, _ = O.verify_temp1(draft, z, seed=s, step=0, seq=0)
        first = draft[0] if a >= 1 else nxt
        counts[first] += 1
        accepted += a >= 1
    p = scipy.special.softmax(z[0])
    chi2 = float(np.sum((counts - n * p) ** 2 / (n * p)))
    assert scipy.stats.chi2.sf(chi2, V - 1) > 1e-4
    # P(accept) = p(d_1)
    pd = p[draft[0]]
    assert abs(accepted / n - pd) < 5 * math.sqrt(pd * (1 - pd) / n)


# ----------------------------------- sampled drafts, general verification
def test_sampled_draft_follows_softmax_over_tau_chi_square():
    r = np.random.default_rng(50)
    V, n, tau = 6, 20000, 0.7
    z = r.standard_normal((1, V)).astype(np.float32).astype(np.float64)
    counts = np.zeros(V)
    for sd in range(n):
        d, _ = O.draft_sample(z, tau, seed=sd, step=3, seq=1)
        counts[d[0]] += 1
    q = scipy.special.softmax(z[0] / tau)
    chi2 = float(np.sum((counts - n * q) ** 2 / (n * q)))
    assert scipy.stats.chi2.sf(chi2, V - 1) > 1e-4


def test_sampled_draft_uses_its_own_noise_stream():
    # the draft's Gumbel noise (stream 2, all four words of each Philox block)
    # is not the verification's (stream 1, word 0 of one block per entry)
    g1 = O.rng_gumbel_row(7, 0, 0, 0, 64, stream=1)
    g2 = O.rng_gumbel_row_words(7, 0, 0, 0, 64, stream=2)
    assert not np.array_equal(g1, g2)
    z = np.zeros((1, 64))
    d, _ = O.draft_sample(z, 1.0, seed=7, step=0, seq=0)
    assert d[0] == int(np.argmax(g2))


def test_four_word_gumbel_noise_against_scalar_philox():
    # entry k is word k % 4 of the scalar generator's block at counter k // 4
    seed, step, seq, row, V = 11, 3, 5, 2, 22
    g = O.rng_gumbel_row_words(seed, step, seq, row, V, stream=2)
    for k in range(V):
        w = O.philox4x64_10((k // 4, row | (2 << 32), seq, step), (seed, 0))[k % 4]
        u = np.float32((float(w >> 41) + 0.5) * 2.0 ** -23)
        assert g[k] == np.float32(-np.log(-np.log(u))), k


def test_sampled_verify_with_one_hot_proposal_is_the_temp1_rule():
    r = np.random.default_rng(51)
    N, V = 5, 16
    for sd in range(300):
        z = r.standard_normal((N, V))
        draft = r.integers(0, V, N - 1)
        zq = np.zeros((N - 1, V))
        zq[np.arange(N - 1), draft] = 10.0   # q one-hot at tau = 1e-2: exp(-1000) == 0
        got = O.verify_sampled(draft, zq, 1e-2, z, seed=sd, step=2, seq=3)
        ref = O.verify_temp1(draft, z, seed=sd, step=2, seq=3)
        assert got[:3] == ref[:3], (sd, got[:3], ref[:3])


def test_sampled_verify_proposal_equal_to_target_accepts_everything():
    r = np.random.default_rng(52)
    N, V = 6, 12
    for sd in range(200):
        z = r.standard_normal((N, V))
        draft = r.integers(0, V, N - 1)
        a, nxt, com, _ = O.verify_sampled(draft, z[: N - 1], 1.0, z, seed=sd, step=0, seq=0)
        assert a == N - 1 and com == N
        key = z[N - 1].astype(np.float32) + O.rng_gumbel_row(sd, 0, 0, N - 1, V)
        assert nxt == int(np.argmax(key))


def test_sampled_verify_residual_only_where_target_exceeds_proposal():
    r = np.random.default_rng(53)
    N, V = 3, 10
    seen = 0
    for sd in range(400):
        z = r.standard_normal((N, V))
        zq = r.standard_normal((N - 1, V)) * 2.0
        draft = np.array([int(np.argmax(zq[0])), 0])
        a, nxt, _, info = O.verify_sampled(draft, zq, 1.0, z, seed=sd, step=0, seq=0)
        if a == 0:
            p = scipy.special.softmax(z[0])
            q = scipy.special.softmax(zq[0])
            assert p[nxt] > q[nxt]
            assert info["u"][0] * info["q"][0] >= info["p"][0]
            seen += 1
    assert seen > 50


def test_sampled_draft_and_verify_are_lossless_chi_square():
    """Draft d ~ q = softmax(zq / tau), verify against p = softmax(z[0]):
    the first committed token follows p whatever q (the lossless guarantee,
    DFlash page, key contributions), and P(accept) = sum_k min(p_k, q_k)."""
    r = np.random.default_rng(54)
    V, n, tau = 8, 20000, 0.8
    z = r.standard_normal((2, V)) * 1.2
    zq = (z[:1] + r.standard_normal((1, V))).astype(np.float32).astype(np.float64)
    counts = np.zeros(V)
    accepted = 0
    for sd in range(n):
        d, _ = O.draft_sample(zq, tau, seed=sd, step=1, seq=0)
        a, nxt, _, _ = O.verify_sampled(d, zq, tau, z, seed=sd, step=1, seq=0)
        counts[d[0] if a >= 1 else nxt] += 1
        accepted += a >= 1
    p = scipy.special.softmax(z[0])
    chi2 = float(np.sum((counts - n * p) ** 2 / (n * p)))
    assert scipy.stats.chi2.sf(chi2, V - 1) > 1e-4
    q = scipy.special.softmax(zq[0] / tau)
    pa = float(np.minimum(p, q).sum())
    assert abs(accepted / n - pa) < 5 * math.sqrt(pa * (1 - pa) / n)


# ---------------------------------------------- dual-pass drafting (D2SD)
def test_confidence_is_the_softmax_maximum():
    """Confidence = the largest softmax probability: scipy's softmax on random
    rows; 1/V on a flat row; 1 when one logit dominates by far."""
    r = np.random.default_rng(50)
    z = r.standard_normal((7, 33)) * 3
    assert np.allclose(O.draft_confidence(z), scipy.special.softmax(z, axis=1).max(axis=1), rtol=1e-12)
    assert np.allclose(O.draft_confidence(np.zeros((2, 40))), 1 / 40, rtol=1e-14)
    big = np.zeros((1, 10))
    big[0, 3] = 800.0
    assert O.draft_confidence(big)[0] == 1.0


def test_cut_points_brute_force_and_ties():
    # worked example: the three lowest confidences are 0.1 (position 5) and the
    # tie 0.2 at positions 2 and 3; returned in position order
    assert O.d2sd_cut_points([0.5, 0.2, 0.2, 0.9, 0.1], 3) == [2, 3, 5]
    # a tie at the boundary goes to the lower position
    assert O.d2sd_cut_points([0.3, 0.1, 0.3, 0.3], 2) == [1, 2]
    assert O.d2sd_cut_points([0.3, 0.1], 5) == [1, 2]
    r = np.random.default_rng(51)
    for _ in range(300):
        n = int(r.integers(1, 9))
        conf = r.integers(0, 4, size=n) / 4.0                      # many ties
        K = int(r.integers(0, 6))
        got = O.d2sd_cut_points(conf, K)
        k = min(K, n)
        # brute force: the chosen set has the smallest (conf, position) keys
        keys = sorted((conf[j], j + 1) for j in range(n))
        assert got == sorted(p for _, p in keys[:k])
        assert all(conf[g - 1] <= conf[j] for g in got for j in range(n) if j + 1 not in got)


def test_candidate_tokens_layout():
    # N = 8, cut at 3: anchor, d_1, d_2 kept, masks from position 3 on
    assert O.d2sd_candidate_tokens(7, [11, 12, 13, 14, 15, 16, 17], 3, 8, 99) == [7, 11, 12, 99, 99, 99, 99, 99]
    assert O.d2sd_candidate_tokens(7, [11, 12, 13], 1, 4, 99) == [7, 99, 99, 99]
    assert O.d2sd_candidate_tokens(7, [11, 12, 13], 4, 4, 99) == [7, 11, 12, 13]


def test_candidates_keep_the_prefix_and_cut_at_one_reproduces_the_first_draft():
    c = tiny_cfg(block_size=6)
    m = _model(c, tiny_weights(c, seed=52))
    cache, _ = _prefill(m, c, 7)
    out = O.d2sd_candidates(m, cache, 0, 5, K=5, storage=False)
    first = out["first"]["draft"]
    assert out["cuts"] == [1, 2, 3, 4, 5]                       # K >= N-1: every position
    assert np.array_equal(out["drafts"][0], first)
    for k, cp in enumerate(out["cuts"]):
        d = out["drafts"][k + 1]
        assert np.array_equal(d[:cp - 1], first[:cp - 1])        # the kept prefix
        assert np.array_equal(d[cp - 1:], out["second"][k]["draft"][cp - 1:])
    # cut at 1 re-drafts from [anchor, mask...]: the first pass itself
    assert np.array_equal(out["drafts"][1], first)
    assert np.array_equal(out["second"][0]["logits"], out["first"]["logits"])
    # a longer kept prefix changes what the second pass sees: its hidden
    # states differ from the first pass's from the first real token on
    assert not np.allclose(out["second"][2]["hidden"][-1][1:], out["first"]["hidden"][-1][1:])


def test_verify_multi_brute_force_and_ties():
    r = np.random.default_rng(53)
    for _ in range(300):
        C, N, V = int(r.integers(1, 5)), 5, 4
        z = r.integers(0, 3, size=(C, N, V)).astype(np.float64)
        t = [[int(np.argmax(row)) for row in zc] for zc in z]
        drafts = np.array([[t[ci][j] if r.random() < 0.7 else int(r.integers(0, V)) for j in range(N - 1)]
                           for ci in range(C)])
        a, nxt, commit, chosen = O.verify_greedy_multi(drafts, z)
        acc = [_brute_accept(list(drafts[ci]), t[ci]) for ci in range(C)]
        assert a == max(acc) and chosen == acc.index(max(acc))      # lowest index on ties
        assert nxt == t[chosen][a] and commit == a + 1
    # one candidate: plain greedy verification
    z = np.eye(5)[[1, 2, 3, 4, 0]] * 3.0
    assert O.verify_greedy_multi(np.array([[1, 2, 0, 4]]), z[None])[:3] == O.verify_greedy(np.array([1, 2, 0, 4]), z)


import scipy.stats  # noqa: E402  (used above)
