"""Sampled drafts and their lossless verification on the GPU against the oracle.

* Drafting at temperature tau: the drafter's logits within 2e-2 (max-norm
  relative) of the oracle's; the sampled tokens exact where the oracle's
  Gumbel-key top-2 gap (on the oracle's logits) is >= 1e-2; and, on the
  GPU's own logits, the oracle's sampler picks the GPU's tokens wherever its
  key gap is >= 1e-3 (the same noise, float32 keys either side).
* Verification at target temperature 1 with the general proposal q: the
  same draft tokens, drafter logits and target logits on both sides; accept
  length, next token and commit exact, except decisions where
  |u q - p| < 1e-4 max(p, u q) or the sampled row's Gumbel top-2 gap is
  < 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle as O
from _cases import Case, FLOAT_TOL, GAP_MIN, rel_err, say
from block_diffusion_drafter_softmax_amd import synth
from block_diffusion_drafter_softmax_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def small_cfg(**kw):
    c = synth.config("tiny")
    c.update(kw)
    c["mask_token_id"] = c["vocab"] - 1
    return c


def _draft(case, tau, seed, step):
    cfg, dev = case.cfg, case.dev
    N, V = cfg["block_size"], cfg["vocab"]
    draft = torch.full((case.B, N - 1), -1, dtype=torch.int32, device=dev)
    logits = torch.zeros((case.B, N - 1, V), dtype=torch.float32, device=dev)
    case.dr.draft_sample(case.t_i32(case.seq_ids), case.t_i32(case.anchor), tau, draft, logits, seed=seed, step=step)
    torch.cuda.synchronize()
    assert case.dr.read_error() == 0
    return draft.cpu().numpy(), logits.cpu().numpy()


def check_sampled_draft(case, tau, seed, step, orc=None):
    d_gpu, z_gpu = _draft(case, tau, seed, step)
    orc = orc if orc is not None else case.oracle_draft()
    compared = own = 0
    for b, o in enumerate(orc):
        seq = case.seq_ids[b]
        assert rel_err(z_gpu[b], o["logits"]) <= FLOAT_TOL
        d_or, gap_or = O.draft_sample(o["logits"], tau, seed, step, seq)
        d_own, gap_own = O.draft_sample(z_gpu[b].astype(np.float64), tau, seed, step, seq)
        for j in range(len(d_or)):
            if gap_or[j] >= GAP_MIN:
                assert d_gpu[b, j] == d_or[j], (b, j, d_gpu[b], d_or, gap_or)
                compared += 1
            if gap_own[j] >= 1e-3:
                assert d_gpu[b, j] == d_own[j], (b, j, d_gpu[b], d_own, gap_own)
                own += 1
    say(f"  sampled draft tau {tau}: {compared} positions against the oracle, {own} on the GPU's logits")
    assert compared > 0 and own > 0
    return d_gpu, z_gpu, orc


def check_sampled_verify(case, draft, zq, tau, logits_f64, logits_dev, seeds):
    """Same inputs on both sides; returns (compared, excluded)."""
    dev, Bn = case.dev, case.B
    zq_dev = torch.from_numpy(np.ascontiguousarray(zq, dtype=np.float32)).to(dev)
    d_dev = torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).to(dev)
    compared = excluded = 0
    for seed, step in seeds:
        acc, nxt, com = (torch.full((Bn,), -1, dtype=torch.int32, device=dev) for _ in range(3))
        case.dr.verify_sample(case.t_i32(case.seq_ids), d_dev, zq_dev, tau, logits_dev, acc, nxt, com,
                              seed=seed, step=step)
        torch.cuda.synchronize()
        for b in range(Bn):
            a, n, c, info = O.verify_sampled(draft[b], zq[b], tau, logits_f64[b], seed, step, case.seq_ids[b])
            # relative margin: at a 152k vocabulary p and q are often ~1e-5
            near = any(abs(u * q - p) < 1e-4 * max(p, u * q) for u, q, p in zip(info["u"], info["q"], info["p"]))
            if near or info["gumbel_gap"] < GAP_MIN:
                excluded += 1
                continue
            assert (int(acc[b]), int(nxt[b]), int(com[b])) == (a, n, c), (seed, step, b, (int(acc[b]), int(nxt[b])),
                                                                         (a, n), info)
            compared += 1
    assert case.dr.read_error() == 0
    return compared, excluded


def test_sampled_draft_and_verify_tiny_batch():
    cfg = small_cfg()
    case = Case(cfg, ctx=[66, 130, 17], n_new=[8, 4, 0], seed=91, page_order="shuffled", prefill_chunk=48)
    case.prefill()
    case.step_append()
    for tau in (0.6, 1.3):
        d_gpu, z_gpu, orc = check_sampled_draft(case, tau, seed=11, step=4)
    # verification: the oracle's draft and logits (f32 values), synthetic fp32 target logits
    zq = np.stack([o["logits"] for o in orc])
    draft, _ = zip(*[O.draft_sample(o["logits"], 1.3, 11, 4, case.seq_ids[b]) for b, o in enumerate(orc)])
    draft = np.stack(draft)
    z = synth.make_logits(cfg, draft, 91)                                  # [B, N, V] fp32
    comp, exc = check_sampled_verify(case, draft, zq, 1.3, z.astype(np.float64), torch.from_numpy(z).to(case.dev),
                                     [(s, t) for s in range(12) for t in (0, 7)])
    say(f"  sampled verify: compared {comp}, excluded {exc}")
    assert comp >= 40


def test_sampled_full_vocab_bf16_target():
    # head_dim 128, block 16, the Qwen3 vocabulary (151936: 19 sampling and
    # 5 verification chunks per row), bf16 target logits with agreement
    cfg = small_cfg(hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=256, vocab=151936,
                    block_size=16, logit_model="top_plus1", agreement=0.8)
    case = Case(cfg, ctx=[150, 40], n_new=[8, 8], seed=93, prefill_chunk=64)
    case.prefill()
    case.step_append()
    d_gpu, z_gpu, orc = check_sampled_draft(case, 0.9, seed=3, step=1)
    zq = np.stack([o["logits"] for o in orc])
    draft = np.stack([O.draft_sample(o["logits"], 0.9, 3, 1, case.seq_ids[b])[0] for b, o in enumerate(orc)])
    bits = synth.make_logits(cfg, draft, 93)
    logits_dev = torch.from_numpy(bits.view(np.int16)).to(case.dev).view(torch.bfloat16)
    comp, exc = check_sampled_verify(case, draft, zq, 0.9, O.bf16_bits_to_f64(bits), logits_dev,
                                     [(s, 2) for s in range(10)])
    say(f"  sampled verify: compared {comp}, excluded {exc}")
    assert comp >= 12


def test_sampled_rejects_bad_arguments():
    cfg = small_cfg()
    case = Case(cfg, ctx=[20], n_new=[4], seed=95, prefill_chunk=32)
    case.prefill()
    case.step_append()
    dev, N, V = case.dev, cfg["block_size"], cfg["vocab"]
    seq, anchor = case.t_i32(case.seq_ids), case.t_i32(case.anchor)
    d = torch.zeros((1, N - 1), dtype=torch.int32, device=dev)
    zl = torch.zeros((1, N - 1, V), dtype=torch.float32, device=dev)
    with pytest.raises(B.DFlashError, match="temperature"):
        case.dr.draft_sample(seq, anchor, 0.0, d, zl)
    with pytest.raises(B.DFlashError, match="reciprocal"):  # subnormal: 1 / tau overflows fp32
        case.dr.draft_sample(seq, anchor, 1e-40, d, zl)
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    tl = torch.zeros((1, N, V), dtype=torch.float32, device=dev)
    with pytest.raises(B.DFlashError, match="draft_temperature"):
        case.dr.verify_sample(seq, d, zl, float("inf"), tl, one, one)
    assert case.dr.read_error() == 0
