"""Dual-pass drafting (D2SD) on the GPU against the oracle: the first
draft's confidence, the cut points, the K re-anchored candidates of the
second pass, and the greedy verification of all candidates that keeps the
longest accept.

Parity bar (as for the single draft): confidences within 2e-2 (max-norm
relative); cut points exact unless the oracle's K-th and (K+1)-th lowest
confidences lie within that tolerance; candidate tokens exact where the
oracle's top-2 gap is >= 1e-2, and a re-anchored candidate is compared only
when its kept prefix matches the oracle's (else its second pass saw other
input tokens); multi-candidate verification bit-exact on the oracle's
candidates and the same logits."""
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


def run_d2sd(case, K):
    case.prefill()
    case.step_append()
    dev, Bn, N = case.dev, case.B, case.cfg["block_size"]
    drafts = torch.full((Bn, K + 1, N - 1), -1, dtype=torch.int32, device=dev)
    conf = torch.zeros((Bn, N - 1), dtype=torch.float32, device=dev)
    cuts = torch.full((Bn, K), -1, dtype=torch.int32, device=dev)
    case.dr.d2sd_draft(case.t_i32(case.seq_ids), case.t_i32(case.anchor), K, drafts, conf, cuts)
    torch.cuda.synchronize()
    assert case.dr.read_error() == 0
    g = dict(drafts=drafts.cpu().numpy(), conf=conf.cpu().numpy(), cuts=cuts.cpu().numpy())
    orc = [O.d2sd_candidates(case.model, case.cache, case.seq_ids[b], int(case.anchor[b]), K)
           for b in range(Bn)]
    compared = excluded = 0
    for b, o in enumerate(orc):
        assert rel_err(g["conf"][b], o["conf"]) <= FLOAT_TOL, (b, g["conf"][b], o["conf"])
        srt = np.sort(o["conf"])
        stable = K >= len(srt) or srt[K] - srt[K - 1] > FLOAT_TOL * float(np.max(o["conf"]))
        first = o["first"]
        for j in range(N - 1):  # candidate 0: the first draft
            if first["gap"][j] < GAP_MIN:
                excluded += 1
                continue
            compared += 1
            assert g["drafts"][b, 0, j] == first["draft"][j], (b, j, g["drafts"][b, 0], first["draft"])
        if not stable:
            excluded += K
            continue
        assert list(g["cuts"][b]) == o["cuts"], (b, g["cuts"][b], o["cuts"], o["conf"])
        for k, cp in enumerate(o["cuts"]):
            gd = g["drafts"][b, k + 1]
            assert np.array_equal(gd[:cp - 1], g["drafts"][b, 0, :cp - 1])  # the kept prefix, exactly
            if not np.array_equal(g["drafts"][b, 0, :cp - 1], first["draft"][:cp - 1]):
                excluded += 1
                continue
            sec = o["second"][k]
            for j in range(cp - 1, N - 1):
                if sec["gap"][j] < GAP_MIN:
                    excluded += 1
                    continue
                compared += 1
                assert gd[j] == o["drafts"][k + 1][j], (b, k, cp, j, gd, o["drafts"][k + 1])
    say(f"  candidates: compared {compared} positions, excluded {excluded}")
    assert compared > excluded
    return g, orc


def check_verify_multi(case, orc, K):
    """The oracle's candidates against synthetic logits for every candidate
    block: GPU and oracle pick the same candidate, accept length and next token."""
    cfg, dev, Bn = case.cfg, case.dev, case.B
    C = K + 1
    d_or = np.stack([o["drafts"] for o in orc]).astype(np.int32)           # [B, C, N-1]
    z = synth.make_logits(cfg, d_or.reshape(Bn * C, -1), case.seed + 1)     # [B*C, N, V]
    if z.dtype == np.float32:
        zt = torch.from_numpy(z).to(dev)
        zf = z.astype(np.float64)
    else:
        zt = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
        zf = O.bf16_bits_to_f64(z)
    zt = zt.view(Bn, C, cfg["block_size"], -1)                              # [B, C, N, V]
    acc, nxt, com, cho = (torch.full((Bn,), -1, dtype=torch.int32, device=dev) for _ in range(4))
    case.dr.verify_multi(case.t_i32(case.seq_ids), torch.from_numpy(d_or).to(dev), zt, acc, nxt, com, cho)
    torch.cuda.synchronize()
    zf = zf.reshape(Bn, C, cfg["block_size"], -1)
    for b in range(Bn):
        exp = O.verify_greedy_multi(d_or[b], zf[b])
        got = (int(acc[b]), int(nxt[b]), int(com[b]), int(cho[b]))
        assert got == exp, (b, got, exp)
    say(f"  verify: accept {acc.tolist()} chosen {cho.tolist()}")


def test_d2sd_tiny_batch():
    cfg = small_cfg()
    K = 3
    case = Case(cfg, ctx=[60, 133, 21], n_new=[8, 2, 5], seed=61, page_order="shuffled", prefill_chunk=40,
                max_batch=3 * (K + 1))
    _, orc = run_d2sd(case, K)
    check_verify_multi(case, orc, K)


def test_d2sd_gpt_oss_geometry_all_cuts():
    # d_h 64, GQA 8:1, block 16; K = N-1 cuts every position, so the second
    # pass runs 2 x 15 blocks over the same two contexts
    cfg = small_cfg(hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64, intermediate=512, vocab=4096,
                    n_target_layers=9, block_size=16)
    K = 15
    case = Case(cfg, ctx=[150, 77], n_new=[8, 3], seed=63, prefill_chunk=64, max_batch=2 * (K + 1))
    _, orc = run_d2sd(case, K)
    check_verify_multi(case, orc, K)


def test_d2sd_gpt_oss_geometry_long_contexts_ring():
    # d_h 64, GQA 8:1, block 16, K = 3: the second pass runs 4 candidate
    # blocks per sequence. A pool of 2000 pages per sequence makes its
    # chunk grid (2 sequences x 4 candidates x 2 kv heads x 251 chunks)
    # about 8 times the attention's 512 work items: items of 8 chunks
    # through the persistent DMA ring, whose per-XCD list keeps the 4
    # candidates of an item together (the first pass: items of 2 chunks).
    # Contexts after the append: 1508 (a full item of 1024 keys and a
    # partial one of 4 chunks) and 603 (one partial item of 5 chunks).
    cfg = small_cfg(hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64, intermediate=512, vocab=4096,
                    n_target_layers=9, block_size=16)
    K = 3
    ctx = [1500, 600]
    pps_min = (max(ctx) + 16 + 15) // 16
    case = Case(cfg, ctx=ctx, n_new=[8, 3], seed=69, page_order="shuffled", prefill_chunk=256,
                extra_pages=2000 - pps_min, max_batch=2 * (K + 1))
    _, orc = run_d2sd(case, K)
    check_verify_multi(case, orc, K)


def test_d2sd_head_dim_128_shared_context_multi_chunk():
    # d_h 128, GQA 4:1, block 16: 64 query rows (4 computing waves) per kv
    # head, so one 8-wave attention workgroup takes 2 candidates of a
    # sequence (K = 6: 3 splits). The page pool (120 pages per sequence)
    # makes the second pass's chunk grid (2 sequences x 3 splits x 8 kv heads
    # x 16 chunks = 768) exceed the target of 512 work items, so items take 2
    # chunks each: item 0 (block page) per candidate, then the 700-token
    # context's shared items of 2 and 2 partial chunks.
    cfg = small_cfg(hidden=512, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=512, vocab=4096,
                    n_target_layers=3, block_size=16)
    K = 6
    ctx = [700, 150]
    pps_min = (max(ctx) + 16 + 15) // 16
    case = Case(cfg, ctx=ctx, n_new=[8, 3], seed=67, page_order="shuffled", prefill_chunk=128,
                extra_pages=120 - pps_min, max_batch=2 * (K + 1))
    _, orc = run_d2sd(case, K)
    check_verify_multi(case, orc, K)


def test_d2sd_rejects_bad_arguments_and_times_its_kernels():
    cfg = small_cfg()
    case = Case(cfg, ctx=[30], n_new=[4], seed=65, prefill_chunk=32, max_batch=3)
    case.prefill()
    case.step_append()
    dev, N = case.dev, cfg["block_size"]
    seq, anchor = case.t_i32(case.seq_ids), case.t_i32(case.anchor)
    d = torch.zeros((1, 5, N - 1), dtype=torch.int32, device=dev)
    with pytest.raises(B.DFlashError, match="max_batch"):
        case.dr.d2sd_draft(seq, anchor, 4, d)          # 4 second-pass blocks > max_batch 3
    with pytest.raises(B.DFlashError, match="K=0"):
        case.dr.d2sd_draft(seq, anchor, 0, torch.zeros((1, 1, N - 1), dtype=torch.int32, device=dev))
    logits = torch.zeros((1, 4, N, cfg["vocab"]), dtype=torch.float32, device=dev)
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(B.DFlashError, match="max_batch"):
        case.dr.verify_multi(seq, torch.zeros((1, 4, N - 1), dtype=torch.int32, device=dev), logits, one, one)
    h = case.dr.handle
    B.check(B.dflash_kernel_timer(h, B.K_D2SD, 1), "timer")
    d2 = torch.zeros((1, 3, N - 1), dtype=torch.int32, device=dev)
    case.dr.d2sd_draft(seq, anchor, 2, d2)
    torch.cuda.synchronize()
    rc, ms, n = B.dflash_kernel_timer_read(h, B.K_D2SD)
    B.check(rc, "timer read")
    assert n == 2 and ms > 0
    assert case.dr.read_error() == 0
