"""GPU parity of the HIP path against the oracle, through the C ABI.

Every case: seeded inputs -> prefill (several append calls) -> one decode
step (append, draft, verify) on both sides; the bar is stated in _cases.py.
Sizes span several tiles of every kernel and end on ragged tails (context
lengths that are not multiples of the page, chunk or tile sizes; batch
entries with zero appended rows; shuffled page tables).
"""
import numpy as np
import pytest
import torch

import oracle as O
from _cases import Case, FLOAT_TOL, say, nan_free, check_positions
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


def run_step(case, verify=True, check_cache=True, positions=0):
    """positions > 0: the oracle's drafts must hold at least that many
    distinct decided tokens per sequence, and every GPU logits row must sit
    closest to its own oracle row (check_positions)."""
    case.prefill()
    case.step_append()
    assert case.dr.read_error() == 0
    g = case.draft(dbg=True)
    orc = case.oracle_draft()
    assert nan_free(g["hidden"], g["logits"], g["gap"])
    he, le, n_cmp, n_exc = case.compare_draft(g, orc)
    ce = case.check_cache() if check_cache else 0.0
    say(f"  cache rel {ce:.2e}  hidden rel {he:.2e}  logits rel {le:.2e}  draft compared {n_cmp} excluded {n_exc}")
    assert ce <= FLOAT_TOL and he <= FLOAT_TOL and le <= FLOAT_TOL
    assert n_cmp > 0
    assert case.dr.read_error() == 0
    if positions:
        fewest = check_positions(g, orc, case.oracle_seqs, positions)
        say(f"  per-position drafts: {[list(map(int, o['draft'])) for o in orc]} (>= {fewest} distinct)")
    if verify:
        check_verify_greedy(case, orc)
    return g, orc


def check_verify_greedy(case, orc):
    cfg = case.cfg
    assert case.oracle_seqs == list(range(case.B))
    d_or = np.stack([o["draft"] for o in orc]).astype(np.int32)
    z = synth.make_logits(cfg, d_or, case.seed)
    dev = case.dev
    if z.dtype == np.float32:
        zt = torch.from_numpy(z).to(dev)
        zf = z.astype(np.float64)
    else:
        zt = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
        zf = O.bf16_bits_to_f64(z)
    acc = torch.full((case.B,), -1, dtype=torch.int32, device=dev)
    nxt = torch.full((case.B,), -1, dtype=torch.int32, device=dev)
    com = torch.full((case.B,), -1, dtype=torch.int32, device=dev)
    case.dr.verify(case.t_i32(case.seq_ids), torch.from_numpy(d_or).to(dev), zt, acc, nxt, com)
    torch.cuda.synchronize()
    for b in range(case.B):
        a, n, c = O.verify_greedy(d_or[b], zf[b])
        assert (int(acc[b]), int(nxt[b]), int(com[b])) == (a, n, c), b
    say(f"  verify accept {acc.tolist()} next {nxt.tolist()}")


# ------------------------------------------------------------ small shapes
def test_tiny_single_sequence():
    run_step(Case(synth.config("tiny"), ctx=[128], n_new=[8], prefill_chunk=40))


def test_tiny_ragged_batch_shuffled_pages():
    # M = 24 draft rows (two 16-row MFMA tiles, ragged), one sequence with no
    # appended rows, one with an empty context before the step, shuffled pages
    run_step(Case(synth.config("tiny"), ctx=[37, 133, 301, 5], n_new=[1, 8, 0, 5], seed=3,
                  page_order="shuffled", prefill_chunk=48))


# Parity inputs whose drafts differ from position to position: the query and
# key projections drawn so that attention logits have variance 2.5 (as std
# 0.02 gives at H = 4096), see synth.make_weights. Every case asserts at
# least 3 distinct decided tokens per sequence and row identity.
SHARP = dict(qk_score_var=2.5)


def test_tiny_diverse_drafts():
    cfg = synth.config("tiny", **SHARP)
    run_step(Case(cfg, ctx=[128], n_new=[8], prefill_chunk=40), positions=3)


def test_diverse_ragged_batch_shuffled_pages():
    cfg = synth.config("tiny", **SHARP)
    run_step(Case(cfg, ctx=[37, 133, 301, 5], n_new=[1, 8, 0, 5], seed=3, page_order="shuffled",
                  prefill_chunk=48), positions=3)


def test_diverse_head_dim_128_block_16():
    # the Qwen3 attention geometry (d_h 128, GQA 4:1, N 16) at a small width
    cfg = small_cfg(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024,
                    vocab=8192, n_target_layers=5, block_size=16, **SHARP)
    run_step(Case(cfg, ctx=[200, 257], n_new=[8, 3], seed=7, page_order="shuffled", prefill_chunk=64),
             positions=3)


def test_diverse_gqa_8_to_1_multi_chunk():
    # GPT-OSS attention geometry (d_h 64, GQA 8:1) with multi-chunk work
    # items (the page pool of test_attention_multi_chunk_items)
    cfg = small_cfg(hidden=512, n_q_heads=64, n_kv_heads=8, head_dim=64, intermediate=512, vocab=2048,
                    block_size=16, **SHARP)
    ctx, n_new = [1200, 383], [8, 5]
    pps_min = (max(ctx) + 16 + 15) // 16
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=51, page_order="shuffled", prefill_chunk=256,
                  extra_pages=300 - pps_min), positions=3)


def test_diverse_persistent_ring():
    # d_h 128, GQA 4:1, block 16 with 8-chunk attention items through the
    # persistent ring (560 pages per sequence); contexts after the append
    # 1024 (a full item), 2049 (two full items and a 1-key partial one) and
    # 1023 (one partial item of 8 chunks)
    cfg = small_cfg(hidden=512, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=512, vocab=4096,
                    block_size=16, **SHARP)
    ctx, n_new = [1016, 2041, 1023], [8, 8, 0]
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=81, page_order="shuffled", prefill_chunk=512,
                  extra_pages=560 - (max(ctx) + 16 + 15) // 16), positions=3)


def test_diverse_fc_fusion_tied():
    cfg = small_cfg(fusion="fc", tied_kv=1, n_target_layers=5, block_size=16, n_q_heads=8, n_kv_heads=2,
                    **SHARP)
    run_step(Case(cfg, ctx=[200, 97], n_new=[16, 3], seed=73, prefill_chunk=80), positions=3)


def test_tiny_tied_kv_without_rope():
    cfg = small_cfg(tied_kv=1, use_rope=0)
    case = Case(cfg, ctx=[70], n_new=[6], seed=5, prefill_chunk=32)
    g, orc = run_step(case)
    # without RoPE, identical mask tokens give identical rows in every layer
    hid = g["hidden"][:, 0]
    assert np.array_equal(hid[:, 2:], np.broadcast_to(hid[:, 1:2], hid[:, 2:].shape))


def test_head_dim_128_block_16():
    # the Qwen3 attention geometry (d_h 128, GQA 4:1, N 16) at a small width
    cfg = small_cfg(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024,
                    vocab=8192, n_target_layers=5, block_size=16)
    run_step(Case(cfg, ctx=[200, 257], n_new=[8, 3], seed=7, page_order="shuffled", prefill_chunk=64))


def test_gqa_8_to_1_head_dim_64():
    # the GPT-OSS attention geometry (d_h 64, GQA 8:1 -> 128 query rows per kv head)
    cfg = small_cfg(hidden=640, n_q_heads=16, n_kv_heads=2, head_dim=64, intermediate=640,
                    vocab=4096 + 96, n_target_layers=9, block_size=16)
    run_step(Case(cfg, ctx=[150], n_new=[8], seed=9, prefill_chunk=72))


def test_gqa_16_to_1_rows_256_both_head_dims():
    # 256 query rows per kv head: the attention's one-wave-per-row-group
    # variant (16 computing waves), for d_h 64 and 128; contexts end inside
    # and at the edge of a 128-key chunk; an empty context attends to the
    # block alone
    for d, ctx, n_new in ((64, [200, 112], [8, 3]), (128, [241, 0], [8, 0])):
        cfg = small_cfg(hidden=256, n_q_heads=16, n_kv_heads=1, head_dim=d, intermediate=512,
                        vocab=2048, block_size=16)
        run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=17 + d, page_order="shuffled", prefill_chunk=64))


def test_context_fills_every_page():
    # Page table exactly full: the step's 16 appended rows land in the last
    # page of sequence 0 (368 = 23 pages), whose 16 + 368 virtual keys end
    # exactly on the third 128-key chunk, the last slot of the attention's
    # chunk grid; sequence 1's 112 context keys plus the block fill exactly
    # one chunk.
    cfg = small_cfg(hidden=384, n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=768,
                    vocab=2048 + 32, n_target_layers=4, block_size=16)
    case = Case(cfg, ctx=[368, 112], n_new=[16, 16], seed=61, page_order="shuffled", prefill_chunk=64,
                extra_pages=-1)
    assert case.dr.pages_per_seq * 16 == 368
    run_step(case)
    assert int(case.dr.ctx_len[case.seq_ids[0]]) == 368


def test_attention_multi_chunk_items():
    # GPT-OSS attention geometry (d_h 64, 8 kv heads, 128 query rows per kv
    # head) with a page pool (300 pages per sequence) whose chunk grid
    # (4 x 8 x 38 = 1216) is between 2 and 3 times the attention's target of
    # 512 work items: every work item then takes 4 chunks of 128 keys in a
    # row (the count is rounded up to 1, 2, 4 or 8), 512 keys, through the
    # direct-to-LDS ring when it has all 4, else staged through registers.
    # Context lengths after the append: 1208 (items of 512, 512 and 184
    # keys: two chunks), 388 (one item whose fourth chunk holds 4 keys),
    # 0 (the block alone) and 2333 (5 items, the last with 285 keys).
    cfg = small_cfg(hidden=512, n_q_heads=64, n_kv_heads=8, head_dim=64, intermediate=512, vocab=2048,
                    block_size=16)
    ctx, n_new = [1200, 383, 0, 2317], [8, 5, 0, 16]
    pps_min = (max(ctx) + 16 + 15) // 16
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=51, page_order="shuffled", prefill_chunk=256,
                  extra_pages=300 - pps_min))


@pytest.mark.parametrize("head_dim,n_q", [(128, 32), (64, 64), (128, 64)])
def test_attention_ring_eight_chunks(head_dim, n_q):
    # A page pool of 2000 pages per sequence makes the chunk grid (2 x 8 x
    # 251 = 4016) about 8 times the attention's 512 work items: items of 8
    # chunks (1024 keys) through the persistent direct-to-LDS ring (d_h 128,
    # GQA 4:1: two key groups per item; GQA 8:1 at d_h 64 and 128: one).
    # Contexts after the append: 2508 (full items of 1024 and 1024 keys,
    # then a partial item of 460 keys in 4 chunks) and 1000 (one partial
    # item of 8 chunks whose last holds 104 keys: its invalid V slots are
    # zeroed in LDS); the last page of each sequence is partly filled.
    cfg = small_cfg(hidden=512, n_q_heads=n_q, n_kv_heads=8, head_dim=head_dim, intermediate=512, vocab=2048,
                    block_size=16)
    ctx, n_new = [2500, 1000], [8, 0]
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=58, page_order="shuffled", prefill_chunk=512,
                  extra_pages=2000 - (max(ctx) + 16 + 15) // 16))


def test_attention_persistent_ring_list_edges():
    # d_h 128, GQA 4:1, items of 8 chunks with two key groups: the
    # persistent ring kernel, whose per-XCD work lists order full items,
    # then partial last items (most chunks first), then block items.
    # Contexts after the append: 1024 (one full item, no partial one), 0
    # (the block item alone), 2049 (two full items and a 1-key partial
    # item) and 1023 (one partial item of 8 chunks, its last holding 127
    # keys); 560 pages per sequence give 71 chunk slots per (sequence, kv
    # head), 2272 chunks in all: 8 chunks per item.
    cfg = small_cfg(hidden=512, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=512, vocab=2048,
                    block_size=16)
    ctx, n_new = [1016, 0, 2041, 1023], [8, 0, 8, 0]
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=59, page_order="shuffled", prefill_chunk=512,
                  extra_pages=560 - (max(ctx) + 16 + 15) // 16))


def test_long_context_multi_chunk_head_dim_128():
    # One sequence at 32000 tokens with the Qwen3 attention geometry (d_h
    # 128, GQA 4:1, block 16) at a small width: the chunk grid (8 kv heads x
    # 251 chunks) is about 4 times the attention's target of 512 work items,
    # so every item streams 4 chunks (512 virtual keys) with the online
    # softmax, 63 items, the last one 272 keys long.
    cfg = small_cfg(hidden=512, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=512, vocab=4096,
                    n_target_layers=3, block_size=16)
    case = Case(cfg, ctx=[32000], n_new=[8], seed=57, page_order="shuffled", prefill_chunk=1024)
    assert case.dr.pages_per_seq == 2002
    run_step(case)


def test_fc_fusion_ragged_batch():
    # DFlash's FC fusion: one shared context from W_fc [H, T*H] for every
    # layer; ragged appends (one entry appends nothing), shuffled pages
    cfg = small_cfg(fusion="fc")
    run_step(Case(cfg, ctx=[70, 9, 131], n_new=[8, 0, 5], seed=71, page_order="shuffled", prefill_chunk=40))


def test_fc_fusion_tied_many_rows():
    # FC fusion with tied context/block K/V (DFlash's shared projection),
    # T = 5, appends of 2 x 80 rows: the FC layer and the context K/V run on
    # the tiled GEMM, with a partial last row tile
    cfg = small_cfg(fusion="fc", tied_kv=1, n_target_layers=5, block_size=16, n_q_heads=8, n_kv_heads=2)
    run_step(Case(cfg, ctx=[200, 97], n_new=[16, 3], seed=73, prefill_chunk=80))


def test_wide_batch_multi_group_rows():
    # M = 5 * 16 = 80 rows -> several 64-row groups in the projection kernels
    cfg = small_cfg(hidden=256, block_size=16, n_q_heads=4, n_kv_heads=4)
    run_step(Case(cfg, ctx=[40, 41, 96, 0, 129], n_new=[8, 0, 16, 0, 9], seed=11,
                  page_order="shuffled", prefill_chunk=80))


def test_many_rows_tiled_gemm_tails():
    # 19 sequences x 8 block rows = 152 rows: the tiled MFMA GEMMs and LM
    # head, with a partial last row tile in a second row block, odd numbers
    # of k steps, column blocks that end inside a segment and a vocabulary
    # of 250 tiles; the 24-row prefill chunks take the same kernels for the
    # context K/V. Hidden 352 (11 k steps) keeps every product in one k
    # split except the down projection (23 steps, 2 splits); hidden 544 (17
    # steps) also splits the QKV and gate/up projections; the SwiGLU then
    # runs in its own kernel over the summed splits.
    for hidden, inter, seed in ((352, 736, 41), (544, 608, 43)):
        cfg = small_cfg(hidden=hidden, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=inter, vocab=4000,
                        block_size=8)
        rng = np.random.default_rng(seed)
        n_new = rng.integers(0, 9, size=19)
        ctx = n_new + rng.integers(0, 70, size=19)
        run_step(Case(cfg, ctx=ctx.tolist(), n_new=n_new.tolist(), seed=seed, page_order="shuffled",
                      prefill_chunk=24))


def test_deterministic_bitwise():
    case = Case(synth.config("tiny"), ctx=[99], n_new=[8], seed=13, prefill_chunk=50)
    case.prefill()
    case.step_append()
    g1 = case.draft(dbg=True)
    g2 = case.draft(dbg=True)
    for k in ("draft", "gap", "hidden", "logits"):
        assert np.array_equal(g1[k].view(np.uint32) if g1[k].dtype == np.float32 else g1[k],
                              g2[k].view(np.uint32) if g2[k].dtype == np.float32 else g2[k]), k


# ------------------------------------------------------- verification only
def verify_only_drafter(V, N, batch):
    """A one-layer drafter with the given vocabulary and block: only its
    verify entry point is used (verification reads no weights)."""
    from block_diffusion_drafter_softmax_amd.drafter import Drafter
    G = 16 // np.gcd(16, N)  # query rows per kv head, G * N, must fill 16-row tiles
    cfg = small_cfg(vocab=V, hidden=256, n_layers=1, intermediate=256, block_size=N,
                    n_q_heads=2 * G, n_kv_heads=2)
    return Drafter(cfg, synth.make_weights(cfg, 0), max_batch=batch, max_new=1, max_seqs=batch + 3,
                   pages_per_seq=2)


def test_verify_greedy_full_vocab_bf16():
    cfg = synth.config("qwen3_8b")
    B_, N, V = 4, cfg["block_size"], cfg["vocab"]
    rng = np.random.default_rng(21)
    draft = rng.integers(0, V - 1, size=(B_, N - 1)).astype(np.int32)
    z = synth.make_logits(cfg, draft, seed=21)
    dev = torch.device("cuda")
    dr = verify_only_drafter(V, N, B_)
    zt = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
    acc, nxt, com = (torch.full((B_,), -1, dtype=torch.int32, device=dev) for _ in range(3))
    seq = torch.arange(B_, dtype=torch.int32, device=dev)
    dr.verify(seq, torch.from_numpy(draft).to(dev), zt, acc, nxt, com)
    torch.cuda.synchronize()
    zf = O.bf16_bits_to_f64(z)
    for b in range(B_):
        assert (int(acc[b]), int(nxt[b]), int(com[b])) == O.verify_greedy(draft[b], zf[b]), b
    say(f"  accept {acc.tolist()}")


def test_verify_temperature_one_batched():
    cfg = synth.config("qwen3_8b_batched")
    B_, N, V = cfg["batch"], cfg["block_size"], cfg["vocab"]
    rng = np.random.default_rng(22)
    draft = rng.integers(0, V - 1, size=(B_, N - 1)).astype(np.int32)
    z = synth.make_logits(cfg, draft, seed=22)
    dev = torch.device("cuda")
    dr = verify_only_drafter(V, N, B_)
    zt = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
    seq_np = np.arange(B_, dtype=np.int32) + 3
    seed, step = 1234567, 42
    acc, nxt, com = (torch.full((B_,), -1, dtype=torch.int32, device=dev) for _ in range(3))
    dr.verify(torch.from_numpy(seq_np).to(dev), torch.from_numpy(draft).to(dev), zt, acc, nxt, com,
              temperature=1.0, seed=seed, step=step)
    torch.cuda.synchronize()
    zf = O.bf16_bits_to_f64(z)
    compared_a = compared_n = 0
    for b in range(B_):
        a, n, c, info = O.verify_temp1(draft[b], zf[b], seed, step, int(seq_np[b]))
        if any(abs(u - p) < 1e-5 for u, p in zip(info["u"], info["p"])):
            continue
        compared_a += 1
        assert int(acc[b]) == a and int(com[b]) == c, (b, int(acc[b]), a)
        if info["gumbel_gap"] >= 1e-2:
            compared_n += 1
            assert int(nxt[b]) == n, (b, int(nxt[b]), n)
        if a < N - 1:
            assert int(nxt[b]) != int(draft[b, a])
    say(f"  accept {acc.tolist()}  compared {compared_a}/{B_} accept, {compared_n} next")
    assert compared_a >= B_ - 2 and compared_n >= B_ - 4


def test_verify_temperature_one_fp32_logits():
    """Temperature-1 verification of fp32 target logits (the tiny shape's
    logits dtype) against the oracle: a 4096 vocabulary at block 8 and the
    full 151936 vocabulary at block 16, logits with the draft token's
    probability set to 0.75 (no bf16 rounding)."""
    dev = torch.device("cuda")
    for V, N, B_, seed in ((4096, 8, 16, 23), (151936, 16, 8, 24)):
        cfg = small_cfg(vocab=V, block_size=N, logit_model="accept_p", agreement=0.75, logits_f32=True)
        rng = np.random.default_rng(seed)
        draft = rng.integers(0, V - 1, size=(B_, N - 1)).astype(np.int32)
        z = synth.make_logits(cfg, draft, seed=seed)
        assert z.dtype == np.float32
        dr = verify_only_drafter(V, N, B_)
        seq_np = np.arange(B_, dtype=np.int32) + 2
        step = 7
        acc, nxt, com = (torch.full((B_,), -1, dtype=torch.int32, device=dev) for _ in range(3))
        dr.verify(torch.from_numpy(seq_np).to(dev), torch.from_numpy(draft).to(dev), torch.from_numpy(z).to(dev),
                  acc, nxt, com, temperature=1.0, seed=seed, step=step)
        torch.cuda.synchronize()
        compared_a = compared_n = 0
        for b in range(B_):
            a, n, c, info = O.verify_temp1(draft[b], z[b].astype(np.float64), seed, step, int(seq_np[b]))
            if any(abs(u - p) < 1e-5 for u, p in zip(info["u"], info["p"])):
                continue
            compared_a += 1
            assert int(acc[b]) == a and int(com[b]) == c, (V, b, int(acc[b]), a)
            if info["gumbel_gap"] >= 1e-2:
                compared_n += 1
                assert int(nxt[b]) == n, (V, b, int(nxt[b]), n)
            if a < N - 1:
                assert int(nxt[b]) != int(draft[b, a])
        say(f"  V {V}: accept {acc.tolist()}  compared {compared_a}/{B_} accept, {compared_n} next")
        assert compared_a >= B_ - 2 and compared_n >= B_ - 4
        assert len(set(acc.tolist())) >= 2  # accept lengths differ across the batch
        dr.close()


# ------------------------------------------------------ error word (host-forced)
def test_device_error_bits_and_skips():
    cfg = synth.config("tiny")
    case = Case(cfg, ctx=[20, 20], n_new=[4, 4], seed=31, prefill_chunk=16)
    case.prefill()
    dr = case.dr
    before = dr.ctx_len.clone()
    T, H = cfg["n_target_layers"], cfg["hidden"]
    hid = torch.zeros((2, 16, T, H), dtype=torch.bfloat16, device=case.dev)
    # n_new above the call's max_new: flagged, sequence untouched
    dr.ctx_append(case.t_i32(case.seq_ids), case.t_i32([17, 2]), hid, 16)
    err = dr.read_error()
    assert err & B.DEV_BAD_N_NEW
    assert int(dr.ctx_len[case.seq_ids[0]]) == int(before[case.seq_ids[0]])
    assert int(dr.ctx_len[case.seq_ids[1]]) == int(before[case.seq_ids[1]]) + 2
    # a page-table hole where the append lands
    pt = dr.page_table.clone()
    L0 = int(dr.ctx_len[case.seq_ids[0]])
    dr.page_table[case.seq_ids[0], L0 // 16] = -1
    dr.ctx_append(case.t_i32(case.seq_ids[:1]), case.t_i32([16]), hid[:1], 16)
    assert dr.read_error() & B.DEV_BAD_PAGE
    assert int(dr.ctx_len[case.seq_ids[0]]) == L0
    dr.page_table.copy_(pt)
    # out-of-range anchor and sequence id are flagged; kernels stay in bounds
    draft = torch.zeros((2, cfg["block_size"] - 1), dtype=torch.int32, device=case.dev)
    dr.draft_block(case.t_i32([case.seq_ids[0], 10 ** 6]), case.t_i32([cfg["vocab"], 0]), draft)
    err = dr.read_error()
    assert err & B.DEV_BAD_TOKEN and err & B.DEV_BAD_SEQ
    # a hole in an already appended context page, seen by the draft: the
    # attention flags it and clamps the entry, so every access stays in
    # bounds (the clamped page here is an unwritten, NaN-filled one: the
    # affected sequence's results are unspecified); the other sequence's
    # draft is untouched
    gap = torch.zeros((2, cfg["block_size"] - 1), dtype=torch.float32, device=case.dev)
    dr.draft_block(case.t_i32(case.seq_ids), case.t_i32([3, 4]), draft, gap)
    assert dr.read_error() == 0
    clean_draft, clean_gap = draft.clone(), gap.clone()
    dr.page_table[case.seq_ids[0], 0] = -1
    dr.draft_block(case.t_i32(case.seq_ids), case.t_i32([3, 4]), draft, gap)
    assert dr.read_error() & B.DEV_BAD_PAGE
    torch.cuda.synchronize()
    assert torch.equal(draft[1], clean_draft[1]) and torch.equal(gap[1], clean_gap[1])
    dr.page_table.copy_(pt)
    dr.draft_block(case.t_i32(case.seq_ids), case.t_i32([3, 4]), draft, gap)
    assert dr.read_error() == 0
    torch.cuda.synchronize()
    assert torch.equal(draft, clean_draft) and torch.equal(gap, clean_gap)
    # capacity: more rows than the sequence's pages hold
    dr.ctx_len[case.seq_ids[1]] = dr.pages_per_seq * 16 - 2
    dr.ctx_append(case.t_i32(case.seq_ids[1:]), case.t_i32([4]), hid[:1], 16)
    assert dr.read_error() & B.DEV_NO_PAGES
    assert int(dr.ctx_len[case.seq_ids[1]]) == dr.pages_per_seq * 16 - 2


def test_host_validation_enqueues_nothing():
    cfg = synth.config("tiny")
    case = Case(cfg, ctx=[16], n_new=[1], seed=33, prefill_chunk=16)
    dr = case.dr
    with pytest.raises(B.DFlashError):
        dr.verify(case.t_i32([1]), case.t_i32(np.zeros((1, 7))), torch.zeros((1, 8, cfg["vocab"]), device=case.dev),
                  case.t_i32([0]), case.t_i32([0]), temperature=0.5)
    assert "temperature" in B.last_error()
    hid = torch.zeros((1, 16, cfg["n_target_layers"], cfg["hidden"]), dtype=torch.bfloat16, device=case.dev)
    # straight through the C ABI (the binding would refuse the buffer's shape first)
    seq1, one = case.t_i32([1]), case.t_i32([1])
    rc = B.dflash_ctx_append(dr.handle, 1, seq1.data_ptr(), one.data_ptr(), hid.data_ptr(), 10 ** 4,
                             torch.cuda.current_stream().cuda_stream)
    assert rc < 0 and "max_new" in B.last_error()
    assert int(dr.ctx_len.sum()) == 0
    # the binding refuses tensors whose shape, dtype or device the library cannot check
    with pytest.raises(ValueError, match="hidden"):
        dr.ctx_append(seq1, one, hid[:, :8], 16)
    with pytest.raises(ValueError, match="draft"):
        dr.draft_block(seq1, one, torch.zeros((1, 3), dtype=torch.int32, device=case.dev))
    with pytest.raises(ValueError, match="logits"):
        dr.verify(seq1, case.t_i32(np.zeros((1, 7))), torch.zeros((1, 8, 100), device=case.dev), one, one)
    with pytest.raises(ValueError, match="device"):
        dr.verify(seq1, case.t_i32(np.zeros((1, 7))), torch.zeros((1, 8, cfg["vocab"])), one, one)
    assert int(dr.ctx_len.sum()) == 0
