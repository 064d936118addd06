"""GPU parity at the full drafter shapes, in the launch configuration the
benchmark times (one decode step after a prefill), against the oracle.

* Qwen3-8B-shaped DFLARE drafter (T=9, 7 layers, context 4096, block 16,
  batch 1, 8 appended rows, greedy verify): every output; then drafts
  sampled at temperature 1 and their lossless verification.
* Qwen3-4B-shaped DFlash-style drafter (tied context/block K/V, T=5,
  context 2048): every output; the same with DFlash's FC fusion.
* GPT-OSS-20B-shaped drafter (d_h 64, GQA 8:1, V 201088, batch 8, context
  8192): the whole batch runs on the GPU, the oracle reproduces two of the
  eight sequences (sequences never interact).
* Batched Qwen3-8B serving shape (32 sequences, ragged contexts drawn from
  [512, 8192], ragged appends, shuffled pages): the whole batch on the GPU,
  the oracle reproduces the two shortest sequences.
"""
import numpy as np
import pytest
import torch

import oracle as O
from _cases import Case, FLOAT_TOL, say, nan_free, check_positions
from block_diffusion_drafter_softmax_amd import synth
from test_gpu_parity import check_verify_greedy

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def full_step(case, verify=True, positions=0):
    case.prefill()
    case.step_append()
    assert case.dr.read_error() == 0
    g = case.draft(dbg=True)
    say("  oracle draft ...")
    orc = case.oracle_draft()
    assert nan_free(g["hidden"], g["logits"], g["gap"])
    he, le, n_cmp, n_exc = case.compare_draft(g, orc)
    ce = case.check_cache()
    say(f"  cache rel {ce:.2e}  hidden rel {he:.2e}  logits rel {le:.2e}  draft compared {n_cmp} excluded {n_exc}")
    assert ce <= FLOAT_TOL and he <= FLOAT_TOL and le <= FLOAT_TOL
    assert n_cmp >= n_exc
    if positions:  # the drafted tokens differ by block position (see check_positions)
        fewest = check_positions(g, orc, case.oracle_seqs, positions)
        say(f"  per-position drafts: {[list(map(int, o['draft'])) for o in orc]} (>= {fewest} distinct)")
    if verify:
        check_verify_greedy(case, orc)
    return g, orc


@pytest.mark.timeout(1200)
def test_qwen3_8b_full_step():
    cfg = synth.config("qwen3_8b")
    case = Case(cfg, ctx=[cfg["context"]], n_new=[cfg["n_new"]], prefill_chunk=512, seq_offset=0)
    # at this width std-0.02 projections already give attention logits of
    # variance ~2.7: the oracle's 15 drafted tokens differ by position
    _, orc = full_step(case, positions=3)
    # the same step with drafts sampled at temperature 1 and the lossless
    # verification, on the oracle's logits of this step
    from test_gpu_sampled import check_sampled_draft, check_sampled_verify
    check_sampled_draft(case, 1.0, seed=5, step=9, orc=orc)
    zq = np.stack([o["logits"] for o in orc])
    draft = np.stack([O.draft_sample(o["logits"], 1.0, 5, 9, case.seq_ids[b])[0] for b, o in enumerate(orc)])
    bits = synth.make_logits(cfg, draft, 7)
    logits_dev = torch.from_numpy(bits.view(np.int16)).to(case.dev).view(torch.bfloat16)
    comp, exc = check_sampled_verify(case, draft, zq, 1.0, O.bf16_bits_to_f64(bits), logits_dev,
                                     [(s, 9) for s in range(8)])
    say(f"  sampled verify: compared {comp}, excluded {exc}")
    assert comp >= 4


@pytest.mark.timeout(1200)
def test_qwen3_4b_tied_full_step():
    cfg = synth.config("qwen3_4b")
    assert cfg["tied_kv"] == 1
    full_step(Case(cfg, ctx=[cfg["context"]], n_new=[cfg["n_new"]], prefill_chunk=512, seq_offset=0), positions=3)


@pytest.mark.timeout(1200)
def test_qwen3_4b_fc_fusion_full_step():
    cfg = synth.config("qwen3_4b_fc")
    assert cfg["fusion"] == "fc" and cfg["tied_kv"] == 1
    full_step(Case(cfg, ctx=[cfg["context"]], n_new=[cfg["n_new"]], prefill_chunk=512, seq_offset=0), positions=3)


@pytest.mark.timeout(1200)
def test_gpt_oss_20b_batch8_sampled():
    cfg = synth.config("gpt_oss_20b")
    B = cfg["batch"]
    full_step(Case(cfg, ctx=[cfg["context"]] * B, n_new=[cfg["n_new"]] * B, prefill_chunk=512,
                   oracle_seqs=[0, 5]), verify=False, positions=3)


@pytest.mark.timeout(1200)
def test_qwen3_8b_batched_ragged_sampled():
    cfg = synth.config("qwen3_8b_batched")
    ctx = synth.context_lengths(cfg, 0)
    n_new = synth.appended_rows(cfg, 0)
    order = np.argsort(ctx)
    sample = [int(order[0]), int(order[1])]
    say(f"  contexts {ctx.min()}..{ctx.max()} (mean {ctx.mean():.0f}), appends {n_new.tolist()}, oracle on {sample}")
    full_step(Case(cfg, ctx=ctx, n_new=n_new, prefill_chunk=512, page_order="shuffled", oracle_seqs=sample),
              verify=False, positions=3)
