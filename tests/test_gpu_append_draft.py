"""dflash_append_draft gives, bit for bit, what dflash_ctx_append followed by
dflash_draft_block gives: the drafts, their top-2 gaps, the context lengths,
every context K/V page and the error word. Cases: a ragged batch (one
sequence appending nothing) on shuffled pages, a batch large enough for the
tiled GEMMs (128 block rows), one whose appended and block rows fill whole
XCD tiles, an append whose page check fails (the draft then sees the old
context) and an append with n_new above max_new."""
import numpy as np
import pytest
import torch

from _cases import Case, say
from block_diffusion_drafter_softmax_amd import synth
from block_diffusion_drafter_softmax_amd import _binding as B

pytestmark = pytest.mark.gpu


def small_cfg(**kw):
    c = synth.config("tiny")
    c.update(kw)
    c["mask_token_id"] = c["vocab"] - 1
    return c


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(case, n_new, max_new, hole=None):
    """Run append + draft and append_draft from the same state; return both
    results. hole: (sequence index, page index) set to -1 before both runs."""
    dr, dev, cfg = case.dr, case.dev, case.cfg
    N, T, H = cfg["block_size"], cfg["n_target_layers"], cfg["hidden"]
    buf = np.zeros((case.B, max_new, T, H), dtype=np.uint16)
    for b, r in enumerate(case.hidden_step):
        buf[b, : min(len(r), max_new)] = r[:max_new]
    hid = torch.from_numpy(buf.view(np.int16)).to(dev).view(torch.bfloat16)
    seq, nn, anchor = case.t_i32(case.seq_ids), case.t_i32(n_new), case.t_i32(case.anchor)
    if hole is not None:
        dr.page_table[case.seq_ids[hole[0]], hole[1]] = -1
    state = (dr.kv_pages.clone(), dr.ctx_len.clone())
    assert dr.read_error() == 0
    out = []
    for fused in (False, True):
        dr.kv_pages.copy_(state[0])
        dr.ctx_len.copy_(state[1])
        draft = torch.full((case.B, N - 1), -1, dtype=torch.int32, device=dev)
        gap = torch.zeros((case.B, N - 1), dtype=torch.float32, device=dev)
        if fused:
            dr.append_draft(seq, nn, hid, anchor, draft, gap, max_new=max_new)
        else:
            dr.ctx_append(seq, nn, hid, max_new)
            dr.draft_block(seq, anchor, draft, gap)
        err = dr.read_error()
        torch.cuda.synchronize()
        out.append(dict(draft=draft.cpu(), gap=gap.cpu().view(torch.int32), ctx_len=dr.ctx_len.cpu(),
                        pages=dr.kv_pages.view(torch.int16).cpu(), err=err))
    return out


def _same(a, b):
    for k in ("draft", "gap", "ctx_len", "pages"):
        assert torch.equal(a[k], b[k]), k
    assert a["err"] == b["err"], (a["err"], b["err"])


def test_append_draft_ragged_batch_shuffled_pages():
    cfg = synth.config("tiny")
    case = Case(cfg, ctx=[77, 130, 16], n_new=[8, 5, 0], seed=31, prefill_chunk=64, page_order="shuffled")
    case.prefill()
    a, b = _both(case, case.n_new, 8)
    _same(a, b)
    assert a["err"] == 0
    say(f"  drafts {a['draft'].tolist()}, ctx_len {a['ctx_len'][1:4].tolist()}")


def test_append_draft_tiled_gemm_batch():
    # 8 blocks of 16 rows: the draft's GEMMs take the tiled path (128 rows)
    cfg = small_cfg(block_size=16)
    ctx = [40 + 37 * b for b in range(8)]
    case = Case(cfg, ctx=ctx, n_new=[(3 * b) % 9 for b in range(8)], seed=32, prefill_chunk=64,
                page_order="shuffled")
    case.prefill()
    a, b = _both(case, case.n_new, 8)
    _same(a, b)
    assert a["err"] == 0


def test_append_draft_rows_in_whole_xcd_tiles():
    # 8 sequences x 16 appended-row slots and 8 blocks of 16 rows: both
    # multiples of 128, so the fused launch places the 16 rows of each
    # output tile on one XCD (fusion and first norm); ragged appends of
    # 0 .. 16 rows
    cfg = small_cfg(block_size=16)
    ctx = [40 + 37 * b for b in range(8)]
    case = Case(cfg, ctx=ctx, n_new=[(5 * b) % 17 for b in range(8)], seed=34, prefill_chunk=64,
                page_order="shuffled")
    case.prefill()
    a, b = _both(case, case.n_new, 16)
    _same(a, b)
    assert a["err"] == 0


def test_append_draft_failed_append_and_bad_n_new():
    cfg = synth.config("tiny")
    case = Case(cfg, ctx=[64, 100], n_new=[16, 4], seed=33, prefill_chunk=64, page_order="shuffled")
    case.prefill()
    dr = case.dr
    pt = dr.page_table.clone()
    L0 = int(dr.ctx_len[case.seq_ids[0]])
    # a hole where sequence 0's append lands: its append is skipped, its
    # draft runs on the old context; sequence 1 appends and drafts normally
    a, b = _both(case, case.n_new, 16, hole=(0, L0 // 16))
    _same(a, b)
    assert a["err"] & B.DEV_BAD_PAGE
    assert int(a["ctx_len"][case.seq_ids[0]]) == L0
    dr.page_table.copy_(pt)
    # n_new above max_new: flagged, that sequence untouched
    a, b = _both(case, [17, 2], 16)
    _same(a, b)
    assert a["err"] & B.DEV_BAD_N_NEW
    assert int(a["ctx_len"][case.seq_ids[0]]) == L0
