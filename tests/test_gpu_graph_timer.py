"""A decode step captured as a HIP graph and replayed gives, on every replay,
bit-identical results to the same step launched eagerly (the library puts
no memset nodes in a capture and its passes are separated by kernel
boundaries; the one counter set, the persistent attention's per-XCD work
counters, is zeroed by the kernel before each attention launch); and the
kernel timer reports launch durations for the kinds a step runs."""
import numpy as np
import pytest
import torch

from _cases import Case, say
from block_diffusion_drafter_softmax_amd import synth
from block_diffusion_drafter_softmax_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _step_setup(temperature, geometry="tiny"):
    if geometry == "tiny":
        cfg = synth.config("tiny")
        case = Case(cfg, ctx=[77, 130, 16], n_new=[8, 5, 0], seed=21, prefill_chunk=64, page_order="shuffled")
    else:
        # d_h 128, GQA 4:1, 2000 pages per sequence: 8-chunk attention items
        # through the persistent ring kernel and its work counters
        cfg = synth.config("tiny")
        cfg.update(hidden=512, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=512, vocab=2048,
                   block_size=16)
        cfg["mask_token_id"] = cfg["vocab"] - 1
        ctx = [2500, 1000]
        case = Case(cfg, ctx=ctx, n_new=[8, 0], seed=22, prefill_chunk=512, page_order="shuffled",
                    extra_pages=2000 - (max(ctx) + 16 + 15) // 16)
    case.prefill()
    torch.cuda.synchronize()
    dr, dev = case.dr, case.dev
    Bn, N, V, T, H = case.B, cfg["block_size"], cfg["vocab"], cfg["n_target_layers"], cfg["hidden"]
    max_new = max(case.n_new)
    buf = np.zeros((Bn, max_new, T, H), dtype=np.uint16)
    for b, r in enumerate(case.hidden_step):
        buf[b, : len(r)] = r
    io = dict(
        seq=case.t_i32(case.seq_ids), n_new=case.t_i32(case.n_new), anchor=case.t_i32(case.anchor),
        hid=torch.from_numpy(buf.view(np.int16)).to(dev).view(torch.bfloat16),
        ctx0=dr.ctx_len.clone(),
        logits=torch.randn((Bn, N, V), generator=torch.Generator().manual_seed(5)).to(dev),
        draft=torch.zeros((Bn, N - 1), dtype=torch.int32, device=dev),
        gap=torch.zeros((Bn, N - 1), dtype=torch.float32, device=dev),
        acc=torch.zeros(Bn, dtype=torch.int32, device=dev),
        nxt=torch.zeros(Bn, dtype=torch.int32, device=dev),
        com=torch.zeros(Bn, dtype=torch.int32, device=dev),
    )

    def step():
        dr.ctx_len.copy_(io["ctx0"])
        dr.ctx_append(io["seq"], io["n_new"], io["hid"], max_new)
        dr.draft_block(io["seq"], io["anchor"], io["draft"], io["gap"])
        dr.verify(io["seq"], io["draft"], io["logits"], io["acc"], io["nxt"], io["com"],
                  temperature=temperature, seed=99, step=3)

    return case, io, step


def _outputs(case, io):
    torch.cuda.synchronize()
    out = {k: io[k].clone() for k in ("draft", "gap", "acc", "nxt", "com")}
    out["ctx_len"] = case.dr.ctx_len.clone()
    out["pages"] = case.dr.kv_pages.view(torch.int16).clone()
    return out


@pytest.mark.parametrize("temperature,geometry", [(0.0, "tiny"), (1.0, "tiny"), (0.0, "ring")])
def test_graph_replay_matches_eager(temperature, geometry):
    case, io, step = _step_setup(temperature, geometry)
    step()
    ref = _outputs(case, io)
    assert case.dr.read_error() == 0

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for r in range(4):
        for k in ("draft", "gap", "acc", "nxt", "com"):
            io[k].fill_(-7)  # eager work between replays
        if r == 2:
            step()  # an eager step between replays, too
            torch.cuda.synchronize()
            for k in ("draft", "gap", "acc", "nxt", "com"):
                io[k].fill_(-7)
        graph.replay()
        got = _outputs(case, io)
        for k, v in ref.items():
            a, b = v.cpu().numpy(), got[k].cpu().numpy()
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), (r, k)
    assert case.dr.read_error() == 0
    say(f"  {geometry}, temperature {temperature}: 4 replays bit-identical, accept {ref['acc'].tolist()}")


def test_kernel_timer_reports_every_kind_of_a_step():
    case, io, step = _step_setup(0.0)
    h = case.dr.handle
    kinds = [B.K_FUSE, B.K_CTX_KV, B.K_CTX_FINISH, B.K_NORM, B.K_QKV, B.K_QKV_FINISH, B.K_ATTN,
             B.K_ATTN_MERGE, B.K_OPROJ, B.K_GATE_UP, B.K_DOWN, B.K_LM_HEAD, B.K_ARGMAX, B.K_VERIFY]
    assert len(kinds) == B.K_COUNT - 1  # all but the dual-pass drafter's (tests/test_gpu_d2sd.py)
    for k in kinds:
        B.check(B.dflash_kernel_timer(h, k, 1), "timer")
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    D = case.cfg["n_layers"]
    expect = {B.K_GATE_UP: 3 * D, B.K_LM_HEAD: 3, B.K_VERIFY: 3, B.K_NORM: 3 * (2 * D + 1)}
    for k in kinds:
        rc, ms, n = B.dflash_kernel_timer_read(h, k)
        B.check(rc, "timer read")
        B.check(B.dflash_kernel_timer(h, k, 0), "timer off")
        assert n > 0 and ms > 0 and ms / n < 50.0, (k, ms, n)
        if k in expect:
            assert n == expect[k], (k, n)
