"""dflash_verify_noalloc (the verification that allocates nothing: partials
in a static per-GPU scratch array) against dflash_verify (partials in the
handle's workspace), through the C ABI: identical accept lengths, next and
committed tokens on consecutive calls (greedy and temperature 1, bf16 and
fp32 logits, each call smaller or larger than the last, so stale scratch
contents would show), and a host-side refusal of a call whose partials
would not fit the scratch."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_softmax_amd import _binding as B
from block_diffusion_drafter_softmax_amd import synth
from block_diffusion_drafter_softmax_amd.drafter import Drafter

pytestmark = pytest.mark.gpu

V, N = 262144, 16   # 8 rows-pass chunks of 32768 logits per row
MAX_B = 1040


@pytest.fixture(scope="module")
def drafter():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.config("tiny")
    cfg.update(vocab=V, hidden=256, n_layers=1, intermediate=256, block_size=N, n_q_heads=2, n_kv_heads=2)
    cfg["mask_token_id"] = V - 1
    dr = Drafter(cfg, synth.make_weights(cfg, 0), max_batch=MAX_B, max_new=1, max_seqs=MAX_B + 3, pages_per_seq=2)
    yield dr
    dr.close()


def logits_for(cfg_over, draft, seed):
    cfg = synth.config("tiny")
    cfg.update(vocab=V, block_size=N, **cfg_over)
    z = synth.make_logits(cfg, draft, seed)
    if z.dtype == np.float32:
        return torch.from_numpy(z).cuda(), B.DTYPE_F32
    return torch.from_numpy(z.view(np.int16)).cuda().view(torch.bfloat16), B.DTYPE_BF16


def outputs(Bn):
    return [torch.full((Bn,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]


def call(fn, dr, seq, draft, z, dt, temp, seed, step, out):
    st = torch.cuda.current_stream().cuda_stream
    return fn(dr.handle, seq.numel(), seq.data_ptr(), draft.data_ptr(), z.data_ptr(), dt, temp, seed, step,
              out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), st)


@pytest.mark.parametrize("Bn,temp,over,seed", [
    (12, 1.0, dict(logit_model="accept_p", agreement=0.75, logits_f32=False), 3),  # temperature 1, bf16
    (3, 0.0, dict(logit_model="top_plus1", agreement=0.8, logits_f32=True), 4),     # smaller, greedy fp32
    (5, 1.0, dict(logit_model="accept_p", agreement=0.6, logits_f32=True), 5),      # temperature 1, fp32
    (2, 1.0, dict(logit_model="accept_p", agreement=0.9, logits_f32=False), 6),     # smaller again
])
def test_noalloc_matches_workspace_verify(drafter, Bn, temp, over, seed):
    rng = np.random.default_rng(seed)
    draft_np = rng.integers(0, V - 1, size=(Bn, N - 1)).astype(np.int32)
    z, dt = logits_for(over, draft_np, seed)
    draft = torch.from_numpy(draft_np).cuda()
    seq = torch.arange(Bn, dtype=torch.int32, device="cuda") + 1
    ref, got = outputs(Bn), outputs(Bn)
    B.check(call(B.dflash_verify, drafter, seq, draft, z, dt, temp, 11, seed, ref), "dflash_verify")
    B.check(call(B.dflash_verify_noalloc, drafter, seq, draft, z, dt, temp, 11, seed, got), "dflash_verify_noalloc")
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g), (r.tolist(), g.tolist())
    assert int(ref[0].min()) >= 0 and int(ref[0].max()) <= N - 1
    assert torch.equal(ref[2], ref[0] + 1)
    assert drafter.read_error() == 0
    print(f"B={Bn} temperature {temp}: accept {got[0].tolist()}", flush=True)


def test_noalloc_refuses_more_than_its_scratch(drafter):
    # 1030 sequences x 16 rows x 8 chunks x 8 bytes > 1 MiB: refused on the
    # host before anything is enqueued (the buffers are real and sized
    # anyway, so nothing could read past them)
    Bn = 1030
    assert Bn * N * 8 * 8 > B.VERIFY_SCRATCH_BYTES
    z = torch.empty((Bn, N, V), dtype=torch.bfloat16, device="cuda")
    draft = torch.zeros((Bn, N - 1), dtype=torch.int32, device="cuda")
    seq = torch.arange(Bn, dtype=torch.int32, device="cuda")
    out = outputs(Bn)
    rc = call(B.dflash_verify_noalloc, drafter, seq, draft, z, B.DTYPE_BF16, 0.0, 0, 0, out)
    assert rc == B.ERR_CAPACITY
    assert "scratch" in B.last_error()
    torch.cuda.synchronize()
    assert int(out[0].max()) == -1 and int(out[0].min()) == -1  # nothing ran
    del z
    # the scratch still serves the next call
    test_noalloc_matches_workspace_verify(drafter, 4, 1.0, dict(logit_model="accept_p", agreement=0.75,
                                                                logits_f32=False), 9)
