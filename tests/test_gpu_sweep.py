"""Parity over a seeded sweep of small drafter geometries.

Each case draws a shape within what the library supports (head dim 64 or
128; GQA group and block size with (n_q / n_kv) * N a multiple of 16 up to
256; hidden, intermediate and vocabulary multiples of 32 that are not powers
of two; 1 to 9 target layers; softmax or FC fusion; tied or separate
context K/V) and a ragged batch (context lengths off the page, chunk and
tile grids, one entry often appending nothing, shuffled pages), then runs
one decode step on both sides under the parity bar of _cases.py: context
K/V, the residual stream after every layer and the logits within 2e-2,
draft tokens exact where the oracle's top-2 gap is >= 1e-2, greedy
verification exact.
"""
import numpy as np
import pytest
import torch

from _cases import Case, say
from block_diffusion_drafter_softmax_amd import synth
from test_gpu_parity import run_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sweep_case(seed):
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([64, 128]))
    N = (16, 8, 4, 2)[seed % 4]  # down to the smallest block: an anchor and one mask position
    G = int(r.choice([g for g in (1, 2, 4, 8, 16) if (g * N) % 16 == 0 and g * N <= 256]))
    n_kv = int(r.integers(1, 4))
    H = 32 * int(r.integers(5, 14))          # 160 .. 416
    cfg = synth.config("tiny")
    cfg.update(hidden=H, n_layers=int(r.integers(1, 4)), n_q_heads=G * n_kv, n_kv_heads=n_kv, head_dim=d,
               intermediate=32 * int(r.integers(7, 23)), vocab=32 * int(r.integers(70, 200)),
               n_target_layers=int(r.integers(1, 10)), block_size=N, tied_kv=int(r.integers(0, 2)),
               fusion="fc" if seed % 2 else "softmax")
    cfg["mask_token_id"] = cfg["vocab"] - 1
    B = int(r.integers(1, 4))
    if N == 2:  # one draft position per sequence: enough sequences to compare some
        B = max(B, 3)
    ctx = [int(x) for x in r.integers(0, 300, size=B)]
    n_new = [int(min(c, x)) for c, x in zip(ctx, r.integers(0, 18, size=B))]
    return cfg, ctx, n_new


@pytest.mark.parametrize("seed", range(16))
def test_seeded_geometry_sweep(seed):
    cfg, ctx, n_new = sweep_case(seed)
    say(f"  H {cfg['hidden']} D {cfg['n_layers']} heads {cfg['n_q_heads']}/{cfg['n_kv_heads']}x{cfg['head_dim']} "
        f"I {cfg['intermediate']} V {cfg['vocab']} T {cfg['n_target_layers']} N {cfg['block_size']} "
        f"tied {cfg['tied_kv']} fusion {cfg['fusion']}")
    run_step(Case(cfg, ctx=ctx, n_new=n_new, seed=200 + seed, page_order="shuffled", prefill_chunk=48))
