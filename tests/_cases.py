"""Parity harness: the same seeded inputs through the HIP path (C ABI via the
binding) and through the oracle, and the comparisons of the parity bar.

Parity bar (stated once, used by every GPU test):
  * token ids, accept lengths, next tokens: bit-exact, except draft positions
    where the oracle's top-1/top-2 logit gap is below 1e-2 (and, for
    temperature-1 verification, decisions where |u - p| < 1e-5 or the
    oracle's Gumbel top-2 gap is below 1e-2);
  * floating point (context K/V, the residual stream after every layer,
    logits): max |gpu - oracle| / max |oracle| <= 2e-2 per tensor.
"""
import numpy as np
import torch

import oracle as O
from block_diffusion_drafter_softmax_amd import synth
from block_diffusion_drafter_softmax_amd.drafter import Drafter

FLOAT_TOL = 2e-2
GAP_MIN = 1e-2
NAN_FILL = 0x7FC07FC0  # fp32 NaN / bf16 NaN pairs: reads of unwritten workspace show up


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(gpu - ref))) / den


def say(msg):
    print(msg, flush=True)


class Case:
    """One seeded decode step on both sides.

    ctx: context length per sequence after the step's append; n_new: rows
    appended in the step (the rest is prefilled before it, in calls of at
    most `prefill_chunk` rows per sequence).
    """

    def __init__(self, cfg, ctx, n_new, seed=0, page_order="contiguous", seq_offset=1,
                 prefill_chunk=64, extra_pages=1, oracle_seqs=None, oracle_chunk=1024, max_batch=None):
        self.cfg = cfg
        self.B = len(ctx)
        self.ctx = [int(x) for x in ctx]
        self.n_new = [int(x) for x in n_new]
        self.seed = seed
        self.seq_ids = [b + seq_offset for b in range(self.B)]
        N = cfg["block_size"]
        say(f"[case] {cfg.get('name', '?')} B={self.B} ctx={self.ctx} n_new={self.n_new} seed={seed} "
            f"pages={page_order}")
        self.w = synth.make_weights(cfg, seed)
        self.model = O.OracleModel(cfg, self.w)
        self.cache = O.OracleCache(cfg["n_layers"])
        self.max_new = max(prefill_chunk, max(self.n_new))
        pps = (max(self.ctx) + N + 15) // 16 + extra_pages
        self.dr = Drafter(cfg, self.w, max_batch=max_batch or self.B, max_new=self.max_new,
                          max_seqs=self.B + seq_offset, pages_per_seq=pps, page_order=page_order,
                          seed=seed, fill_workspace=NAN_FILL)
        self.dev = self.dr.device
        # unwritten cache slots hold NaN: masked keys must never reach the output
        self.dr.kv_pages.view(torch.int16).fill_(0x7FC0)
        self.hidden_pre = [synth.make_hidden(cfg, c - n, seed, f"pre/{b}") for b, (c, n) in
                           enumerate(zip(self.ctx, self.n_new))]
        self.hidden_step = [synth.make_hidden(cfg, n, seed, f"step/{b}") for b, n in enumerate(self.n_new)]
        self.anchor = synth.make_anchor(cfg, self.B, seed)
        self.prefill_chunk = prefill_chunk
        # batch entries the oracle reproduces (sequences never interact, so a
        # sample of them checks the batched launch); appends in row chunks
        self.oracle_seqs = list(range(self.B)) if oracle_seqs is None else list(oracle_seqs)
        self.oracle_chunk = oracle_chunk

    def t_i32(self, a):
        return torch.tensor(np.asarray(a, dtype=np.int32), device=self.dev)

    def _append_gpu(self, rows, max_new):
        """rows[b]: bf16 bits [n_b, T, H] for sequence b (n_b may be 0)."""
        cfg = self.cfg
        T, H = cfg["n_target_layers"], cfg["hidden"]
        buf = np.zeros((self.B, max_new, T, H), dtype=np.uint16)
        for b, r in enumerate(rows):
            buf[b, : len(r)] = r
        hid = torch.from_numpy(buf.view(np.int16)).to(self.dev).view(torch.bfloat16)
        self.dr.ctx_append(self.t_i32(self.seq_ids), self.t_i32([len(r) for r in rows]), hid, max_new)

    def prefill(self):
        pre = [len(h) for h in self.hidden_pre]
        done = [0] * self.B
        while any(d < p for d, p in zip(done, pre)):
            rows = []
            for b in range(self.B):
                n = min(self.prefill_chunk, pre[b] - done[b])
                rows.append(self.hidden_pre[b][done[b]: done[b] + n])
                done[b] += n
            self._append_gpu(rows, self.prefill_chunk)
        for b in self.oracle_seqs:
            for r0 in range(0, pre[b], self.oracle_chunk):
                rows = self.hidden_pre[b][r0: r0 + self.oracle_chunk]
                O.ctx_append(self.model, self.cache, self.seq_ids[b], O.bf16_bits_to_f64(rows))

    def step_append(self):
        self._append_gpu(self.hidden_step, max(1, max(self.n_new)))
        for b in self.oracle_seqs:
            if self.n_new[b]:
                O.ctx_append(self.model, self.cache, self.seq_ids[b], O.bf16_bits_to_f64(self.hidden_step[b]))

    def draft(self, dbg=True):
        cfg = self.cfg
        N, H, V, D = cfg["block_size"], cfg["hidden"], cfg["vocab"], cfg["n_layers"]
        dev = self.dev
        out = dict(
            draft=torch.full((self.B, N - 1), -1, dtype=torch.int32, device=dev),
            gap=torch.zeros((self.B, N - 1), dtype=torch.float32, device=dev),
            hidden=torch.zeros((D + 1, self.B, N, H), dtype=torch.float32, device=dev) if dbg else None,
            logits=torch.zeros((self.B, N - 1, V), dtype=torch.float32, device=dev) if dbg else None,
        )
        self.dr.draft_block(self.t_i32(self.seq_ids), self.t_i32(self.anchor), out["draft"], out["gap"],
                            out["hidden"], out["logits"])
        torch.cuda.synchronize()
        return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}

    def oracle_draft(self):
        """Oracle drafts of the sampled batch entries, in oracle_seqs order."""
        return [O.draft_block(self.model, self.cache, self.seq_ids[b], int(self.anchor[b]))
                for b in self.oracle_seqs]

    # ------------------------------------------------------------ checks
    def check_cache(self):
        errs = []
        for i in range(self.cfg["n_layers"]):
            for b in self.oracle_seqs:
                L = self.ctx[b]
                if L == 0:
                    continue
                k, v = self.dr.cache_rows(i, self.seq_ids[b], L)
                ok, ov = self.cache.k[i][self.seq_ids[b]], self.cache.v[i][self.seq_ids[b]]
                errs.append(rel_err(k, ok))
                errs.append(rel_err(v, ov))
        return max(errs) if errs else 0.0

    def compare_draft(self, g, orc):
        """Returns (max hidden rel err, max logits rel err, n compared, n excluded)."""
        he, le = 0.0, 0.0
        compared = excluded = 0
        for b, o in zip(self.oracle_seqs, orc):
            if g["hidden"] is not None:
                for layer in range(o["hidden"].shape[0]):
                    he = max(he, rel_err(g["hidden"][layer, b], o["hidden"][layer]))
            if g["logits"] is not None:
                for j in range(o["logits"].shape[0]):
                    le = max(le, rel_err(g["logits"][b, j], o["logits"][j]))
        for b, o in zip(self.oracle_seqs, orc):
            if g["gap"] is not None:  # the top-2 gap is a float output: same bar, on the row's logit scale
                for j in range(len(o["draft"])):
                    scale = float(np.max(np.abs(o["logits"][j])))
                    assert abs(float(g["gap"][b, j]) - o["gap"][j]) <= FLOAT_TOL * scale, (
                        f"gap mismatch seq {b} pos {j}: gpu {g['gap'][b, j]} oracle {o['gap'][j]} (|logit| {scale})")
            for j in range(len(o["draft"])):
                if o["gap"][j] < GAP_MIN:
                    excluded += 1
                    continue
                compared += 1
                assert int(g["draft"][b, j]) == int(o["draft"][j]), (
                    f"draft mismatch seq {b} pos {j}: gpu {g['draft'][b]} oracle {o['draft']} gap {o['gap']} "
                    f"(hidden rel {he:.2e}, logits rel {le:.2e})")
        return he, le, compared, excluded


def check_positions(g, orc, oracle_seqs, min_distinct=3):
    """Per-position checks of a draft whose positions differ.

    * diversity: each sampled sequence's oracle draft holds at least
      `min_distinct` distinct tokens at positions whose top-2 gap is >= 1e-2
      (otherwise the exact token comparison decides only one argmax);
    * row identity: every GPU logits row is closer (max abs difference over
      the oracle row's max abs value) to its own oracle row than to any
      other row of the block, and the margin is wider than the float bar,
      so a block-row mix-up (a RoPE position, a page-table row, the
      LM-head row -> draft position map) cannot pass.
    Returns the smallest distinct count seen."""
    fewest = None
    for b, o in zip(oracle_seqs, orc):
        ok = [int(t) for t, gp in zip(o["draft"], o["gap"]) if gp >= GAP_MIN]
        n = len(set(ok))
        fewest = n if fewest is None else min(fewest, n)
        assert n >= min_distinct, f"seq {b}: oracle draft {list(o['draft'])} has {n} distinct decided tokens"
        if g["logits"] is None:
            continue
        z, zo = g["logits"][b].astype(np.float64), o["logits"]
        for j in range(zo.shape[0]):
            errs = [float(np.max(np.abs(z[j] - zo[k]))) / max(float(np.max(np.abs(zo[k]))), 1e-30)
                    for k in range(zo.shape[0])]
            own = errs[j]
            other = min(e for k, e in enumerate(errs) if k != j)
            assert own < other and other > 2 * FLOAT_TOL, (
                f"seq {b} row {j}: own-row error {own:.2e}, nearest other row {other:.2e}")
    return fewest


def nan_free(*arrays):
    return all(np.all(np.isfinite(a)) for a in arrays if a is not None)
