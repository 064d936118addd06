"""Device-memory owner around the C ABI.

PyTorch supplies the device memory (weights, paged KV cache, page table,
ctx_len, error word, workspace) and the stream; every step of the path runs
in libdflash.so's kernels. This module only allocates, marshals pointers
and checks return codes.
"""
import numpy as np
import torch

from . import _binding as B


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(name, t, shape, dtypes, optional=False):
    """The library cannot see a buffer's size: a tensor handed to it must be a
    contiguous device tensor of exactly the documented shape and dtype.
    `shape` entries of None match any extent (at least 1)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.dim() != len(shape) or any(e is not None and e != g for e, g in zip(shape, t.shape)) or \
            any(g < 1 for g in t.shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


I32, F32, BF16, LOGITS = (torch.int32,), (torch.float32,), (torch.bfloat16,), (torch.float32, torch.bfloat16)


def _bits_to_bf16(a, device):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class Drafter:
    """One drafter (weights + paged context cache + workspace) on one GPU.

    cfg: a shape dict (see synth.CONFIGS). weights: dict of bf16 bits
    (numpy uint16) and float32 w_fuse, or already-placed torch tensors.
    Pages: `pages_per_seq` per sequence slot; page_order "contiguous" or
    "shuffled" (a seeded permutation of the pool).
    """

    def __init__(self, cfg, weights, max_batch, max_new, max_seqs, pages_per_seq, max_pos=None,
                 device="cuda", page_order="contiguous", seed=0, fill_workspace=None):
        self.cfg = cfg
        self.device = torch.device(device)
        dev = self.device
        D, H = cfg["n_layers"], cfg["hidden"]
        n_kv, d = cfg["n_kv_heads"], cfg["head_dim"]
        self.max_batch, self.max_new, self.max_seqs = max_batch, max_new, max_seqs
        self.pages_per_seq = pages_per_seq
        n_pages = max_seqs * pages_per_seq
        self.n_pages = n_pages
        self.max_pos = max_pos or pages_per_seq * 16 + cfg["block_size"]

        self.w = {}
        for k, v in weights.items():
            if isinstance(v, torch.Tensor):
                self.w[k] = v.to(dev)
            elif k == "w_fuse":
                self.w[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev)
            else:
                self.w[k] = _bits_to_bf16(v, dev)

        self.kv_pages = torch.zeros((D, n_pages, 2, n_kv, 16 * d), dtype=torch.bfloat16, device=dev)
        order = np.arange(n_pages, dtype=np.int32)
        if page_order == "shuffled":
            order = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
        self.page_table_host = order.reshape(max_seqs, pages_per_seq)
        self.page_table = torch.from_numpy(self.page_table_host.copy()).to(dev)
        self.ctx_len = torch.zeros(max_seqs, dtype=torch.int32, device=dev)
        self.error_word = torch.zeros(1, dtype=torch.int32, device=dev)

        c = B.Config()
        for f, _ in B.Config._fields_:
            if f in cfg and f != "fusion":
                setattr(c, f, cfg[f])
        c.fusion = B.FUSION[cfg.get("fusion", "softmax")]
        c.page_size = 16
        c.max_seqs = max_seqs
        c.max_pages_per_seq = pages_per_seq
        c.n_pages = n_pages
        c.max_pos = self.max_pos
        c.max_batch = max_batch
        c.max_new = max_new
        c.mask_token_id = cfg["mask_token_id"]
        c.tied_kv = int(cfg.get("tied_kv", 0))
        c.use_rope = int(cfg.get("use_rope", 1))
        self.c = c
        ws = B.dflash_workspace_bytes(c)
        if ws == 0:
            raise B.DFlashError("unsupported config: " + B.last_error())
        self.ws_bytes = ws
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        if fill_workspace is not None:  # e.g. NaN bits, to catch reads of unwritten memory
            self.workspace.view(torch.int32)[: ws // 4].fill_(fill_workspace)

        wt = B.Weights()
        for f, _ in B.Weights._fields_:
            t = self.w.get(f)
            setattr(wt, f, t.data_ptr() if t is not None else None)
        kv = B.KV(kv_pages=self.kv_pages.data_ptr(), page_table=self.page_table.data_ptr(),
                  ctx_len=self.ctx_len.data_ptr(), error_word=self.error_word.data_ptr())
        torch.cuda.synchronize(dev)
        rc, h = B.dflash_create(c, wt, kv, self.workspace.data_ptr(), ws)
        B.check(rc, "dflash_create")
        self.handle = h
        # the library keeps its own packed copies of the streamed matrices
        for k in ("wq", "wk_d", "wv_d", "wk_t", "wv_t", "wo", "wg", "wu", "wd", "lm_head", "w_fc"):
            self.w.pop(k, None)

    # ---------------------------------------------------------------- calls
    def _dims(self):
        c = self.cfg
        return c["block_size"], c["vocab"], c["hidden"], c["n_layers"], c["n_target_layers"]

    def ctx_append(self, seq_ids, n_new, hidden, max_new=None, stream=None):
        """hidden: bf16 tensor [B, max_new, T, H]; seq_ids, n_new: int32 [B]."""
        Bn = seq_ids.numel()
        max_new = max_new or hidden.shape[1]
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("n_new", n_new, (Bn,), I32)
        _need("hidden", hidden, (Bn, max_new, T, H), BF16)
        rc = B.dflash_ctx_append(self.handle, Bn, seq_ids.data_ptr(), n_new.data_ptr(), hidden.data_ptr(),
                                 max_new, _stream(stream))
        return B.check(rc, "dflash_ctx_append")

    def draft_block(self, seq_ids, anchor, draft, gap=None, dbg_hidden=None, dbg_logits=None, stream=None):
        Bn = seq_ids.numel()
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("anchor", anchor, (Bn,), I32)
        _need("draft", draft, (Bn, N - 1), I32)
        _need("gap", gap, (Bn, N - 1), F32, optional=True)
        _need("dbg_hidden", dbg_hidden, (D + 1, Bn, N, H), F32, optional=True)
        _need("dbg_logits", dbg_logits, (Bn, N - 1, V), F32, optional=True)
        p = lambda t: t.data_ptr() if t is not None else None
        rc = B.dflash_draft_block(self.handle, Bn, seq_ids.data_ptr(), anchor.data_ptr(), draft.data_ptr(),
                                  p(gap), p(dbg_hidden), p(dbg_logits), _stream(stream))
        return B.check(rc, "dflash_draft_block")

    def append_draft(self, seq_ids, n_new, hidden, anchor, draft, gap=None, max_new=None, stream=None):
        """ctx_append then draft_block for the same sequences, as one call
        (the same results, fewer launches)."""
        Bn = seq_ids.numel()
        max_new = max_new or hidden.shape[1]
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("n_new", n_new, (Bn,), I32)
        _need("hidden", hidden, (Bn, max_new, T, H), BF16)
        _need("anchor", anchor, (Bn,), I32)
        _need("draft", draft, (Bn, N - 1), I32)
        _need("gap", gap, (Bn, N - 1), F32, optional=True)
        rc = B.dflash_append_draft(self.handle, Bn, seq_ids.data_ptr(), n_new.data_ptr(), hidden.data_ptr(), max_new,
                                   anchor.data_ptr(), draft.data_ptr(), gap.data_ptr() if gap is not None else None,
                                   _stream(stream))
        return B.check(rc, "dflash_append_draft")

    def verify(self, seq_ids, draft, logits, accept_len, next_token, commit_len=None, temperature=0.0,
               seed=0, step=0, stream=None):
        Bn = seq_ids.numel()
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("draft", draft, (Bn, N - 1), I32)
        _need("logits", logits, (Bn, N, V), LOGITS)
        for name, t in (("accept_len", accept_len), ("next_token", next_token)):
            _need(name, t, (Bn,), I32)
        _need("commit_len", commit_len, (Bn,), I32, optional=True)
        dt = B.DTYPE_F32 if logits.dtype == torch.float32 else B.DTYPE_BF16
        rc = B.dflash_verify(self.handle, Bn, seq_ids.data_ptr(), draft.data_ptr(), logits.data_ptr(), dt,
                             temperature, seed, step, accept_len.data_ptr(), next_token.data_ptr(),
                             commit_len.data_ptr() if commit_len is not None else None, _stream(stream))
        return B.check(rc, "dflash_verify")

    def draft_sample(self, seq_ids, anchor, temperature, draft, draft_logits, seed=0, step=0, stream=None):
        """Sampled draft at `temperature`: draft int32 [B, N-1] and the
        drafter's logits fp32 [B, N-1, V] (out; verify_sample reads them)."""
        Bn = seq_ids.numel()
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("anchor", anchor, (Bn,), I32)
        _need("draft", draft, (Bn, N - 1), I32)
        _need("draft_logits", draft_logits, (Bn, N - 1, V), F32)
        rc = B.dflash_draft_sample(self.handle, Bn, seq_ids.data_ptr(), anchor.data_ptr(), temperature, seed, step,
                                   draft.data_ptr(), draft_logits.data_ptr(), _stream(stream))
        return B.check(rc, "dflash_draft_sample")

    def verify_sample(self, seq_ids, draft, draft_logits, draft_temperature, logits, accept_len, next_token,
                      commit_len=None, seed=0, step=0, stream=None):
        """Lossless verification of a sampled draft at target temperature 1."""
        Bn = seq_ids.numel()
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("draft", draft, (Bn, N - 1), I32)
        _need("draft_logits", draft_logits, (Bn, N - 1, V), F32)
        _need("logits", logits, (Bn, N, V), LOGITS)
        for name, t in (("accept_len", accept_len), ("next_token", next_token)):
            _need(name, t, (Bn,), I32)
        _need("commit_len", commit_len, (Bn,), I32, optional=True)
        dt = B.DTYPE_F32 if logits.dtype == torch.float32 else B.DTYPE_BF16
        rc = B.dflash_verify_sample(self.handle, Bn, seq_ids.data_ptr(), draft.data_ptr(), draft_logits.data_ptr(),
                                    draft_temperature, logits.data_ptr(), dt, seed, step, accept_len.data_ptr(),
                                    next_token.data_ptr(),
                                    commit_len.data_ptr() if commit_len is not None else None, _stream(stream))
        return B.check(rc, "dflash_verify_sample")

    def d2sd_draft(self, seq_ids, anchor, K, drafts, conf=None, cuts=None, stream=None):
        """Dual-pass drafting: drafts int32 [B, K+1, N-1] (candidate 0 = the
        first draft); conf fp32 [B, N-1] and cuts int32 [B, K] optional."""
        Bn = seq_ids.numel()
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("anchor", anchor, (Bn,), I32)
        _need("drafts", drafts, (Bn, K + 1, N - 1), I32)
        _need("conf", conf, (Bn, N - 1), F32, optional=True)
        _need("cuts", cuts, (Bn, K), I32, optional=True)
        p = lambda t: t.data_ptr() if t is not None else None
        rc = B.dflash_d2sd_draft(self.handle, Bn, seq_ids.data_ptr(), anchor.data_ptr(), K, drafts.data_ptr(),
                                 p(conf), p(cuts), _stream(stream))
        return B.check(rc, "dflash_d2sd_draft")

    def verify_multi(self, seq_ids, drafts, logits, accept_len, next_token, commit_len=None, chosen=None,
                     stream=None):
        """Greedy verification of C candidates per sequence: drafts [B, C, N-1],
        logits [B, C, N, V]; the longest accept wins (lowest index on ties)."""
        Bn, C = drafts.shape[0], drafts.shape[1]
        N, V, H, D, T = self._dims()
        _need("seq_ids", seq_ids, (Bn,), I32)
        _need("drafts", drafts, (Bn, C, N - 1), I32)
        _need("logits", logits, (Bn, C, N, V), LOGITS)
        for name, t in (("accept_len", accept_len), ("next_token", next_token)):
            _need(name, t, (Bn,), I32)
        for name, t in (("commit_len", commit_len), ("chosen", chosen)):
            _need(name, t, (Bn,), I32, optional=True)
        dt = B.DTYPE_F32 if logits.dtype == torch.float32 else B.DTYPE_BF16
        p = lambda t: t.data_ptr() if t is not None else None
        rc = B.dflash_verify_multi(self.handle, Bn, C, seq_ids.data_ptr(), drafts.data_ptr(), logits.data_ptr(), dt,
                                   accept_len.data_ptr(), next_token.data_ptr(), p(commit_len), p(chosen),
                                   _stream(stream))
        return B.check(rc, "dflash_verify_multi")

    def read_error(self, stream=None):
        rc, v = B.dflash_read_error(self.handle, _stream(stream))
        B.check(rc, "dflash_read_error")
        return v

    def close(self):
        if getattr(self, "handle", None):
            B.dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ----------------------------------------------------- host-side views
    def cache_rows(self, layer, seq, length):
        """Context K [L, n_kv, d] (rotated) and V [L, n_kv, d] of one
        sequence, gathered through the page table (host float32)."""
        n_kv, d = self.cfg["n_kv_heads"], self.cfg["head_dim"]
        pages = self.page_table_host[seq, : (length + 15) // 16]
        kv = self.kv_pages[layer, torch.from_numpy(pages.astype(np.int64)).to(self.device)].float().cpu()
        k = kv[:, 0].reshape(len(pages), n_kv, 16, d).permute(0, 2, 1, 3).reshape(-1, n_kv, d)[:length]
        v = kv[:, 1].reshape(len(pages), n_kv, d, 16).permute(0, 3, 1, 2).reshape(-1, n_kv, d)[:length]
        return k.numpy(), v.numpy()
