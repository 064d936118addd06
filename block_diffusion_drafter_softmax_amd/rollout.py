"""Device-resident roll-out: S decode steps with no host round trip.

Each step appends the target hidden states of the tokens the previous step
committed (their number is the previous verification's commit_len, read by
the append from device memory), drafts a block anchored on the previous
step's next token, and verifies it; the context grows by the committed
count every step (DFlash summary, Methodology step 4: the window advances
by the accepted tokens; D^2SD summary, Methodology step 5). Because every
per-step quantity stays on the device, the S steps can be captured once as
a HIP graph and replayed.

The target model is not part of this path. Its two outputs are stood in for
by synthetic data, supplied per step: hidden states [S, B, N, T, H] (rows
0 .. commit-1 of step s are appended at step s + 1) and target logits built
on the device around the step's own draft by the agreement model of the
synthetic workloads: noise logits with, where agree[s, b, r], the draft
token d_{r+1} of row r set to (row maximum + 1). This module only moves
device buffers and calls the library; the stand-in's few torch ops (copy,
gather, scatter) are harness, not drafter arithmetic.
"""
import torch


class Rollout:
    """S steps of (append, draft, target stand-in, verify) for B sequences.

    dr: a Drafter whose sequences `seq_ids` hold their prefilled contexts.
    anchor0, n_new0: int32 [B] device tensors, the first step's anchor and
    appended row count. hidden: bf16 [S, B, N, T, H]; noise: bf16 [S, B, N, V]
    target logits before agreement; agree: bool [S, B, N-1]; top1: bf16
    [S, B, N-1], the value an agreeing draft token gets (row maximum + 1).
    Per-step outputs go to `draft` [S, B, N-1], `accept`, `next_token`,
    `commit` [S, B] (int32).
    """

    def __init__(self, dr, seq_ids, anchor0, n_new0, hidden, noise, agree, top1):
        self.dr, self.seq = dr, seq_ids
        S, Bn, N = noise.shape[0], noise.shape[1], noise.shape[2]
        self.S, self.B, self.N = S, Bn, N
        self.hidden, self.noise, self.agree, self.top1 = hidden, noise, agree, top1
        self.anchor0, self.n_new0 = anchor0, n_new0
        dev = noise.device
        self.ctx0 = dr.ctx_len.clone()
        self.anchor = anchor0.clone()
        self.n_new = n_new0.clone()
        self.logits = torch.empty_like(noise[0])
        self.draft = torch.zeros((S, Bn, N - 1), dtype=torch.int32, device=dev)
        self.accept = torch.zeros((S, Bn), dtype=torch.int32, device=dev)
        self.next_token = torch.zeros((S, Bn), dtype=torch.int32, device=dev)
        self.commit = torch.zeros((S, Bn), dtype=torch.int32, device=dev)

    def reset(self):
        """Back to the prefilled state (device copies only)."""
        self.dr.ctx_len.copy_(self.ctx0)
        self.anchor.copy_(self.anchor0)
        self.n_new.copy_(self.n_new0)

    def _target(self, s):
        """Synthetic target logits for step s around its draft."""
        d = self.draft[s].long().unsqueeze(2)                       # [B, N-1, 1]
        self.logits.copy_(self.noise[s])
        head = self.logits[:, : self.N - 1]
        cur = head.gather(2, d)
        head.scatter_(2, d, torch.where(self.agree[s].unsqueeze(2), self.top1[s].unsqueeze(2), cur))

    def step(self, s):
        dr = self.dr
        dr.append_draft(self.seq, self.n_new, self.hidden[s], self.anchor, self.draft[s], max_new=self.N)
        self._target(s)
        dr.verify(self.seq, self.draft[s], self.logits, self.accept[s], self.next_token[s], self.commit[s])
        # the next step appends the committed rows and drafts from the next token
        self.n_new.copy_(self.commit[s])
        self.anchor.copy_(self.next_token[s])

    def run(self):
        self.reset()
        for s in range(self.S):
            self.step(s)

    def capture(self):
        """Record reset + S steps as one graph; returns it (replay() runs it)."""
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return graph
