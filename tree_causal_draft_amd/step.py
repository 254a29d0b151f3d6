"""One draft-and-verify step on the device: buffers allocated once, four library calls.

    top-W over the draft logits -> ancestor mask -> tree attention -> greedy verify

Used by the benchmark, the smoke check and the tests.  Nothing here computes: it moves a
seeded workload (numpy) to device memory, preallocates every output and workspace, and
calls the libjt entry points in stream order.  The tree (parent, tokens) is an input of
the step, built by the workload generator; tree() builds the best-first tree of the
step's top-W lists on the device into separate buffers.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (build_tree_best_first, build_tree_mask, commit_accepted_kv, draft_verify_step,
               step_workspace_size, topw_per_depth, verify_sampled,
               verify_sampled_workspace_size,
               tree_attention, tree_attention_workspace_size, topw_workspace_size, verify_greedy,
               verify_workspace_size, JT_BF16, JT_F32)
from .workload import Workload


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are raw bf16 words."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceStep:
    def __init__(self, w: Workload, device="cuda:0", parts=("topw", "mask", "attn", "verify")):
        cfg = w.cfg
        self.w = w
        self.cfg = cfg
        self.dev = torch.device(device)
        self.parts = parts
        dev = self.dev
        S, B, N, W = cfg.S, cfg.B, cfg.N, cfg.W
        dt = JT_BF16 if cfg.dtype == "bf16" else JT_F32
        self.parent = to_device(w.parent, dev)
        self.tokens = to_device(w.tokens, dev)
        self.anc = torch.empty((S, B, 4), dtype=torch.int64, device=dev)
        self.depth = torch.empty((S, B), dtype=torch.int32, device=dev)
        self.err_mask = torch.empty(S, dtype=torch.int32, device=dev)
        if "attn" in parts:
            self.q = to_device(w.q, dev)
            self.k_tree = to_device(w.k_tree, dev)
            self.v_tree = to_device(w.v_tree, dev)
            self.k_prefix = to_device(w.k_prefix, dev)
            self.v_prefix = to_device(w.v_prefix, dev)
            self.prefix_len = to_device(w.prefix_len, dev)
            self.block_table = None if w.block_table is None else to_device(w.block_table, dev)
            self.attn_out = torch.empty_like(self.q)
            self.lse = torch.empty((S, B, cfg.Hq), dtype=torch.float32, device=dev)
            self.err_attn = torch.empty(S, dtype=torch.int32, device=dev)
            nb = self.attn_ws_bytes = tree_attention_workspace_size(
                S, B, cfg.Hq, cfg.Hkv, cfg.d, w.max_prefix, dt,
                cfg.block_size if w.block_table is not None else 0)
            self.attn_ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device=dev) if nb else None
            if w.block_table is None:
                # a prefix cache with room for an accepted path, written by commit()
                cap = w.max_prefix + N + 1
                self.commit_k = torch.zeros((S, cap) + tuple(self.k_prefix.shape[2:]),
                                            dtype=self.k_prefix.dtype, device=dev)
                self.commit_v = torch.zeros_like(self.commit_k)
                self.commit_len = torch.empty(S, dtype=torch.int32, device=dev)
                self.err_commit = torch.empty(S, dtype=torch.int32, device=dev)
        if "topw" in parts:
            self.draft = to_device(w.draft_logits, dev)
            self.ids = torch.empty((S * N, W), dtype=torch.int32, device=dev)
            self.logprob = torch.empty((S * N, W), dtype=torch.float32, device=dev)
            self.row_lse = torch.empty(S * N, dtype=torch.float32, device=dev)
            nb = topw_workspace_size(S * N, cfg.V, W, dt)
            self.topw_ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
            # the best-first tree of the top-W lists (kept apart from the step's own tree)
            self.tree_parent = torch.empty((S, B), dtype=torch.int32, device=dev)
            self.tree_tokens = torch.empty((S, B), dtype=torch.int32, device=dev)
            self.tree_score = torch.empty((S, B), dtype=torch.float32, device=dev)
            self.tree_n = torch.empty(S, dtype=torch.int32, device=dev)
        if "verify" in parts:
            self.target = to_device(w.target_logits, dev)
            self.accept_len = torch.empty(S, dtype=torch.int32, device=dev)
            self.accept_path = torch.empty((S, N + 1), dtype=torch.int32, device=dev)
            self.bonus = torch.empty(S, dtype=torch.int32, device=dev)
            self.argmax = torch.empty((S, B), dtype=torch.int32, device=dev)
            self.err_verify = torch.empty(S, dtype=torch.int32, device=dev)
            nb = verify_workspace_size(S, B, cfg.V, dt)
            self.verify_ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
            # stochastic verification (temperature 1) at seeded uniforms, into its own outputs
            rng = np.random.default_rng(12345)
            self.uniform = to_device(rng.random((S, B)).astype(np.float32), dev)
            self.smp_accept_len = torch.empty(S, dtype=torch.int32, device=dev)
            self.smp_accept_path = torch.empty((S, N + 1), dtype=torch.int32, device=dev)
            self.smp_bonus = torch.empty(S, dtype=torch.int32, device=dev)
            self.smp_sample = torch.empty((S, B), dtype=torch.int32, device=dev)
            self.err_smp = torch.empty(S, dtype=torch.int32, device=dev)
            nb = verify_sampled_workspace_size(S, B, cfg.V, dt)
            self.smp_ws = torch.zeros(nb, dtype=torch.uint8, device=dev)

        if parts == ("topw", "mask", "attn", "verify"):
            self.err_step = torch.empty(S, dtype=torch.int32, device=dev)
            nb = step_workspace_size(S, B, N, W, cfg.V, cfg.Hq, cfg.Hkv, cfg.d, w.max_prefix, dt,
                                     cfg.block_size if w.block_table is not None else 0)
            self.step_ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    # ---- the four calls
    def topw(self):
        topw_per_depth(self.draft, self.cfg.W, ids=self.ids, logprob=self.logprob,
                       row_lse=self.row_lse, workspace=self.topw_ws)

    def tree(self):
        """Best-first tree construction from this step's top-W lists (not part of run())."""
        build_tree_best_first(self.ids, self.logprob, self.cfg.N, self.cfg.B,
                              parent=self.tree_parent, tokens=self.tree_tokens,
                              score=self.tree_score, n_nodes=self.tree_n)

    def commit(self):
        """The accepted paths of the last verification into the commit cache (not part of
        run())."""
        commit_accepted_kv(self.accept_len, self.accept_path, self.k_tree, self.v_tree,
                           self.commit_k, self.commit_v, self.prefix_len,
                           new_prefix_len=self.commit_len, err=self.err_commit)

    def mask(self):
        build_tree_mask(self.parent, self.anc, self.depth, self.err_mask)

    def attention(self):
        w = self.w
        tree_attention(self.q, self.k_tree, self.v_tree, self.k_prefix, self.v_prefix,
                       self.prefix_len, self.anc, block_table=self.block_table,
                       block_size=self.cfg.block_size, num_blocks=w.num_blocks or None,
                       max_prefix=w.max_prefix, out=self.attn_out, lse=self.lse,
                       err=self.err_attn, workspace=self.attn_ws)

    def verify(self):
        verify_greedy(self.target, self.parent, self.tokens, self.anc, self.depth, self.cfg.N,
                      accept_len=self.accept_len, accept_path=self.accept_path, bonus=self.bonus,
                      argmax_out=self.argmax, err=self.err_verify, workspace=self.verify_ws)

    def sampled(self, temperature=1.0):
        """Stochastic verification of the same tree (reads anc / depth of the last mask)."""
        verify_sampled(self.target, self.parent, self.tokens, self.anc, self.depth, self.cfg.N,
                       temperature, self.uniform, accept_len=self.smp_accept_len,
                       accept_path=self.smp_accept_path, bonus=self.smp_bonus,
                       sample_out=self.smp_sample, err=self.err_smp, workspace=self.smp_ws)

    def run(self):
        """The four calls in order on the current stream."""
        if "topw" in self.parts:
            self.topw()
        self.mask()
        if "attn" in self.parts:
            self.attention()
        if "verify" in self.parts:
            self.verify()

    def run_concurrent(self):
        """The same four calls with their independence exposed to the GPU: top-W (draft
        logits only) on a side stream from the start; after the mask, verification on a
        second side stream beside the attention.  Both side streams rejoin the current
        stream before return, so the step is still one stream-ordered unit (and can be
        captured into one graph).  Streams keep the default priority."""
        cur = torch.cuda.current_stream()
        if not hasattr(self, "_side"):
            self._side = (torch.cuda.Stream(device=self.dev), torch.cuda.Stream(device=self.dev))
        s_topw, s_verify = self._side
        if "topw" in self.parts:
            s_topw.wait_stream(cur)
            with torch.cuda.stream(s_topw):
                self.topw()
        self.mask()
        if "verify" in self.parts:
            s_verify.wait_stream(cur)
            with torch.cuda.stream(s_verify):
                self.verify()
        if "attn" in self.parts:
            self.attention()
        if "topw" in self.parts:
            cur.wait_stream(s_topw)
        if "verify" in self.parts:
            cur.wait_stream(s_verify)

    def run_fused(self):
        """The whole step through jt_draft_verify_step (two launches), into the same output
        buffers as the four calls; err goes to err_step."""
        w = self.w
        draft_verify_step(self.draft, self.target, self.parent, self.tokens, self.cfg.N,
                          self.cfg.W, self.q, self.k_tree, self.v_tree, self.k_prefix,
                          self.v_prefix, self.prefix_len, block_table=self.block_table,
                          block_size=self.cfg.block_size, num_blocks=w.num_blocks or None,
                          max_prefix=w.max_prefix, out=self.attn_out, lse=self.lse, ids=self.ids,
                          logprob=self.logprob, row_lse=self.row_lse, anc=self.anc,
                          depth=self.depth, accept_len=self.accept_len,
                          accept_path=self.accept_path, bonus=self.bonus, argmax_out=self.argmax,
                          err=self.err_step, workspace=self.step_ws)
