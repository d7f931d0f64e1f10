"""Device buffers for one verification step (torch is used for device memory
and streams only) and the step itself as three library calls."""
from __future__ import annotations

import numpy as np

from . import binding as sv


def _torch():
    import torch
    return torch


class StepBuffers:
    """Inputs of a Case resident in HBM, plus outputs and workspaces.

    ``inputs`` is the dict made by ``synth.make_inputs``; float32 arrays of
    bf16 cases hold bf16-representable values, so the device conversion is
    exact.
    """

    def __init__(self, case, inputs: dict, device="cuda", parts=("attn", "accept")):
        torch = _torch()
        self.case = case
        self.device = device
        c = case
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.dtype_code = sv.SV_BF16 if c.dtype == "bf16" else sv.SV_F32

        def up(a, to=None):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
            return t.to(to) if to is not None else t

        self.tau = up(inputs["tau"])
        if "attn" in parts:
            self.q = up(inputs["q"], dt)
            self.k_new = up(inputs["k_new"], dt)
            self.v_new = up(inputs["v_new"], dt)
            self.k_cache = up(inputs["k_cache"], dt)
            self.v_cache = up(inputs["v_cache"], dt)
            self.out = torch.empty_like(self.q)
            n = sv.spec_verify_attn_workspace_size(self.dtype_code, c.batch, c.block, c.prefix_len, c.n_qh,
                                                   c.n_kvh, c.head_dim)
            self.attn_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.attn_ws_bytes = n
        if "accept" in parts:
            self.target_logits = up(inputs["target_logits"])
            self.draft_probs = up(inputs["draft_probs"])
            self.draft_tokens = up(inputs["draft_tokens"])
            self.uniforms = up(inputs["uniforms"])
            self.accept_len = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.out_tokens = torch.empty((c.batch, c.block), dtype=torch.int32, device=device)
            self.alpha = torch.empty((c.batch, c.gamma), dtype=torch.float32, device=device)
            n = sv.spec_verify_accept_workspace_size(c.batch, c.block, c.gamma, c.vocab)
            self.acc_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.acc_ws_bytes = n
        if "copies" in parts:
            if not hasattr(self, "k_cache"):
                self.k_cache = up(inputs["k_cache"], dt)
                self.v_cache = up(inputs["v_cache"], dt)
            self.q_c = up(inputs["q_c"], dt)
            self.k_new_c = up(inputs["k_new_c"], dt)
            self.v_new_c = up(inputs["v_new_c"], dt)
            self.out_c = torch.empty_like(self.q_c)
            n = sv.spec_verify_attn_copies_workspace_size(self.dtype_code, c.batch, c.block, c.n_copies, c.prefix_len,
                                                          c.n_qh, c.n_kvh, c.head_dim)
            self.copies_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.copies_ws_bytes = n
        if "paged" in parts:
            self.k_pages = up(inputs["k_pages"], dt)
            self.v_pages = up(inputs["v_pages"], dt)
            self.block_table = up(inputs["block_table"])
            self.prefix_lens = up(inputs["prefix_lens"])
            self.prefix_lens0 = self.prefix_lens.clone()   # lengths before any append
            self.block_tokens = up(inputs["block_tokens"])
            self.block_tokens0 = self.block_tokens.clone()
            self.max_pages = int(inputs["block_table"].shape[1])
            self.n_pages = int(inputs["k_pages"].shape[0])
            self.remaining = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.state = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.n_append = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.append_status = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.out_paged = torch.empty_like(self.q_c if "copies" in parts else self.q)
            nc = c.n_copies if "copies" in parts else 0
            n = sv.spec_verify_attn_paged_workspace_size(self.dtype_code, c.batch, c.block, nc, c.prefix_len,
                                                         c.n_qh, c.n_kvh, c.head_dim)
            self.paged_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.paged_ws_bytes = n
        if "tree" in parts:
            N = c.n_copies
            self.tree_logits = up(inputs["tree_logits"])
            self.tree_gumbel = up(inputs["tree_gumbel"])
            self.parent, self.node_pos = up(inputs["parent"]), up(inputs["node_pos"])
            self.node_tok, self.target_pos = up(inputs["node_tok"]), up(inputs["target_pos"])
            self.path_len = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.path = torch.empty((c.batch, N), dtype=torch.int32, device=device)
            self.commit_pos = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.commit_tok = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.tree_target_tok = torch.empty((c.batch, N), dtype=torch.int32, device=device)
            n = sv.spec_verify_tree_workspace_size(c.batch, N, c.vocab)
            self.tree_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.tree_ws_bytes = n
        if "states" in parts:
            N = c.n_copies
            self.st_logits = up(inputs["st_logits"])
            self.st_gumbel = up(inputs["st_gumbel"])
            self.st_parent, self.st_state = up(inputs["st_parent"]), up(inputs["st_state"])
            self.st_path_len = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.st_path = torch.empty((c.batch, N), dtype=torch.int32, device=device)
            self.st_next = torch.empty((c.batch, c.block), dtype=torch.int32, device=device)
            self.st_commit = torch.empty((c.batch, N, c.block), dtype=torch.int32, device=device)
            self.st_conf = torch.empty((c.batch, N, c.block), dtype=torch.float32, device=device)
            n = sv.spec_verify_tree_states_workspace_size(c.batch, N, c.block, c.vocab)
            self.st_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.st_ws_bytes = n
        if "route" in parts:
            if not hasattr(self, "draft_probs"):
                self.draft_probs = up(inputs["draft_probs"])
            self.khat = torch.empty(c.batch, dtype=torch.float32, device=device)
            self.alpha_hat = torch.empty((c.batch, c.gamma), dtype=torch.float32, device=device)
            n = sv.spec_verify_route_workspace_size(c.batch, c.block, c.gamma, c.vocab)
            self.route_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.route_ws_bytes = n
        if "coupled" in parts:
            if not hasattr(self, "target_logits"):
                self.target_logits = up(inputs["target_logits"])
            self.gumbel = up(inputs["gumbel"])
            self.coupled_tokens = up(inputs["coupled_tokens"])
            self.cpl_accept_len = torch.empty(c.batch, dtype=torch.int32, device=device)
            self.cpl_out_tokens = torch.empty((c.batch, c.block), dtype=torch.int32, device=device)
            self.cpl_target_tokens = torch.empty((c.batch, c.block), dtype=torch.int32, device=device)
            n = sv.spec_verify_accept_coupled_workspace_size(c.batch, c.block, c.gamma, c.vocab)
            self.cpl_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
            self.cpl_ws_bytes = n

    def attn(self, rope_theta=None, stream=None, q=None, k_new=None):
        c = self.case
        theta = c.theta if rope_theta is None else rope_theta
        sv.spec_verify_attn(self.q if q is None else q, self.k_new if k_new is None else k_new, self.v_new,
                            self.k_cache, self.v_cache, self.tau, self.out, self.dtype_code, c.batch, c.block,
                            c.prefix_len, c.n_qh, c.n_kvh, c.head_dim, theta, 0.0, self.attn_ws,
                            self.attn_ws_bytes, stream)

    def accept(self, stream=None, temperature=None):
        """Rejection-sampling verification of the batch; with a temperature,
        the tempered call (the target distribution softmax(logits / T))."""
        c = self.case
        if temperature is None:
            sv.spec_verify_accept(self.target_logits, self.draft_probs, self.draft_tokens, self.tau, self.uniforms,
                                  c.batch, c.block, c.gamma, c.vocab, self.accept_len, self.out_tokens, self.alpha,
                                  self.acc_ws, self.acc_ws_bytes, stream)
        else:
            sv.spec_verify_accept_temperature(self.target_logits, self.draft_probs, self.draft_tokens, self.tau,
                                              self.uniforms, c.batch, c.block, c.gamma, c.vocab, temperature,
                                              self.accept_len, self.out_tokens, self.alpha, self.acc_ws,
                                              self.acc_ws_bytes, stream)

    def accept_coupled(self, stream=None, temperature=None):
        """Shared-noise (T > 0) or greedy (T = 0) verification of the batch."""
        c = self.case
        T = c.temperature if temperature is None else temperature
        sv.spec_verify_accept_coupled(self.target_logits, self.gumbel if T > 0 else None, self.coupled_tokens,
                                      self.tau, c.batch, c.block, c.gamma, c.vocab, T, self.cpl_accept_len,
                                      self.cpl_out_tokens, self.cpl_target_tokens, self.cpl_ws, self.cpl_ws_bytes,
                                      stream)

    def attn_copies(self, rope_theta=None, stream=None):
        """Multi-copy verification attention: the root and draft states of the block."""
        c = self.case
        theta = c.theta if rope_theta is None else rope_theta
        sv.spec_verify_attn_copies(self.q_c, self.k_new_c, self.v_new_c, self.k_cache, self.v_cache, self.out_c,
                                   self.dtype_code, c.batch, c.block, c.n_copies, c.prefix_len, c.n_qh, c.n_kvh,
                                   c.head_dim, theta, 0.0, self.copies_ws, self.copies_ws_bytes, stream)

    def attn_paged(self, n_copies: int = 0, rope_theta=None, max_prefix=None, stream=None):
        """Verification attention over the paged prompt cache (paired layout, or
        n_copies copies of the block), each sequence with its own length (at
        most max_prefix, default the case's prompt length; the pages have room
        for one appended block beyond it)."""
        c = self.case
        mp = c.prefix_len if max_prefix is None else max_prefix
        theta = c.theta if rope_theta is None else rope_theta
        q, kn, vn = (self.q_c, self.k_new_c, self.v_new_c) if n_copies else (self.q, self.k_new, self.v_new)
        ws, ws_bytes = self.paged_ws, self.paged_ws_bytes
        if mp != c.prefix_len:
            ws_bytes = sv.spec_verify_attn_paged_workspace_size(self.dtype_code, c.batch, c.block, n_copies, mp,
                                                                c.n_qh, c.n_kvh, c.head_dim)
            if ws_bytes > self.paged_ws.numel():
                ws = self.paged_ws = _torch().empty(ws_bytes, dtype=_torch().uint8, device=self.device)
        sv.spec_verify_attn_paged(q, kn, vn, self.k_pages, self.v_pages, self.block_table, self.prefix_lens,
                                  None if n_copies else self.tau, self.out_paged, self.dtype_code, c.batch, c.block,
                                  n_copies, mp, c.page_size, self.max_pages, self.n_pages, c.n_qh,
                                  c.n_kvh, c.head_dim, theta, 0.0, ws, ws_bytes, stream)

    def commit(self, out_tokens, stream=None):
        """Commit step: the verification's out_tokens into the block."""
        c = self.case
        sv.spec_verify_commit(out_tokens, self.block_tokens, c.batch, c.block, c.gamma, self.remaining, self.state,
                              self.n_append, stream)

    def kv_append(self, k_rows, v_rows, src_stride: int, rope_theta=None, stream=None):
        """Append each finished block's rows (n_append, as commit left it) to the
        paged prompt cache and advance the prompt lengths."""
        c = self.case
        theta = c.theta if rope_theta is None else rope_theta
        sv.spec_verify_kv_append(k_rows, v_rows, src_stride, self.n_append, self.k_pages, self.v_pages,
                                 self.block_table, self.prefix_lens, self.append_status, self.dtype_code, c.batch,
                                 c.page_size, self.max_pages, self.n_pages, c.n_kvh, c.head_dim, theta, stream)

    def tree(self, temperature=None, stream=None):
        """Draft-tree verification ("SPOT") of the case's n_copies nodes."""
        c = self.case
        T = c.temperature if temperature is None else temperature
        sv.spec_verify_tree(self.tree_logits, self.tree_gumbel if T > 0 else None, self.parent, self.node_pos,
                            self.node_tok, self.target_pos, c.batch, c.n_copies, c.vocab, T, self.path_len,
                            self.path, self.commit_pos, self.commit_tok, self.tree_target_tok, self.tree_ws,
                            self.tree_ws_bytes, stream)

    def tree_states(self, temperature=None, threshold=None, details=True, stream=None):
        """Verification of the case's tree of block states ("SPOT"): the
        target's own transition from every copy's logits, then the walk.
        details=False leaves the optional per-node outputs unwritten."""
        c = self.case
        T = c.temperature if temperature is None else temperature
        thr = c.threshold if threshold is None else threshold
        sv.spec_verify_tree_states(self.st_logits, self.st_gumbel if T > 0 else None, self.st_parent, self.st_state,
                                   c.batch, c.n_copies, c.block, c.vocab, T, thr, self.st_path_len, self.st_path,
                                   self.st_next, self.st_commit if details else None,
                                   self.st_conf if details else None, self.st_ws, self.st_ws_bytes, stream)

    def route(self, estimator: str, param: float, stream=None):
        """S2D2 verify-routing estimate K of every sequence (margin or entropy)."""
        c = self.case
        est = {"margin": sv.SV_ROUTE_MARGIN, "entropy": sv.SV_ROUTE_ENTROPY}[estimator]
        sv.spec_verify_route(self.draft_probs, self.tau, c.batch, c.block, c.gamma, c.vocab, est, param, self.khat,
                             self.alpha_hat, self.route_ws, self.route_ws_bytes, stream)

    def step(self, stream=None):
        """One verification step: attention with fused copy-aligned RoPE,
        then the acceptance epilogue."""
        self.attn(stream=stream)
        self.accept(stream=stream)
