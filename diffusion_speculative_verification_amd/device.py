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

    def accept(self, stream=None):
        c = self.case
        sv.spec_verify_accept(self.target_logits, self.draft_probs, self.draft_tokens, self.tau, self.uniforms,
                              c.batch, c.block, c.gamma, c.vocab, self.accept_len, self.out_tokens, self.alpha,
                              self.acc_ws, self.acc_ws_bytes, stream)

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
