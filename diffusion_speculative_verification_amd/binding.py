"""ctypes binding of libspecverify.so -- argument marshalling only.

Functions carry the names and argument order of ``include/spec_verify.h``.
Pointer arguments accept a torch tensor (its ``data_ptr()``), a plain
integer address, or None (NULL).  ``stream`` defaults to torch's current
stream on the current device.  Every step of the computation runs in the HIP
library; a non-zero status raises ``SpecVerifyError``.  There is no fallback:
if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_E_NULL, SV_E_SHAPE, SV_E_UNSUPPORTED, SV_E_ALIGN, SV_E_WORKSPACE, SV_E_LAUNCH = 0, -1, -2, -3, -4, -5, -6
SV_E_INVALID_TAU, SV_E_SCRATCH = -7, -8
SCRATCH_BYTES = 4 << 20   # SPEC_VERIFY_SCRATCH_BYTES
SV_F32, SV_BF16 = 0, 1

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load(path: str | None = None):
    """Load the built library (raises OSError if it is missing)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"libspecverify.so not built at {p}: run __graft_entry__.build() "
                      "or python -m diffusion_speculative_verification_amd.build")
    lib = ctypes.CDLL(p)
    V, I, D, F, SZ, I64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float,
                           ctypes.c_size_t, ctypes.c_int64)
    lib.spec_verify_abi_version.restype = I
    lib.spec_verify_abi_version.argtypes = []
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [I]
    lib.spec_verify_rope.restype = I
    lib.spec_verify_rope.argtypes = [V, V, V, V, I, I, I, I, I, I, I, D, V]
    lib.spec_verify_attn_workspace_size.restype = SZ
    lib.spec_verify_attn_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.spec_verify_attn.restype = I
    lib.spec_verify_attn.argtypes = [V, V, V, V, V, V, V, I, I, I, I, I, I, I, D, F, V, SZ, V]
    lib.spec_verify_accept_workspace_size.restype = SZ
    lib.spec_verify_accept_workspace_size.argtypes = [I, I, I, I64]
    lib.spec_verify_accept.restype = I
    lib.spec_verify_accept.argtypes = [V, V, V, V, V, I, I, I, I64, V, V, V, V, SZ, V]
    lib.spec_verify_accept_noalloc.restype = I
    lib.spec_verify_accept_noalloc.argtypes = [V, V, V, V, V, I, I, I, I64, V, V, V, V]
    lib.spec_verify_accept_temperature.restype = I
    lib.spec_verify_accept_temperature.argtypes = [V, V, V, V, V, I, I, I, I64, F, V, V, V, V, SZ, V]
    lib.spec_verify_accept_coupled_workspace_size.restype = SZ
    lib.spec_verify_accept_coupled_workspace_size.argtypes = [I, I, I, I64]
    lib.spec_verify_accept_coupled.restype = I
    lib.spec_verify_accept_coupled.argtypes = [V, V, V, V, I, I, I, I64, F, V, V, V, V, SZ, V]
    lib.spec_verify_attn_copies_workspace_size.restype = SZ
    lib.spec_verify_attn_copies_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.spec_verify_attn_copies.restype = I
    lib.spec_verify_attn_copies.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, I, I, D, F, V, SZ, V]
    lib.spec_verify_attn_paged_workspace_size.restype = SZ
    lib.spec_verify_attn_paged_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.spec_verify_attn_paged.restype = I
    lib.spec_verify_attn_paged.argtypes = [V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, I, I, I, I, I, D, F, V,
                                           SZ, V]
    lib.spec_verify_tree_workspace_size.restype = SZ
    lib.spec_verify_tree_workspace_size.argtypes = [I, I, I64]
    lib.spec_verify_tree.restype = I
    lib.spec_verify_tree.argtypes = [V, V, V, V, V, V, I, I, I64, F, V, V, V, V, V, V, SZ, V]
    lib.spec_verify_tree_states_workspace_size.restype = SZ
    lib.spec_verify_tree_states_workspace_size.argtypes = [I, I, I, I64]
    lib.spec_verify_tree_states.restype = I
    lib.spec_verify_tree_states.argtypes = [V, V, V, V, I, I, I, I64, F, F, V, V, V, V, V, V, SZ, V]
    lib.spec_verify_check_tau.restype = I
    lib.spec_verify_check_tau.argtypes = [V, I, I, V, V]
    lib.spec_verify_commit.restype = I
    lib.spec_verify_commit.argtypes = [V, V, I, I, I, V, V, V, V]
    lib.spec_verify_kv_append.restype = I
    lib.spec_verify_kv_append.argtypes = [V, V, I, V, V, V, V, V, V, I, I, I, I, I, I, I, D, V]
    lib.spec_verify_route_workspace_size.restype = SZ
    lib.spec_verify_route_workspace_size.argtypes = [I, I, I, I64]
    lib.spec_verify_route.restype = I
    lib.spec_verify_route.argtypes = [V, V, I, I, I, I64, I, D, V, V, V, SZ, V]
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int):
    if rc != SV_OK:
        raise SpecVerifyError(rc, spec_verify_status_string(rc))


def spec_verify_abi_version() -> int:
    return load().spec_verify_abi_version()


def spec_verify_status_string(status: int) -> str:
    return load().spec_verify_status_string(status).decode()


def spec_verify_rope(q_in, k_in, q_out, k_out, dtype, batch, block, n_qh, n_kvh, head_dim, prefix_len,
                     theta, stream=None) -> None:
    _check(load().spec_verify_rope(_ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out), dtype, batch, block,
                                   n_qh, n_kvh, head_dim, prefix_len, float(theta), _stream(stream)))


def spec_verify_attn_workspace_size(dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim) -> int:
    return int(load().spec_verify_attn_workspace_size(dtype, batch, block, prefix_len, n_qh, n_kvh, head_dim))


def spec_verify_attn(q, k_new, v_new, k_cache, v_cache, tau, out, dtype, batch, block, prefix_len, n_qh,
                     n_kvh, head_dim, rope_theta, softmax_scale, workspace, workspace_bytes,
                     stream=None) -> None:
    _check(load().spec_verify_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(tau), _ptr(out), dtype, batch, block, prefix_len, n_qh, n_kvh,
                                   head_dim, float(rope_theta), float(softmax_scale), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)))


def spec_verify_accept_workspace_size(batch, block, gamma, vocab) -> int:
    return int(load().spec_verify_accept_workspace_size(batch, block, gamma, vocab))


def spec_verify_accept(target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block, gamma, vocab,
                       accept_len, out_tokens, alpha, workspace, workspace_bytes, stream=None) -> None:
    _check(load().spec_verify_accept(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(tau),
                                     _ptr(uniforms), batch, block, gamma, vocab, _ptr(accept_len),
                                     _ptr(out_tokens), _ptr(alpha), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream)))


def spec_verify_accept_noalloc(target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block, gamma, vocab,
                               accept_len, out_tokens, alpha, stream=None) -> None:
    _check(load().spec_verify_accept_noalloc(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(tau),
                                             _ptr(uniforms), batch, block, gamma, vocab, _ptr(accept_len),
                                             _ptr(out_tokens), _ptr(alpha), _stream(stream)))


def spec_verify_accept_temperature(target_logits, draft_probs, draft_tokens, tau, uniforms, batch, block, gamma,
                                   vocab, temperature, accept_len, out_tokens, alpha, workspace, workspace_bytes,
                                   stream=None) -> None:
    _check(load().spec_verify_accept_temperature(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens),
                                                 _ptr(tau), _ptr(uniforms), batch, block, gamma, vocab,
                                                 float(temperature), _ptr(accept_len), _ptr(out_tokens),
                                                 _ptr(alpha), _ptr(workspace), int(workspace_bytes),
                                                 _stream(stream)))


def spec_verify_accept_coupled_workspace_size(batch, block, gamma, vocab) -> int:
    return int(load().spec_verify_accept_coupled_workspace_size(batch, block, gamma, vocab))


def spec_verify_accept_coupled(target_logits, gumbel, draft_tokens, tau, batch, block, gamma, vocab, temperature,
                               accept_len, out_tokens, target_tokens, workspace, workspace_bytes,
                               stream=None) -> None:
    _check(load().spec_verify_accept_coupled(_ptr(target_logits), _ptr(gumbel), _ptr(draft_tokens), _ptr(tau),
                                             batch, block, gamma, vocab, float(temperature), _ptr(accept_len),
                                             _ptr(out_tokens), _ptr(target_tokens), _ptr(workspace),
                                             int(workspace_bytes), _stream(stream)))


SV_ROUTE_MARGIN, SV_ROUTE_ENTROPY = 0, 1


def spec_verify_route_workspace_size(batch, block, gamma, vocab) -> int:
    return int(load().spec_verify_route_workspace_size(batch, block, gamma, vocab))


def spec_verify_route(draft_probs, tau, batch, block, gamma, vocab, estimator, param, khat, alpha_hat, workspace,
                      workspace_bytes, stream=None) -> None:
    _check(load().spec_verify_route(_ptr(draft_probs), _ptr(tau), batch, block, gamma, vocab, int(estimator),
                                    float(param), _ptr(khat), _ptr(alpha_hat), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream)))


def spec_verify_attn_copies_workspace_size(dtype, batch, block, n_copies, prefix_len, n_qh, n_kvh, head_dim) -> int:
    return int(load().spec_verify_attn_copies_workspace_size(dtype, batch, block, n_copies, prefix_len, n_qh, n_kvh,
                                                             head_dim))


def spec_verify_attn_copies(q, k_new, v_new, k_cache, v_cache, out, dtype, batch, block, n_copies, prefix_len, n_qh,
                            n_kvh, head_dim, rope_theta, softmax_scale, workspace, workspace_bytes,
                            stream=None) -> None:
    _check(load().spec_verify_attn_copies(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                          dtype, batch, block, n_copies, prefix_len, n_qh, n_kvh, head_dim,
                                          float(rope_theta), float(softmax_scale), _ptr(workspace),
                                          int(workspace_bytes), _stream(stream)))


def spec_verify_attn_paged_workspace_size(dtype, batch, block, n_copies, max_prefix, n_qh, n_kvh, head_dim) -> int:
    return int(load().spec_verify_attn_paged_workspace_size(dtype, batch, block, n_copies, max_prefix, n_qh, n_kvh,
                                                            head_dim))


def spec_verify_attn_paged(q, k_new, v_new, k_pages, v_pages, block_table, prefix_lens, tau, out, dtype, batch,
                           block, n_copies, max_prefix, page_size, max_pages, n_pages, n_qh, n_kvh, head_dim,
                           rope_theta, softmax_scale, workspace, workspace_bytes, stream=None) -> None:
    _check(load().spec_verify_attn_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                         _ptr(block_table), _ptr(prefix_lens), _ptr(tau), _ptr(out), dtype, batch,
                                         block, n_copies, max_prefix, page_size, max_pages, n_pages, n_qh, n_kvh,
                                         head_dim, float(rope_theta), float(softmax_scale), _ptr(workspace),
                                         int(workspace_bytes), _stream(stream)))


def spec_verify_commit(out_tokens, block_tokens, batch, block, gamma, remaining, state, n_append,
                       stream=None) -> None:
    _check(load().spec_verify_commit(_ptr(out_tokens), _ptr(block_tokens), batch, block, gamma, _ptr(remaining),
                                     _ptr(state), _ptr(n_append), _stream(stream)))


def spec_verify_kv_append(k_rows, v_rows, src_stride, n_append, k_pages, v_pages, block_table, prefix_lens, status,
                          dtype, batch, page_size, max_pages, n_pages, n_kvh, head_dim, rope_theta,
                          stream=None) -> None:
    _check(load().spec_verify_kv_append(_ptr(k_rows), _ptr(v_rows), src_stride, _ptr(n_append), _ptr(k_pages),
                                        _ptr(v_pages), _ptr(block_table), _ptr(prefix_lens), _ptr(status), dtype,
                                        batch, page_size, max_pages, n_pages, n_kvh, head_dim, float(rope_theta),
                                        _stream(stream)))


def spec_verify_check_tau(tau, batch, block, bad, stream=None) -> None:
    _check(load().spec_verify_check_tau(_ptr(tau), batch, block, _ptr(bad), _stream(stream)))


def spec_verify_tree_workspace_size(batch, n_nodes, vocab) -> int:
    return int(load().spec_verify_tree_workspace_size(batch, n_nodes, vocab))


def spec_verify_tree_states_workspace_size(batch, n_nodes, block, vocab) -> int:
    return int(load().spec_verify_tree_states_workspace_size(batch, n_nodes, block, vocab))


def spec_verify_tree_states(target_logits, gumbel, parent, state, batch, n_nodes, block, vocab, temperature,
                            threshold, path_len, path, next_state, commit, confidence, workspace, workspace_bytes,
                            stream=None) -> None:
    _check(load().spec_verify_tree_states(_ptr(target_logits), _ptr(gumbel), _ptr(parent), _ptr(state), batch,
                                          n_nodes, block, int(vocab), float(temperature), float(threshold),
                                          _ptr(path_len), _ptr(path), _ptr(next_state), _ptr(commit),
                                          _ptr(confidence), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def spec_verify_tree(target_logits, gumbel, parent, node_pos, node_tok, target_pos, batch, n_nodes, vocab,
                     temperature, path_len, path, commit_pos, commit_tok, target_tok, workspace, workspace_bytes,
                     stream=None) -> None:
    _check(load().spec_verify_tree(_ptr(target_logits), _ptr(gumbel), _ptr(parent), _ptr(node_pos), _ptr(node_tok),
                                   _ptr(target_pos), batch, n_nodes, int(vocab), float(temperature), _ptr(path_len),
                                   _ptr(path), _ptr(commit_pos), _ptr(commit_tok), _ptr(target_tok),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream)))
