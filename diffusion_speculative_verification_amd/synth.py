"""Seeded synthetic inputs for the speculative verification step.

This module only draws random numbers and lays them out; it holds none of the
verification arithmetic (no RoPE, no mask, no attention, no acceptance).  Both
the CPU oracle's tests and the GPU path draw their inputs from here.

Workloads follow the block-diffusion verification setting of SimSD
("SimSD: Simple Speculative Decoding in Diffusion Language Models",
sections "数据-掩码配对布局" and "投机拒绝采样"): a cached prompt of P tokens,
a response block of B data slots D followed by B mask slots, a permutation tau
of step labels, and per-slot target logits / draft distributions over a vocab.

Recipe (per sequence b, tensor id t, case seed s; generator =
numpy default_rng(SeedSequence([s, t, b]))):
  t=0 Q      [2B][Hq][d]   iid N(0,1)          (pre-RoPE)
  t=1 K_new  [2B][Hkv][d]  iid N(0,1)          (pre-RoPE)
  t=2 V_new  [2B][Hkv][d]  iid N(0,1)
  t=3 K_cache[Hkv][P][d]   iid N(0,1)          (taken as already rotated: an
      orthogonal rotation of an iid standard normal vector is again iid
      standard normal, so this has the law of rotated raw keys)
  t=4 V_cache[Hkv][P][d]   iid N(0,1)
  t=5 tau    [B]           uniform permutation of 1..B (identity for every
      `identity_every`-th sequence, 0-based b % k == k-1)
  t=6 target logits [B][V] N(0, var_t)
  t=7 draft logits  [B][V] iid model: N(0, var_d) independent of the target;
      perturb model: target + N(0, 1)
  t=8 draft sampling uniforms [B]
  t=9 acceptance/resample uniforms [gamma+1]  U[0,1) fp32
  t=10 shared-noise rows [B][V]: standard Gumbel -log(-log U), U uniform on
      (0,1), fp32 -- the rows of the noise table at the slots' absolute
      positions ("SPOT", 前置知识 "Gumbel-Max 技巧与随机耦合")
  t=11 Q, t=12 K_new, t=13 V_new of the multi-copy layout: [C*B][heads][d]
      iid N(0,1), copy-major (the root and draft states of the block)
  t=14 per-sequence prompt length (ragged cases): uniform integer in
      [P/2, P]; otherwise P
  t=16 draft tree of case.n_copies nodes (root = node 0): each node's parent
      among the three nodes before it, the target's next commit position at
      each node (a position its path has not committed), target logits and
      Gumbel rows per node (as t=6 and t=10, at that position), and a
      synthetic drafter: a child commits at its parent's target position the
      draft's own Gumbel-max token (draft logits = target + N(0,1)) with
      probability 3/4, otherwise another (position, token); siblings differ
  t=17 tree of block states of case.n_copies nodes (root = node 0): the
      root block has a uniform number in [B/2, B] of masked slots (-1), the
      others hold uniform tokens; node k's parent is one of the three nodes
      before it that still has a masked slot (else the root).  Per node, the
      logits of every masked slot are iid N(0, var_t) in float32 (rows of
      decided slots are NaN: they must never be read), and the generator
      plants peaks: one masked slot gets +16 at a uniform token (with a
      threshold below 1: 1-3 slots get +18, and with probability 1/2 one
      more gets +13), unless logit_model is "iid".  The synthetic drafter's
      child of a node is, with probability 3/4, the node with its planted
      slots set to their planted tokens, otherwise the node with 1 (with a
      threshold: 1-3) uniform masked slots set to uniform tokens.  Noise
      rows [B][V] as t=10, shared by every node.
  t=15 (one stream for the batch) the page permutation of a paged cache: the
      sequences' page tables take consecutive runs of a random permutation of
      all pages, with one spare page per sequence that no table names
bf16 cases round Q/K/V and the caches to bf16 (round-to-nearest-even) and keep
them as float32 arrays holding exactly bf16-representable values.

The synthetic drafter: p_phi = softmax(draft logits) computed in float64 and
stored as float32; each draft token is drawn from the float64 p_phi by
inverse CDF with its own uniform.  This is input synthesis (the drafter is not
part of the verification step).

For shared-noise verification the synthetic drafter samples with the same
noise rows: its token at slot k is argmax_v (draft logit / T + G[k][v])
(float32, T = case.temperature), or argmax_v draft logit when T = 0.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Case", "CONFIGS", "make_inputs", "round_bf16", "config_by_name"]


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    batch: int
    prefix_len: int
    block: int
    gamma: int
    n_qh: int
    n_kvh: int
    head_dim: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    theta: float
    logit_model: str  # "iid" or "perturb"
    target_var: float
    draft_var: float = 1.0
    identity_every: int = 0
    seed: int = 0
    temperature: float = 1.0  # shared-noise verification (0: greedy)
    n_copies: int = 9          # multi-copy verification: root + 8 draft states
    page_size: int = 64        # paged prompt cache: rows per page
    ragged: bool = False       # paged inputs: per-sequence prompt lengths
    threshold: float = 1.0     # trees of block states: commit threshold (>= 1: one commit per step)

    @property
    def rows(self) -> int:
        return 2 * self.block

    def with_(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five workloads of the verification step (block sizes, prefix lengths,
# head counts and vocab of the block-diffusion setting; sizes as stated).
CONFIGS = [
    Case("tiny", 1, 32, 8, 8, 4, 4, 64, 512, "f32", 1e4, "iid", 2.0, 2.0, 0, seed=0),
    Case("small", 8, 512, 16, 16, 32, 8, 128, 151936, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=1),
    Case("headline", 32, 2048, 32, 32, 32, 8, 128, 151936, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=2),
    Case("longprefix", 4, 16384, 32, 32, 32, 8, 128, 151936, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=3),
    Case("wide", 64, 4096, 64, 64, 64, 8, 128, 151936, "bf16", 1e6, "perturb", 3.0, 1.0, 8, seed=4),
]


def config_by_name(name: str) -> Case:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(case: Case, tensor_id: int, b: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([case.seed, tensor_id, b]))


def _normal(case: Case, tensor_id: int, b: int, shape) -> np.ndarray:
    x = _rng(case, tensor_id, b).standard_normal(shape, dtype=np.float32)
    return round_bf16(x) if case.dtype == "bf16" else x


def _tau(case: Case, b: int) -> np.ndarray:
    if case.identity_every and (b % case.identity_every) == case.identity_every - 1:
        return np.arange(1, case.block + 1, dtype=np.int32)
    return (_rng(case, 5, b).permutation(case.block) + 1).astype(np.int32)


def _logits_and_draft(case: Case, b: int, want_logits: bool = True):
    B, V = case.block, case.vocab
    tgt = _rng(case, 6, b).standard_normal((B, V), dtype=np.float64) * np.sqrt(case.target_var)
    noise = _rng(case, 7, b).standard_normal((B, V), dtype=np.float64)
    if case.logit_model == "perturb":
        drf = tgt + noise * np.sqrt(case.draft_var)
    else:
        drf = noise * np.sqrt(case.draft_var)
    tgt32 = tgt.astype(np.float32)
    # synthetic drafter: its distribution and its sampled tokens
    drf -= drf.max(axis=1, keepdims=True)
    np.exp(drf, out=drf)
    drf /= drf.sum(axis=1, keepdims=True)
    probs32 = drf.astype(np.float32)
    u = _rng(case, 8, b).random(B)
    np.cumsum(drf, axis=1, out=drf)
    tok = np.empty(B, dtype=np.int32)
    for k in range(B):
        t = int(np.searchsorted(drf[k], u[k] * drf[k, -1], side="right"))
        tok[k] = min(t, V - 1)
    return tgt32, probs32, tok


def _coupled_noise_and_draft(case: Case, b: int):
    """Shared-noise rows of the B slots and the shared-noise drafter's tokens."""
    B, V = case.block, case.vocab
    tgt = _rng(case, 6, b).standard_normal((B, V), dtype=np.float64) * np.sqrt(case.target_var)
    noise = _rng(case, 7, b).standard_normal((B, V), dtype=np.float64)
    drf = (tgt + noise * np.sqrt(case.draft_var)) if case.logit_model == "perturb" else noise * np.sqrt(case.draft_var)
    u = _rng(case, 10, b).random((B, V))
    np.maximum(u, np.finfo(np.float64).tiny, out=u)
    g = (-np.log(-np.log(u))).astype(np.float32)
    if case.temperature > 0:
        inv_t = np.float32(1.0) / np.float32(case.temperature)
        score = drf.astype(np.float32) * inv_t + g
    else:
        score = drf
    return g, np.argmax(score, axis=1).astype(np.int32)


def _uniforms(case: Case, b: int) -> np.ndarray:
    return _rng(case, 9, b).random(case.gamma + 1, dtype=np.float32)


def make_inputs(case: Case, parts=("attn", "accept"), seqs=None, threads: int | None = None) -> dict:
    """Generate the inputs of `case` for sequences `seqs` (default: all).

    Returns a dict of float32/int32 numpy arrays with a leading batch axis:
    q [n][2B][Hq][d], k_new/v_new [n][2B][Hkv][d], k_cache/v_cache
    [n][Hkv][P][d], tau [n][B], target_logits/draft_probs [n][B][V],
    draft_tokens [n][B], uniforms [n][gamma+1]; with "coupled" in parts also
    target_logits, gumbel [n][B][V] and coupled_tokens [n][B]; with "copies"
    also q_c [n][C*B][Hq][d], k_new_c/v_new_c [n][C*B][Hkv][d] (C =
    case.n_copies) and the caches.
    """
    seqs = list(range(case.batch)) if seqs is None else list(seqs)
    n = len(seqs)
    B, R, P, d = case.block, case.rows, case.prefix_len, case.head_dim
    out = {"tau": np.stack([_tau(case, b) for b in seqs]) if n else np.zeros((0, B), np.int32)}
    if threads is None:
        threads = max(1, min(8, os.cpu_count() or 1))
    if "attn" in parts:
        out["q"] = np.empty((n, R, case.n_qh, d), np.float32)
        out["k_new"] = np.empty((n, R, case.n_kvh, d), np.float32)
        out["v_new"] = np.empty((n, R, case.n_kvh, d), np.float32)
        out["k_cache"] = np.empty((n, case.n_kvh, P, d), np.float32)
        out["v_cache"] = np.empty((n, case.n_kvh, P, d), np.float32)

        def fill_attn(i):
            b = seqs[i]
            out["q"][i] = _normal(case, 0, b, (R, case.n_qh, d))
            out["k_new"][i] = _normal(case, 1, b, (R, case.n_kvh, d))
            out["v_new"][i] = _normal(case, 2, b, (R, case.n_kvh, d))
            out["k_cache"][i] = _normal(case, 3, b, (case.n_kvh, P, d))
            out["v_cache"][i] = _normal(case, 4, b, (case.n_kvh, P, d))

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill_attn, range(n)))
    if "accept" in parts:
        V = case.vocab
        out["target_logits"] = np.empty((n, B, V), np.float32)
        out["draft_probs"] = np.empty((n, B, V), np.float32)
        out["draft_tokens"] = np.empty((n, B), np.int32)
        out["uniforms"] = np.empty((n, case.gamma + 1), np.float32)

        def fill_acc(i):
            b = seqs[i]
            t, p, k = _logits_and_draft(case, b)
            out["target_logits"][i] = t
            out["draft_probs"][i] = p
            out["draft_tokens"][i] = k
            out["uniforms"][i] = _uniforms(case, b)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill_acc, range(n)))
    if "copies" in parts:
        C, Rc = case.n_copies, case.n_copies * case.block
        out["q_c"] = np.empty((n, Rc, case.n_qh, d), np.float32)
        out["k_new_c"] = np.empty((n, Rc, case.n_kvh, d), np.float32)
        out["v_new_c"] = np.empty((n, Rc, case.n_kvh, d), np.float32)
        if "k_cache" not in out:
            out["k_cache"] = np.empty((n, case.n_kvh, P, d), np.float32)
            out["v_cache"] = np.empty((n, case.n_kvh, P, d), np.float32)
            need_cache = True
        else:
            need_cache = False

        def fill_copies(i):
            b = seqs[i]
            out["q_c"][i] = _normal(case, 11, b, (Rc, case.n_qh, d))
            out["k_new_c"][i] = _normal(case, 12, b, (Rc, case.n_kvh, d))
            out["v_new_c"][i] = _normal(case, 13, b, (Rc, case.n_kvh, d))
            if need_cache:
                out["k_cache"][i] = _normal(case, 3, b, (case.n_kvh, P, d))
                out["v_cache"][i] = _normal(case, 4, b, (case.n_kvh, P, d))

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill_copies, range(n)))
    if "coupled" in parts:
        V = case.vocab
        need_logits = "target_logits" not in out
        if need_logits:
            out["target_logits"] = np.empty((n, B, V), np.float32)
        out["gumbel"] = np.empty((n, B, V), np.float32)
        out["coupled_tokens"] = np.empty((n, B), np.int32)

        def fill_cpl(i):
            b = seqs[i]
            if need_logits:
                out["target_logits"][i] = _logits_and_draft(case, b)[0]
            g, k = _coupled_noise_and_draft(case, b)
            out["gumbel"][i] = g
            out["coupled_tokens"][i] = k

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill_cpl, range(n)))
    if "paged" in parts:
        _paged(case, out, seqs)
    if "tree" in parts:
        _tree(case, out, seqs, threads)
    if "states" in parts:
        _states(case, out, seqs, threads)
    return out


def _states(case: Case, out: dict, seqs, threads: int) -> None:
    """Trees of block states (tensor id 17): st_parent [n][N], st_state
    [n][N][B], st_logits [n][N][B][V], st_gumbel [n][B][V], N = case.n_copies."""
    n, N, B, V = len(seqs), case.n_copies, case.block, case.vocab
    sets, plant = case.threshold < 1.0, case.logit_model != "iid"
    sd = np.float32(np.sqrt(case.target_var))
    out["st_parent"] = np.full((n, N), -1, np.int32)
    out["st_state"] = np.full((n, N, B), -1, np.int32)
    out["st_logits"] = np.empty((n, N, B, V), np.float32)
    out["st_gumbel"] = np.empty((n, B, V), np.float32)

    def fill(i):
        r = _rng(case, 17, seqs[i])
        u = np.maximum(r.random((B, V)), np.finfo(np.float64).tiny)
        out["st_gumbel"][i] = (-np.log(-np.log(u))).astype(np.float32)
        st = out["st_state"][i]
        root = r.integers(0, V, B).astype(np.int32)
        root[r.choice(B, int(r.integers(max(1, B // 2), B + 1)), replace=False)] = -1
        st[0] = root
        planted = []
        for k in range(N):
            if k > 0:
                cand = [q for q in range(max(0, k - 3), k) if (st[q] < 0).any()] or [0]
                p = int(cand[int(r.integers(0, len(cand)))])
                y = st[p].copy()
                if r.random() < 0.75 and planted[p]:
                    for s_, v_ in planted[p].items():
                        y[s_] = v_
                else:
                    m = np.flatnonzero(y < 0)
                    j = min(len(m), int(r.integers(1, 4)) if sets else 1)
                    y[r.choice(m, j, replace=False)] = r.integers(0, V, j)
                out["st_parent"][i, k] = p
                st[k] = y
            lg = out["st_logits"][i, k]
            masked = np.flatnonzero(st[k] < 0)
            lg[st[k] >= 0] = np.nan
            for s_ in masked:
                lg[s_] = r.standard_normal(V, dtype=np.float32) * sd
            pk = {}
            if plant and len(masked):
                if sets:
                    hi = r.choice(masked, min(len(masked), int(r.integers(1, 4))), replace=False)
                    for s_ in hi:
                        pk[int(s_)] = int(r.integers(0, V))
                        lg[s_, pk[int(s_)]] += np.float32(18.0)
                    rest = [q for q in masked if q not in pk]
                    if rest and r.random() < 0.5:
                        q = int(rest[int(r.integers(0, len(rest)))])
                        lg[q, int(r.integers(0, V))] += np.float32(13.0)
                else:
                    s_ = int(masked[int(r.integers(0, len(masked)))])
                    pk[s_] = int(r.integers(0, V))
                    lg[s_, pk[s_]] += np.float32(16.0)
            planted.append(pk)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(n)))


def _tree(case: Case, out: dict, seqs, threads: int) -> None:
    """Draft-tree inputs (tensor id 16): parent, node_pos, node_tok, target_pos
    [n][N], tree_logits and tree_gumbel [n][N][V], N = case.n_copies."""
    n, N, V, B = len(seqs), case.n_copies, case.vocab, case.block
    shape = (n, N)
    out["parent"], out["node_pos"] = np.full(shape, -1, np.int32), np.full(shape, -1, np.int32)
    out["node_tok"], out["target_pos"] = np.full(shape, -1, np.int32), np.zeros(shape, np.int32)
    out["tree_logits"] = np.empty((n, N, V), np.float32)
    out["tree_gumbel"] = np.empty((n, N, V), np.float32)

    def fill(i):
        r = _rng(case, 16, seqs[i])
        tgt = r.standard_normal((N, V)) * np.sqrt(case.target_var)
        u = np.maximum(r.random((N, V)), np.finfo(np.float64).tiny)
        g = -np.log(-np.log(u))
        drf = tgt + r.standard_normal((N, V)) * np.sqrt(case.draft_var)
        out["tree_logits"][i], out["tree_gumbel"][i] = tgt.astype(np.float32), g.astype(np.float32)
        used = [set() for _ in range(N)]       # positions committed on each node's path
        kids = [set() for _ in range(N)]       # (position, token) of each node's children
        for k in range(N):
            if k > 0:
                p = int(r.integers(max(0, k - 3), k))
                while True:
                    if r.random() < 0.75:
                        pos = int(out["target_pos"][i, p])
                        if case.temperature > 0:
                            sc = drf[p].astype(np.float32) * (np.float32(1) / np.float32(case.temperature)) + \
                                out["tree_gumbel"][i, p]
                        else:
                            sc = drf[p]
                        tok = int(np.argmax(sc))
                    else:
                        pos, tok = int(r.integers(0, B)), int(r.integers(0, V))
                    if (pos, tok) not in kids[p] and pos not in used[p]:
                        break
                kids[p].add((pos, tok))
                out["parent"][i, k], out["node_pos"][i, k], out["node_tok"][i, k] = p, pos, tok
                used[k] = used[p] | {pos}
            free = [q for q in range(B) if q not in used[k]] or [0]
            out["target_pos"][i, k] = free[int(r.integers(0, len(free)))]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(n)))


_PAGE_FILL = 8192.0  # rows no prompt row maps to (bf16-exact; a read of one would show)


def _paged(case: Case, out: dict, seqs) -> None:
    """Paged copy of the prompt caches (made by the "attn" or "copies" part):
    prefix_lens [n], block_table [n][max_pages] (room for the prompt plus one
    appended block), k_pages / v_pages [n_pages][Hkv][page_size][d]."""
    assert "k_cache" in out, "paged inputs page the prompt caches of the attn or copies part"
    n, P, B, ps = len(seqs), case.prefix_len, case.block, case.page_size
    assert ps >= 1
    if case.ragged:
        lens = np.array([_rng(case, 14, b).integers(P // 2, P + 1) for b in seqs], np.int32)
    else:
        lens = np.full(n, P, np.int32)
    max_pages = max(1, -(-(P + B) // ps))
    n_pages = n * max_pages + n
    perm = np.random.default_rng(np.random.SeedSequence([case.seed, 15])).permutation(n_pages).astype(np.int32)
    table = perm[:n * max_pages].reshape(n, max_pages)
    shape = (n_pages, case.n_kvh, ps, case.head_dim)
    kp, vp = np.full(shape, _PAGE_FILL, np.float32), np.full(shape, _PAGE_FILL, np.float32)
    for i in range(n):
        for k in range(-(-int(lens[i]) // ps)):
            j0, j1 = k * ps, min((k + 1) * ps, int(lens[i]))
            kp[table[i, k], :, :j1 - j0] = out["k_cache"][i][:, j0:j1]
            vp[table[i, k], :, :j1 - j0] = out["v_cache"][i][:, j0:j1]
    out["prefix_lens"], out["block_table"], out["k_pages"], out["v_pages"] = lens, table, kp, vp
    out["block_tokens"] = np.full((n, B), -1, np.int32)  # a fresh block: every slot masked
