"""CPU oracle for the speculative verification step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check (``__graft_entry__.smoke``) and
the benchmark's ``cpu_baseline`` leg may import this package.  The product
path (the HIP library and its Python binding) never imports, links or runs
anything here, and nothing here imports the product package.

Thin ctypes wrapper over ``svo.c`` (plain C, float64, OpenMP over independent
rows).  Every C function cites the passage it follows.  Parity is pinned by
``tests/test_oracle_*.py`` against facts the pages and mathematics fix
(invariants, closed forms, brute force on tiny inputs, special cases, hand
fixtures under ``tests/golden/``); ``tests/test_oracle_mutants.py`` plants
plausible mistakes in copies of ``svo.c`` and checks that a pin fails for each.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), kept as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
SRC = os.path.join(_HERE, "svo.c")
LIB = os.path.join(_HERE, "libsvo.so")
_lock = threading.Lock()
_default = None


def gcc_cmd(src: str, out: str) -> list:
    return ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
            "-shared", "-fPIC", src, "-o", out, "-lm"]


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile svo.c (or another copy) into a shared library with gcc."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.run(gcc_cmd(src, tmp), check=True)
        os.replace(tmp, out)
    return out


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc):
    if rc == -1:
        raise OracleError("tau is not a permutation of 1..B")
    if rc:
        raise OracleError(f"oracle rejected the arguments (code {rc})")


class Oracle:
    """ctypes handle on one build of svo.c (the default build, or another
    library path, e.g. a deliberately broken copy built by a test)."""

    def __init__(self, path: str | None = None):
        if path is None:
            build(force=False)
            path = LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.svo_mask.argtypes = [i32, i32, P, P]
        lib.svo_rope.argtypes = [P, i64, i32, i32, P, dbl]
        lib.svo_attn.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, dbl, dbl, P]
        lib.svo_softmax.argtypes = [P, i64, P, P, P]
        lib.svo_residual.argtypes = [P, P, i64, dbl, P, P, P]
        lib.svo_residual.restype = i64
        lib.svo_accept.argtypes = [P, P, P, P, P, i32, i32, i32, i64, ctypes.c_float, P, P, P, P]
        lib.svo_coupled_choice.argtypes = [P, P, i64, ctypes.c_float]
        lib.svo_coupled_choice.restype = i64
        lib.svo_accept_coupled.argtypes = [P, P, P, P, i32, i32, i32, i64, ctypes.c_float, P, P, P]
        lib.svo_route.argtypes = [P, P, i32, i32, i32, i64, i32, dbl, P, P]
        lib.svo_attn_copies.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, dbl, dbl, P]
        lib.svo_gather_prefix.argtypes = [P, P, i32, i32, i32, i32, i32, P]
        lib.svo_tree_verify.argtypes = [P, P, P, P, P, P, i32, i32, i64, ctypes.c_float, P, P, P, P, P]
        lib.svo_commit.argtypes = [P, P, i32, i32, i32, P, P, P]
        lib.svo_kv_append.argtypes = [P, P, i32, P, P, i32, i32, i32, i32, dbl, P, P, P]
        lib.svo_confidence.argtypes = [P, i64]
        lib.svo_confidence.restype = dbl
        lib.svo_transition.argtypes = [P, P, P, i32, i64, ctypes.c_float, ctypes.c_float, P, P]
        lib.svo_state_walk.argtypes = [P, P, P, i32, i32, i32, P, P, P]
        lib.svo_tree_states.argtypes = [P, P, P, P, i32, i32, i32, i64, ctypes.c_float, ctypes.c_float, P, P, P,
                                        P, P]
        lib.svo_set_threads.argtypes = [i32]
        self.lib = lib

    def set_threads(self, n: int) -> None:
        self.lib.svo_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.svo_max_threads())

    def mask(self, tau, P: int) -> np.ndarray:
        """Temporal-causal mask A (SimSD 关键设计 2): uint8 [2B][P+2B]."""
        tau = _c(tau, np.int32)
        B = tau.shape[0]
        M = np.empty((2 * B, P + 2 * B), np.uint8)
        _check(self.lib.svo_mask(B, P, _p(tau), _p(M)))
        return M

    def rope(self, x, pos, theta: float) -> np.ndarray:
        """Rotate-half RoPE (SimSD 关键设计 3) of x[n][heads][d] (or [n][d]) at pos[n]."""
        x = np.array(x, dtype=np.float64, copy=True)
        shp = x.shape
        if x.ndim == 2:
            x = x[:, None, :]
        n, h, d = x.shape
        pos = _c(pos, np.float64)
        assert pos.shape == (n,)
        self.lib.svo_rope(_p(x), n, h, d, _p(pos), float(theta))
        return x.reshape(shp)

    def attention(self, q, k_new, v_new, k_cache, v_cache, tau, theta: float,
                  scale: float = 0.0) -> np.ndarray:
        """Masked attention of one sequence's 2B response rows -> float64 [2B][Hq][d].

        q [2B][Hq][d], k_new/v_new [2B][Hkv][d] (pre-RoPE when theta > 0),
        k_cache/v_cache [Hkv][P][d] (prompt keys already rotated), tau [B].
        """
        q, k_new, v_new = _c(q, np.float32), _c(k_new, np.float32), _c(v_new, np.float32)
        k_cache, v_cache, tau = _c(k_cache, np.float32), _c(v_cache, np.float32), _c(tau, np.int32)
        R, Hq, d = q.shape
        B = tau.shape[0]
        assert R == 2 * B
        Hkv, P = k_cache.shape[0], k_cache.shape[1]
        assert k_new.shape == (R, Hkv, d) and v_new.shape == (R, Hkv, d)
        assert k_cache.shape == (Hkv, P, d) and v_cache.shape == (Hkv, P, d)
        out = np.empty((R, Hq, d), np.float64)
        _check(self.lib.svo_attn(_p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(tau),
                                 B, P, Hq, Hkv, d, float(theta), float(scale), _p(out)))
        return out

    def attention_copies(self, q, k_new, v_new, k_cache, v_cache, n_copies: int, theta: float,
                         scale: float = 0.0) -> np.ndarray:
        """Multi-copy verification attention of one sequence ("SPOT": the root and
        draft states as copies of the block) -> float64 [C*L][Hq][d].

        q [C*L][Hq][d], k_new/v_new [C*L][Hkv][d] copy-major (pre-RoPE when
        theta > 0), k_cache/v_cache [Hkv][P][d]."""
        q, k_new, v_new = _c(q, np.float32), _c(k_new, np.float32), _c(v_new, np.float32)
        k_cache, v_cache = _c(k_cache, np.float32), _c(v_cache, np.float32)
        R, Hq, d = q.shape
        assert R % n_copies == 0
        L = R // n_copies
        Hkv, P = k_cache.shape[0], k_cache.shape[1]
        assert k_new.shape == (R, Hkv, d) and v_new.shape == (R, Hkv, d)
        out = np.empty((R, Hq, d), np.float64)
        _check(self.lib.svo_attn_copies(_p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), L, n_copies, P,
                                        Hq, Hkv, d, float(theta), float(scale), _p(out)))
        return out

    def gather_prefix(self, pages, table_row, P: int, page_size: int) -> np.ndarray:
        """Prompt rows 0..P-1 of one sequence from a paged cache -> float32 [Hkv][P][d].

        pages [n_pages][Hkv][page_size][d]; row j sits at row j % page_size of
        page table_row[j // page_size]."""
        pages, table_row = _c(pages, np.float32), _c(table_row, np.int32)
        n_pages, Hkv, ps, d = pages.shape
        assert ps == page_size
        out = np.empty((Hkv, P, d), np.float32)
        _check(self.lib.svo_gather_prefix(_p(pages), _p(table_row), P, page_size, n_pages, Hkv, d, _p(out)))
        return out

    def attention_paged(self, q, k_new, v_new, k_pages, v_pages, block_table, prefix_lens, tau, page_size: int,
                        theta: float, n_copies: int = 0, scale: float = 0.0) -> np.ndarray:
        """Verification attention of a batch whose prompt caches are paged (or
        contiguous with a row stride, block_table None) and of per-sequence
        lengths -> float64 [batch][R][Hq][d].  Each sequence is the one-sequence
        oracle (paired layout with tau, or n_copies copies) over its own prompt
        rows, gathered by gather_prefix."""
        out = []
        for b in range(q.shape[0]):
            P = int(prefix_lens[b])
            if block_table is None:   # contiguous [batch][Hkv][stride][d]
                kc = _c(k_pages[b][:, :P], np.float32)
                vc = _c(v_pages[b][:, :P], np.float32)
            else:
                kc = self.gather_prefix(k_pages, block_table[b], P, page_size)
                vc = self.gather_prefix(v_pages, block_table[b], P, page_size)
            if n_copies == 0:
                out.append(self.attention(q[b], k_new[b], v_new[b], kc, vc, tau[b], theta, scale))
            else:
                out.append(self.attention_copies(q[b], k_new[b], v_new[b], kc, vc, n_copies, theta, scale))
        return np.stack(out) if out else np.zeros((0,) + q.shape[1:], np.float64)

    def commit(self, out_tokens, block_tokens, gamma: int):
        """Commit step (SimSD 关键设计 4) -> (block_tokens after, remaining R,
        state (0 continue / 1 fall back to denoising / 2 finished), n_append)."""
        out_tokens = _c(out_tokens, np.int32)
        bt = np.array(block_tokens, dtype=np.int32, copy=True)
        n, B = out_tokens.shape
        rem, state, napp = (np.empty(n, np.int32) for _ in range(3))
        _check(self.lib.svo_commit(_p(out_tokens), _p(bt), n, B, gamma, _p(rem), _p(state), _p(napp)))
        return bt, rem, state, napp

    def kv_append(self, k_rows, v_rows, n_append, k_pages, v_pages, block_table, prefix_lens, page_size: int,
                  theta: float, round_bf16: bool = True):
        """Append each sequence's first n_append[b] rows to its prompt cache at
        positions prefix_lens[b] + i (keys rotated there when theta > 0) ->
        (k_pages, v_pages, prefix_lens, status), new arrays.

        k_rows/v_rows [batch][stride][Hkv][d]; pages [n_pages][Hkv][page_size][d]
        with block_table [batch][max_pages], or contiguous [batch][Hkv][stride][d]
        with block_table None (page_size = the row stride).  Stored keys are
        rounded to bfloat16 (nearest, ties to even) when round_bf16, as a bf16
        cache holds them; values are stored as given."""
        k_rows, v_rows = _c(k_rows, np.float32), _c(v_rows, np.float32)
        n_append = _c(n_append, np.int32)
        pl = np.array(prefix_lens, dtype=np.int32, copy=True)
        p0 = pl.copy()
        n, S, Hkv, d = k_rows.shape
        cap = page_size * (block_table.shape[1] if block_table is not None else 1)
        ko, vo = np.zeros((n, S, Hkv, d), np.float64), np.zeros((n, S, Hkv, d), np.float64)
        st = np.empty(n, np.int32)
        _check(self.lib.svo_kv_append(_p(k_rows), _p(v_rows), S, _p(n_append), _p(pl), n, cap, Hkv, d,
                                      float(theta), _p(ko), _p(vo), _p(st)))
        kp, vp = np.array(k_pages, np.float32, copy=True), np.array(v_pages, np.float32, copy=True)
        ks = ko.astype(np.float32)
        if round_bf16:
            ks = _round_bf16(ks)
        for b in range(n):
            if st[b]:
                continue
            for i in range(int(n_append[b])):
                j = int(p0[b]) + i
                if block_table is None:
                    kp[b, :, j], vp[b, :, j] = ks[b, i], vo[b, i]
                else:
                    pg = int(block_table[b][j // page_size])
                    kp[pg, :, j % page_size], vp[pg, :, j % page_size] = ks[b, i], vo[b, i]
        return kp, vp, pl, st

    def tree_verify(self, logits, gumbel, parent, node_pos, node_tok, target_pos, temperature: float):
        """Verification of a draft tree ("SPOT"): logits/gumbel [batch][N][V] (row n:
        the target at node n's own next commit position), parent/node_pos/node_tok/
        target_pos [batch][N] -> (path_len [batch], path [batch][N], commit_pos
        [batch], commit_tok [batch], target_tok [batch][N])."""
        logits = _c(logits, np.float32)
        n, N, V = logits.shape
        g = None if gumbel is None or temperature == 0 else _c(gumbel, np.float32)
        parent, node_pos = _c(parent, np.int32), _c(node_pos, np.int32)
        node_tok, target_pos = _c(node_tok, np.int32), _c(target_pos, np.int32)
        pl, cp, ct = (np.empty(n, np.int32) for _ in range(3))
        path, tt = np.empty((n, N), np.int32), np.empty((n, N), np.int32)
        _check(self.lib.svo_tree_verify(_p(logits), _p(g), _p(parent), _p(node_pos), _p(node_tok), _p(target_pos),
                                        n, N, V, float(temperature), _p(pl), _p(path), _p(cp), _p(ct), _p(tt)))
        return pl, path, cp, ct, tt

    def softmax(self, l):
        """Float64 softmax of one logits row -> (p, m, s)."""
        l = _c(l, np.float32)
        p = np.empty(l.shape[0], np.float64)
        m = np.zeros(1, np.float64)
        s = np.zeros(1, np.float64)
        self.lib.svo_softmax(_p(l), l.shape[0], _p(p), _p(m), _p(s))
        return p, float(m[0]), float(s[0])

    def residual(self, l, pphi, u: float):
        """Residual resample of one slot -> (token, cdf[V], total mass, used_target)."""
        l, pphi = _c(l, np.float32), _c(pphi, np.float32)
        V = l.shape[0]
        cdf = np.empty(V, np.float64)
        Z = np.zeros(1, np.float64)
        ut = np.zeros(1, np.int32)
        tok = self.lib.svo_residual(_p(l), _p(pphi), V, float(u), _p(cdf), _p(Z), _p(ut))
        return int(tok), cdf, float(Z[0]), bool(ut[0])

    def accept(self, logits, probs, tokens, tau, u, gamma: int, temperature: float = 1.0):
        """Acceptance + resample for a batch (SimSD 关键设计 4).

        logits/probs [n][B][V], tokens/tau [n][B], u [n][gamma+1].  At
        temperature T the target distribution of a slot is the softmax of its
        logits times 1/T (both rounded to float32); probs are the draft's.
        Returns (accept_len[n], out_tokens[n][B], alpha[n][gamma] float64,
        resample_slot[n]).
        """
        logits, probs = _c(logits, np.float32), _c(probs, np.float32)
        tokens, tau, u = _c(tokens, np.int32), _c(tau, np.int32), _c(u, np.float32)
        n, B, V = logits.shape
        assert probs.shape == (n, B, V) and tokens.shape == (n, B) and tau.shape == (n, B)
        assert u.shape == (n, gamma + 1)
        L = np.empty(n, np.int32)
        ot = np.empty((n, B), np.int32)
        al = np.empty((n, gamma), np.float64)
        rs = np.empty(n, np.int32)
        inv_t = np.float32(1.0) / np.float32(temperature)
        _check(self.lib.svo_accept(_p(logits), _p(probs), _p(tokens), _p(tau), _p(u), n, B, gamma,
                                   V, float(inv_t), _p(L), _p(ot), _p(al), _p(rs)))
        return L, ot, al, rs


    def coupled_choice(self, l, g, temperature: float) -> int:
        """Target choice of one slot under shared-noise verification ("SPOT"):
        argmax_v fmaf(l[v], 1/T, g[v]) in float32 (T > 0), argmax_v l[v] (T = 0)."""
        l = _c(l, np.float32)
        inv_t = np.float32(1.0) / np.float32(temperature) if temperature > 0 else np.float32(0.0)
        gp = None if temperature == 0 else _c(g, np.float32)
        if gp is not None:
            assert gp.shape == l.shape
        return int(self.lib.svo_coupled_choice(_p(l), _p(gp), l.shape[0], float(inv_t)))

    def accept_coupled(self, logits, gumbel, tokens, tau, gamma: int, temperature: float):
        """Shared-noise (T > 0) or greedy (T = 0) verification of a batch ("SPOT").

        logits/gumbel [n][B][V] (gumbel may be None when T = 0), tokens/tau [n][B].
        Returns (accept_len[n], out_tokens[n][B], target_tokens[n][B]).
        """
        logits, tokens, tau = _c(logits, np.float32), _c(tokens, np.int32), _c(tau, np.int32)
        n, B, V = logits.shape
        g = None if gumbel is None else _c(gumbel, np.float32)
        if g is not None:
            assert g.shape == (n, B, V)
        L = np.empty(n, np.int32)
        ot = np.empty((n, B), np.int32)
        tt = np.empty((n, B), np.int32)
        _check(self.lib.svo_accept_coupled(_p(logits), _p(g), _p(tokens), _p(tau), n, B, gamma, V,
                                           float(np.float32(temperature)), _p(L), _p(ot), _p(tt)))
        return L, ot, tt

    def confidence(self, l) -> float:
        """Confidence of one slot ("SPOT", 动态阈值解码): max_v softmax(l)_v in float64."""
        l = _c(l, np.float32)
        return float(self.lib.svo_confidence(_p(l), l.shape[0]))

    def transition(self, logits, gumbel, state, temperature: float, threshold: float = 1.0):
        """The target's own transition at one block state: logits/gumbel [L][V]
        (gumbel None when T = 0), state [L] (-1 masked) -> (commit [L], conf [L]
        float64, number committed).  threshold >= 1: the one-commit decoder."""
        logits, state = _c(logits, np.float32), _c(state, np.int32)
        L, V = logits.shape
        inv_t = np.float32(1.0) / np.float32(temperature) if temperature > 0 else np.float32(0.0)
        g = None if temperature == 0 or gumbel is None else _c(gumbel, np.float32)
        if g is not None:
            assert g.shape == (L, V)
        commit = np.empty(L, np.int32)
        conf = np.empty(L, np.float64)
        n = self.lib.svo_transition(_p(logits), _p(g), _p(state), L, V, float(inv_t), float(np.float32(threshold)),
                                    _p(commit), _p(conf))
        return commit, conf, int(n)

    def state_walk(self, parent, state, commit):
        """The walk down trees of block states given every node's commit:
        parent [n][N], state/commit [n][N][L] -> (path_len [n], path [n][N],
        next_state [n][L])."""
        parent, state, commit = _c(parent, np.int32), _c(state, np.int32), _c(commit, np.int32)
        n, N, L = state.shape
        pl, path, ns = np.empty(n, np.int32), np.empty((n, N), np.int32), np.empty((n, L), np.int32)
        _check(self.lib.svo_state_walk(_p(parent), _p(state), _p(commit), n, N, L, _p(pl), _p(path), _p(ns)))
        return pl, path, ns

    def tree_states(self, logits, gumbel, parent, state, temperature: float, threshold: float = 1.0):
        """Verification of trees of block states ("SPOT"): logits [n][N][L][V],
        gumbel [n][L][V] (None when T = 0), parent [n][N], state [n][N][L] ->
        (path_len [n], path [n][N], next_state [n][L], commit [n][N][L],
        conf [n][N][L] float64)."""
        logits, parent, state = _c(logits, np.float32), _c(parent, np.int32), _c(state, np.int32)
        n, N, L, V = logits.shape
        assert state.shape == (n, N, L) and parent.shape == (n, N)
        g = None if temperature == 0 or gumbel is None else _c(gumbel, np.float32)
        if g is not None:
            assert g.shape == (n, L, V)
        pl, path, ns = np.empty(n, np.int32), np.empty((n, N), np.int32), np.empty((n, L), np.int32)
        commit = np.empty((n, N, L), np.int32)
        conf = np.empty((n, N, L), np.float64)
        _check(self.lib.svo_tree_states(_p(logits), _p(g), _p(parent), _p(state), n, N, L, V,
                                        float(np.float32(temperature)), float(np.float32(threshold)), _p(pl),
                                        _p(path), _p(ns), _p(commit), _p(conf)))
        return pl, path, ns, commit, conf

    def route(self, probs, tau, gamma: int, estimator: str, param: float):
        """S2D2 verify-routing estimator of a batch: probs [n][B][V], tau [n][B];
        estimator "margin" (param = threshold) or "entropy" (param = beta).
        Returns (khat[n] float64, alpha_hat[n][gamma] float64, draft order)."""
        probs, tau = _c(probs, np.float32), _c(tau, np.int32)
        n, B, V = probs.shape
        kh = np.empty(n, np.float64)
        ah = np.empty((n, gamma), np.float64)
        est = {"margin": 0, "entropy": 1}[estimator]
        _check(self.lib.svo_route(_p(probs), _p(tau), n, B, gamma, V, est, float(param), _p(kh), _p(ah)))
        return kh, ah


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle()
    return _default


def set_threads(n): return default().set_threads(n)
def max_threads(): return default().max_threads()
def mask(tau, P): return default().mask(tau, P)
def rope(x, pos, theta): return default().rope(x, pos, theta)
def attention(*a, **k): return default().attention(*a, **k)
def attention_copies(*a, **k): return default().attention_copies(*a, **k)
def attention_paged(*a, **k): return default().attention_paged(*a, **k)
def gather_prefix(*a, **k): return default().gather_prefix(*a, **k)
def commit(*a, **k): return default().commit(*a, **k)
def kv_append(*a, **k): return default().kv_append(*a, **k)
def tree_verify(*a, **k): return default().tree_verify(*a, **k)
def confidence(l): return default().confidence(l)
def transition(*a, **k): return default().transition(*a, **k)
def state_walk(*a, **k): return default().state_walk(*a, **k)
def tree_states(*a, **k): return default().tree_states(*a, **k)
def softmax(l): return default().softmax(l)
def residual(l, pphi, u): return default().residual(l, pphi, u)
def accept(*a, **k): return default().accept(*a, **k)
def coupled_choice(l, g, temperature): return default().coupled_choice(l, g, temperature)
def accept_coupled(*a, **k): return default().accept_coupled(*a, **k)
def route(*a, **k): return default().route(*a, **k)
