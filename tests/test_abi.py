"""The C-ABI library: it loads, exports every symbol the header declares, and
its host-side argument checks return the documented status codes without
touching a GPU (CPU only)."""
import os
import re

import pytest

from diffusion_speculative_verification_amd import binding as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sv.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 24
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    hdr = open(HEADER).read()
    assert sv.spec_verify_abi_version() == int(re.search(r"#define SPEC_VERIFY_ABI_VERSION (\d+)", hdr).group(1))
    for code in range(0, -9, -1):
        assert sv.spec_verify_status_string(code)
    assert sv.spec_verify_status_string(-99) == "unknown status"


def test_workspace_sizes(lib):
    # bf16 headline shape needs no split; the long-prefix shape splits
    assert sv.spec_verify_attn_workspace_size(1, 32, 32, 2048, 32, 8, 128) == 0
    assert sv.spec_verify_attn_workspace_size(1, 4, 32, 16384, 32, 8, 128) > 0
    assert sv.spec_verify_attn_workspace_size(0, 1, 8, 32, 4, 4, 64) > 0   # fp32 rope copies
    assert sv.spec_verify_attn_workspace_size(1, 1, 8, 32, 4, 4, 96) == 0  # unsupported -> 0
    assert sv.spec_verify_accept_workspace_size(32, 32, 32, 151936) > 0
    assert sv.spec_verify_accept_workspace_size(32, 32, 33, 151936) == 0  # gamma > block


A = 1 << 20  # a fake, 16-byte aligned "device" address; never dereferenced


def attn(lib, **kw):
    args = dict(q=A, k_new=A, v_new=A, k_cache=A, v_cache=A, tau=A, out=A, dtype=1, batch=1, block=8,
                prefix=32, n_qh=4, n_kvh=4, head_dim=64, theta=1e4, scale=0.0, ws=A, ws_bytes=1 << 30)
    args.update(kw)
    return lib.spec_verify_attn(args["q"], args["k_new"], args["v_new"], args["k_cache"], args["v_cache"],
                                args["tau"], args["out"], args["dtype"], args["batch"], args["block"],
                                args["prefix"], args["n_qh"], args["n_kvh"], args["head_dim"], args["theta"],
                                args["scale"], args["ws"], args["ws_bytes"], None)


def test_attn_argument_checks(lib):
    assert attn(lib, q=None) == sv.SV_E_NULL
    assert attn(lib, k_cache=None) == sv.SV_E_NULL
    assert attn(lib, head_dim=96) == sv.SV_E_UNSUPPORTED
    assert attn(lib, dtype=7) == sv.SV_E_UNSUPPORTED
    assert attn(lib, n_qh=6, n_kvh=4) == sv.SV_E_SHAPE
    assert attn(lib, block=65) == sv.SV_E_SHAPE
    assert attn(lib, block=0) == sv.SV_E_SHAPE
    assert attn(lib, prefix=-1) == sv.SV_E_SHAPE
    assert attn(lib, q=A + 8) == sv.SV_E_ALIGN
    assert attn(lib, dtype=0, ws=None) == sv.SV_E_WORKSPACE  # fp32 + rope needs workspace
    assert attn(lib, dtype=0, ws_bytes=16) == sv.SV_E_WORKSPACE
    assert attn(lib, batch=4, prefix=16384, block=32, n_qh=32, n_kvh=8, head_dim=128, ws=None) == sv.SV_E_WORKSPACE


def accept(lib, **kw):
    args = dict(tl=A, dp=A, dt=A, tau=A, u=A, batch=2, block=8, gamma=8, vocab=512, L=A, ot=A, al=A, ws=A,
                ws_bytes=1 << 30)
    args.update(kw)
    return lib.spec_verify_accept(args["tl"], args["dp"], args["dt"], args["tau"], args["u"], args["batch"],
                                  args["block"], args["gamma"], args["vocab"], args["L"], args["ot"], args["al"],
                                  args["ws"], args["ws_bytes"], None)


def test_accept_argument_checks(lib):
    assert accept(lib, tl=None) == sv.SV_E_NULL
    assert accept(lib, L=None) == sv.SV_E_NULL
    assert accept(lib, gamma=9) == sv.SV_E_SHAPE
    assert accept(lib, gamma=0) == sv.SV_E_SHAPE
    assert accept(lib, vocab=0) == sv.SV_E_SHAPE
    assert accept(lib, block=65, gamma=8) == sv.SV_E_SHAPE
    assert accept(lib, u=A + 4) == sv.SV_E_ALIGN
    assert accept(lib, ws=None) == sv.SV_E_WORKSPACE
    assert accept(lib, ws_bytes=8) == sv.SV_E_WORKSPACE
    # batch * block beyond 2^26 rows, or batch * block * vocab beyond 2^40
    assert accept(lib, batch=1 << 21, block=64, gamma=8, vocab=4) == sv.SV_E_SHAPE
    assert accept(lib, batch=1 << 14, block=64, gamma=8, vocab=1 << 21) == sv.SV_E_SHAPE
    assert sv.spec_verify_accept_workspace_size(1 << 21, 64, 8, 4) == 0
    assert sv.spec_verify_route_workspace_size(1 << 21, 64, 8, 4) == 0


def test_accept_temperature_argument_checks(lib):
    f = lib.spec_verify_accept_temperature

    def call(T, **kw):
        a = dict(tl=A, dp=A, dt=A, tau=A, u=A, batch=2, block=8, gamma=8, vocab=512, L=A, ot=A, al=A, ws=None,
                 ws_bytes=0)
        a.update(kw)
        return f(a["tl"], a["dp"], a["dt"], a["tau"], a["u"], a["batch"], a["block"], a["gamma"], a["vocab"], T,
                 a["L"], a["ot"], a["al"], a["ws"], a["ws_bytes"], None)
    for T in (0.0, -1.0, float("inf"), float("nan"), 1e-45):   # 1e-45: 1/T overflows float32
        assert call(T) == sv.SV_E_SHAPE, T
    assert call(0.7) == sv.SV_E_WORKSPACE      # checks pass up to the missing workspace: nothing launched
    assert call(0.7, tl=None) == sv.SV_E_NULL
    assert call(0.7, gamma=9) == sv.SV_E_SHAPE


def coupled(lib, **kw):
    args = dict(tl=A, g=A, dt=A, tau=A, batch=2, block=8, gamma=8, vocab=512, T=1.0, L=A, ot=A, tt=A, ws=A,
                ws_bytes=1 << 30)
    args.update(kw)
    return lib.spec_verify_accept_coupled(args["tl"], args["g"], args["dt"], args["tau"], args["batch"],
                                          args["block"], args["gamma"], args["vocab"], args["T"], args["L"],
                                          args["ot"], args["tt"], args["ws"], args["ws_bytes"], None)


def test_coupled_argument_checks(lib):
    assert sv.spec_verify_accept_coupled_workspace_size(32, 32, 32, 151936) > 0
    assert sv.spec_verify_accept_coupled_workspace_size(32, 32, 33, 151936) == 0
    assert coupled(lib, tl=None) == sv.SV_E_NULL
    assert coupled(lib, g=None) == sv.SV_E_NULL            # noise needed at T > 0
    assert coupled(lib, g=None, T=0.0, ws=None) == sv.SV_E_WORKSPACE  # greedy: noise not needed
    assert coupled(lib, T=-1.0) == sv.SV_E_SHAPE
    assert coupled(lib, T=float("inf")) == sv.SV_E_SHAPE
    assert coupled(lib, T=float("nan")) == sv.SV_E_SHAPE
    assert coupled(lib, T=1e-45) == sv.SV_E_SHAPE          # 1/T overflows float32
    assert coupled(lib, gamma=9) == sv.SV_E_SHAPE
    assert coupled(lib, g=A + 4) == sv.SV_E_ALIGN
    assert coupled(lib, tt=A + 4) == sv.SV_E_ALIGN
    assert coupled(lib, ws_bytes=4) == sv.SV_E_WORKSPACE
    assert coupled(lib, batch=1 << 21, block=64, gamma=8, vocab=4) == sv.SV_E_SHAPE


def route(lib, **kw):
    args = dict(dp=A, tau=A, batch=2, block=8, gamma=8, vocab=512, est=1, param=1.0, kh=A, ah=A, ws=A,
                ws_bytes=1 << 30)
    args.update(kw)
    return lib.spec_verify_route(args["dp"], args["tau"], args["batch"], args["block"], args["gamma"],
                                 args["vocab"], args["est"], args["param"], args["kh"], args["ah"], args["ws"],
                                 args["ws_bytes"], None)


def test_route_argument_checks(lib):
    assert sv.spec_verify_route_workspace_size(32, 32, 32, 151936) > 0
    assert sv.spec_verify_route_workspace_size(32, 32, 0, 151936) == 0
    assert route(lib, dp=None) == sv.SV_E_NULL
    assert route(lib, kh=None) == sv.SV_E_NULL
    assert route(lib, est=2) == sv.SV_E_UNSUPPORTED
    assert route(lib, param=float("nan")) == sv.SV_E_SHAPE
    assert route(lib, gamma=9) == sv.SV_E_SHAPE
    assert route(lib, ah=A + 4) == sv.SV_E_ALIGN
    assert route(lib, ws=None) == sv.SV_E_WORKSPACE


def test_copies_argument_checks(lib):
    f = lib.spec_verify_attn_copies
    ok = dict(q=A, k=A, v=A, kc=A, vc=A, o=A, dt=1, b=1, L=32, C=9, P=64, hq=4, hkv=4, d=128, th=1e6, sc=0.0,
              ws=A, wb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["o"], a["dt"], a["b"], a["L"], a["C"], a["P"], a["hq"],
                 a["hkv"], a["d"], a["th"], a["sc"], a["ws"], a["wb"], None)
    assert sv.spec_verify_attn_copies_workspace_size(1, 1, 32, 9, 2048, 4, 4, 128) > 0   # prefix split
    assert sv.spec_verify_attn_copies_workspace_size(1, 64, 32, 9, 2048, 32, 8, 128) == 0  # enough workgroups
    assert sv.spec_verify_attn_copies_workspace_size(1, 1, 32, 33, 64, 4, 4, 128) == 0  # 33 * 32 > 1024
    assert call(P=2048, wb=0) == sv.SV_E_WORKSPACE
    assert call(q=None) == sv.SV_E_NULL
    assert call(kc=None) == sv.SV_E_NULL
    assert call(dt=0) == sv.SV_E_UNSUPPORTED
    assert call(C=0) == sv.SV_E_SHAPE
    assert call(C=33) == sv.SV_E_SHAPE
    assert call(L=65, C=2) == sv.SV_E_SHAPE
    assert call(o=A + 8) == sv.SV_E_ALIGN


def test_paged_argument_checks(lib):
    f = lib.spec_verify_attn_paged
    ok = dict(q=A, k=A, v=A, kp=A, vp=A, tb=A, pl=A, tau=A, o=A, dt=1, b=2, L=32, C=0, P=2048, ps=64, mp=33, npg=66,
              hq=32, hkv=8, d=128, th=1e6, sc=0.0, ws=A, wb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["kp"], a["vp"], a["tb"], a["pl"], a["tau"], a["o"], a["dt"], a["b"],
                 a["L"], a["C"], a["P"], a["ps"], a["mp"], a["npg"], a["hq"], a["hkv"], a["d"], a["th"], a["sc"],
                 a["ws"], a["wb"], None)
    assert sv.spec_verify_attn_paged_workspace_size(1, 2, 32, 0, 2048, 32, 8, 128) > 0   # few units: splits
    assert sv.spec_verify_attn_paged_workspace_size(0, 2, 32, 0, 2048, 32, 8, 128) == 0  # fp32: unsupported
    assert call(dt=0) == sv.SV_E_UNSUPPORTED
    assert call(ps=96) == sv.SV_E_SHAPE            # pages must hold whole 64-key tiles
    assert call(mp=31) == sv.SV_E_SHAPE            # 31 * 64 < 2048
    assert call(npg=0) == sv.SV_E_SHAPE
    assert call(C=-1) == sv.SV_E_SHAPE
    assert call(tb=None, ps=1000) == sv.SV_E_SHAPE   # contiguous stride below the longest prompt
    assert call(tau=None) == sv.SV_E_NULL
    assert call(tau=None, C=9, wb=0) == sv.SV_E_WORKSPACE   # copies need no tau (stops before any launch)
    assert call(kp=None) == sv.SV_E_NULL
    assert call(o=A + 4) == sv.SV_E_ALIGN
    assert call(wb=0) == sv.SV_E_WORKSPACE


def test_tree_states_argument_checks(lib):
    f = lib.spec_verify_tree_states
    ok = dict(l=A, g=A, par=A, st=A, b=32, n=9, L=32, V=151936, T=1.0, thr=1.0, pl=A, path=A, ns=A, cm=A, cf=A,
              ws=A, wb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["l"], a["g"], a["par"], a["st"], a["b"], a["n"], a["L"], a["V"], a["T"], a["thr"], a["pl"],
                 a["path"], a["ns"], a["cm"], a["cf"], a["ws"], a["wb"], None)
    ws = sv.spec_verify_tree_states_workspace_size(32, 9, 32, 151936)
    assert ws >= 32 * 9 * 32 * 24
    assert sv.spec_verify_tree_states_workspace_size(32, 65, 32, 151936) == 0
    assert sv.spec_verify_tree_states_workspace_size(32, 9, 65, 151936) == 0
    assert sv.spec_verify_tree_states_workspace_size(32, 9, 32, (1 << 21) + 1) == 0
    assert call(n=65) == sv.SV_E_SHAPE
    assert call(L=0) == sv.SV_E_SHAPE
    assert call(L=65) == sv.SV_E_SHAPE
    assert call(T=-1.0) == sv.SV_E_SHAPE
    assert call(T=float("nan")) == sv.SV_E_SHAPE
    assert call(thr=float("nan")) == sv.SV_E_SHAPE
    assert call(T=1e-45) == sv.SV_E_SHAPE          # 1/T overflows float32
    assert call(b=(1 << 14) + 1, n=64, L=64, V=4) == sv.SV_E_SHAPE  # more than 2^26 rows
    assert call(g=None) == sv.SV_E_NULL            # T > 0 needs the noise rows
    assert call(st=None) == sv.SV_E_NULL
    assert call(ns=None) == sv.SV_E_NULL
    assert call(l=A + 4) == sv.SV_E_ALIGN
    assert call(g=A + 8) == sv.SV_E_ALIGN
    assert call(wb=ws - 1) == sv.SV_E_WORKSPACE
    assert call(ws=A + 4, wb=ws) == sv.SV_E_ALIGN


def test_tree_argument_checks(lib):
    f = lib.spec_verify_tree
    ok = dict(l=A, g=A, par=A, pos=A, tok=A, tp=A, b=4, n=9, V=151936, T=1.0, pl=A, path=A, cp=A, ct=A, tt=A,
              ws=A, wb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["l"], a["g"], a["par"], a["pos"], a["tok"], a["tp"], a["b"], a["n"], a["V"], a["T"], a["pl"],
                 a["path"], a["cp"], a["ct"], a["tt"], a["ws"], a["wb"], None)
    assert sv.spec_verify_tree_workspace_size(4, 9, 151936) > 0
    assert sv.spec_verify_tree_workspace_size(4, 65, 151936) == 0
    assert call(n=65) == sv.SV_E_SHAPE
    assert call(n=0) == sv.SV_E_SHAPE
    assert call(T=-1.0) == sv.SV_E_SHAPE
    assert call(T=float("inf")) == sv.SV_E_SHAPE
    assert call(T=1e-45) == sv.SV_E_SHAPE          # 1/T overflows float32
    assert call(b=1 << 21, n=64, V=4) == sv.SV_E_SHAPE  # more than 2^26 nodes
    assert sv.spec_verify_tree_workspace_size(1 << 21, 64, 4) == 0
    assert call(g=None) == sv.SV_E_NULL            # T > 0 needs the noise rows
    assert call(par=None) == sv.SV_E_NULL
    assert call(l=A + 4) == sv.SV_E_ALIGN
    assert call(wb=0) == sv.SV_E_WORKSPACE


def test_commit_and_append_argument_checks(lib):
    assert lib.spec_verify_check_tau(A, 4, 65, A, None) == sv.SV_E_SHAPE
    assert lib.spec_verify_check_tau(None, 4, 32, A, None) == sv.SV_E_NULL
    assert "tau" in sv.spec_verify_status_string(sv.SV_E_INVALID_TAU)
    c = lib.spec_verify_commit
    assert c(A, A, 4, 32, 33, A, A, A, None) == sv.SV_E_SHAPE      # gamma > block
    assert c(A, A, 4, 65, 8, A, A, A, None) == sv.SV_E_SHAPE       # block > 64
    assert c(None, A, 4, 32, 8, A, A, A, None) == sv.SV_E_NULL
    f = lib.spec_verify_kv_append
    ok = dict(k=A, v=A, S=64, na=A, kp=A, vp=A, tb=A, pl=A, st=A, dt=1, b=4, ps=64, mp=33, npg=132, hkv=8, d=128,
              th=1e6)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["k"], a["v"], a["S"], a["na"], a["kp"], a["vp"], a["tb"], a["pl"], a["st"], a["dt"], a["b"],
                 a["ps"], a["mp"], a["npg"], a["hkv"], a["d"], a["th"], None)
    assert call(dt=0) == sv.SV_E_UNSUPPORTED
    assert call(d=96) == sv.SV_E_UNSUPPORTED
    assert call(S=0) == sv.SV_E_SHAPE
    assert call(mp=0) == sv.SV_E_SHAPE
    assert call(th=float("nan")) == sv.SV_E_SHAPE
    assert call(pl=None) == sv.SV_E_NULL
    assert call(kp=A + 2) == sv.SV_E_ALIGN


def test_rope_argument_checks(lib):
    f = lib.spec_verify_rope
    assert f(None, A, A, A, 1, 1, 8, 4, 4, 64, 32, 1e4, None) == sv.SV_E_NULL
    assert f(A, A, A, A, 1, 1, 8, 4, 4, 64, 32, 0.0, None) == sv.SV_E_SHAPE
    assert f(A, A, A, A, 1, 1, 8, 4, 4, 80, 32, 1e4, None) == sv.SV_E_UNSUPPORTED
    assert f(A, A, A + 2, A, 1, 1, 8, 4, 4, 64, 32, 1e4, None) == sv.SV_E_ALIGN


def test_binding_raises(lib):
    with pytest.raises(sv.SpecVerifyError) as ei:
        sv.spec_verify_rope(None, A, A, A, 1, 1, 8, 4, 4, 64, 32, 1e4, stream=0)
    assert ei.value.status == sv.SV_E_NULL


def test_accept_noalloc_argument_checks(lib):
    """The allocation-free epilogue checks its arguments on the host like
    spec_verify_accept, and refuses sizes beyond its static scratch buffer
    before it touches a device."""
    def call(**kw):
        a = dict(l=A, p=A, x=A, tau=A, u=A, batch=2, block=8, gamma=8, vocab=1000, L=A, tok=A, alpha=None)
        a.update(kw)
        return lib.spec_verify_accept_noalloc(a["l"], a["p"], a["x"], a["tau"], a["u"], a["batch"], a["block"],
                                              a["gamma"], a["vocab"], a["L"], a["tok"], a["alpha"], None)
    assert call(l=None) == sv.SV_E_NULL
    assert call(tok=None) == sv.SV_E_NULL
    assert call(gamma=9) == sv.SV_E_SHAPE
    assert call(block=65, gamma=1) == sv.SV_E_SHAPE
    assert call(vocab=(1 << 21) + 1) == sv.SV_E_SHAPE
    assert call(u=A + 4) == sv.SV_E_ALIGN
    assert call(alpha=A + 8) == sv.SV_E_ALIGN
    # 2^18 slots need ~8 MiB of partials: more than the 4 MiB buffer
    big = dict(batch=1 << 12, block=64, gamma=64, vocab=1 << 14)
    assert sv.spec_verify_accept_workspace_size(big["batch"], 64, 64, big["vocab"]) > sv.SCRATCH_BYTES
    assert call(**big) == sv.SV_E_SCRATCH
    # the headline and widest workloads fit
    assert sv.spec_verify_accept_workspace_size(32, 32, 32, 151936) <= sv.SCRATCH_BYTES
    assert sv.spec_verify_accept_workspace_size(64, 64, 64, 151936) <= sv.SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert sv.SCRATCH_BYTES == eval(re.search(r"#define SPEC_VERIFY_SCRATCH_BYTES \((.*)\)", hdr).group(1))
