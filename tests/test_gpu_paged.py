"""Paged prompt cache with per-sequence prompt lengths, the commit step and
the cache append: the HIP path vs the CPU oracle, through the C-ABI, on the
same seeded inputs.  Attention within the bf16 tolerance of the contiguous
path; the commit step bit-exact; appended values bit-exact and appended keys
(rotated at their positions) within one bf16 unit in the last place."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import binding as sv
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Case("paged", 3, 300, 16, 16, 8, 2, 128, 1000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=90,
                  n_copies=5, page_size=64, ragged=True)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_paged(o, case, n_copies=0, lens=None, check_seqs=None):
    if n_copies:
        case = case.with_(n_copies=n_copies)
    print(f"[case] {case.name} batch={case.batch} P={case.prefix_len} B={case.block} ps={case.page_size} "
          f"ragged={case.ragged} copies={n_copies} heads={case.n_qh}/{case.n_kvh} d={case.head_dim} lens={lens}",
          flush=True)
    _cuda()
    from diffusion_speculative_verification_amd.device import StepBuffers
    base = ("copies",) if n_copies else ("attn",)
    inp = synth.make_inputs(case, parts=base + ("paged",))
    if lens is not None:
        inp["prefix_lens"] = np.array(lens, np.int32)
    buf = StepBuffers(case, inp, parts=base + ("paged",))
    buf.attn_paged(n_copies=n_copies)
    torch.cuda.synchronize()
    got = buf.out_paged.float().cpu().numpy()
    idx = list(range(case.batch)) if check_seqs is None else list(check_seqs)
    q, kn, vn = (inp["q_c"], inp["k_new_c"], inp["v_new_c"]) if n_copies else (inp["q"], inp["k_new"], inp["v_new"])
    ref = o.attention_paged(q[idx], kn[idx], vn[idx], inp["k_pages"], inp["v_pages"], inp["block_table"][idx],
                            inp["prefix_lens"][idx], inp["tau"][idx], case.page_size, case.theta, n_copies)
    worst = (0.0, 0.0)
    for i, b in enumerate(idx):
        mx, rel = parity.check_attn(got[b], ref[i], case.dtype, f"{case.name} seq {b} P_b={inp['prefix_lens'][b]}")
        worst = (max(worst[0], mx), max(worst[1], rel))
    print(f"[result] {case.name}: max {worst[0]:.3e} relrms {worst[1]:.3e}", flush=True)
    return buf, inp


@pytest.mark.parametrize("kw,n_copies", [
    (dict(ragged=False), 0),                          # every sequence at P, pages of 64
    (dict(), 0),                                      # ragged lengths
    (dict(page_size=128, prefix_len=700), 0),         # larger pages, lengths in [350, 700]
    (dict(head_dim=64, prefix_len=77), 0),            # head_dim 64, lengths in [38, 77]
    (dict(), 5),                                      # the multi-copy layout over pages
    (dict(batch=2, prefix_len=9000, n_qh=8, n_kvh=1), 0),   # prefix splits: empty splits for the shorter
    (dict(batch=2, prefix_len=9000, n_qh=8, n_kvh=1), 3),
    (dict(head_dim=64, prefix_len=600, page_size=256), 6),   # copies, head_dim 64, pages of 256
    (dict(block=64, gamma=64, n_qh=16, n_kvh=2, prefix_len=1500, page_size=512), 0),   # B = 64, pages of 512
])
def test_paged(o, kw, n_copies):
    run_paged(o, BASE.with_(**kw), n_copies)


@pytest.mark.parametrize("n_copies", [0, 4])
def test_paged_edge_lengths(o, n_copies):
    """Prompt lengths 0, 1, 63, 64, 65 and the maximum in one batch (tile and
    page boundaries, an empty prompt)."""
    case = BASE.with_(batch=6, ragged=False)
    run_paged(o, case, n_copies, lens=[0, 1, 63, 64, 65, case.prefix_len])


def test_paged_headline_sampled(o):
    """The headline shape over pages of 64 with ragged lengths, in the launch
    configuration a benchmark would time; sampled sequences checked."""
    case = synth.config_by_name("headline").with_(page_size=64, ragged=True)
    run_paged(o, case, 0, check_seqs=[0, 17, 31])


def test_paged_equals_contiguous(o):
    """With every sequence at the full length, the paged call reads the same
    rows as the contiguous call and does the same arithmetic: bit-identical."""
    _cuda()
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small").with_(page_size=64, ragged=False)
    inp = synth.make_inputs(case, parts=("attn", "paged"))
    buf = StepBuffers(case, inp, parts=("attn", "paged"))
    buf.attn()
    buf.attn_paged()
    torch.cuda.synchronize()
    assert torch.equal(buf.out, buf.out_paged)


def test_paged_contiguous_stride(o):
    """No page table: a contiguous cache with a row stride above the longest
    prompt and per-sequence lengths."""
    _cuda()
    case = BASE.with_(batch=4, ragged=False)
    inp = synth.make_inputs(case, parts=("attn",))
    lens = np.array([300, 0, 129, 64], np.int32)
    stride = 320
    kc = np.zeros((4, case.n_kvh, stride, case.head_dim), np.float32)
    vc = np.zeros_like(kc)
    kc[:, :, :300], vc[:, :, :300] = inp["k_cache"], inp["v_cache"]
    d = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    q, kn, vn, kcd, vcd = d(inp["q"]), d(inp["k_new"]), d(inp["v_new"]), d(kc), d(vc)
    tau, pl = d(inp["tau"], torch.int32), d(lens, torch.int32)
    out = torch.empty_like(q)
    n = sv.spec_verify_attn_paged_workspace_size(sv.SV_BF16, 4, case.block, 0, 300, case.n_qh, case.n_kvh, 128)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    sv.spec_verify_attn_paged(q, kn, vn, kcd, vcd, None, pl, tau, out, sv.SV_BF16, 4, case.block, 0, 300, stride,
                              0, 0, case.n_qh, case.n_kvh, 128, case.theta, 0.0, ws, n)
    torch.cuda.synchronize()
    ref = o.attention_paged(inp["q"], inp["k_new"], inp["v_new"], kc, vc, None, lens, inp["tau"], stride, case.theta)
    got = out.float().cpu().numpy()
    for b in range(4):
        parity.check_attn(got[b], ref[b], "bf16", f"stride seq {b}")


# ------------------------------------------------------------------ commit
@pytest.mark.parametrize("B,gamma", [(32, 32), (32, 8), (7, 3), (1, 1), (64, 17)])
def test_commit(o, B, gamma):
    print(f"[case] commit B={B} gamma={gamma}", flush=True)
    _cuda()
    r = np.random.default_rng(1000 + B + gamma)
    n = 300
    before = np.where(r.random((n, B)) < 0.6, r.integers(0, 151936, (n, B)), -1).astype(np.int32)
    out = np.where(r.random((n, B)) < 0.3, r.integers(0, 151936, (n, B)), -1).astype(np.int32)
    out[0] = np.where(before[0] < 0, 0, -1)        # token id 0 completes sequence 0
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bt, ot = d(before), d(out)
    rem, st, na = (torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(3))
    sv.spec_verify_commit(ot, bt, n, B, gamma, rem, st, na)
    torch.cuda.synchronize()
    bt_o, rem_o, st_o, na_o = o.commit(out, before, gamma)
    assert np.array_equal(bt.cpu().numpy(), bt_o)
    assert np.array_equal(rem.cpu().numpy(), rem_o)
    assert np.array_equal(st.cpu().numpy(), st_o)
    assert np.array_equal(na.cpu().numpy(), na_o)
    assert st_o[0] == 2
    print(f"[result] commit B={B}: states {np.bincount(st_o, minlength=3).tolist()}", flush=True)


# ------------------------------------------------------------------ append
def _bf16_close(got, want):
    """Within one bfloat16 unit in the last place of the larger magnitude."""
    m = np.maximum(np.abs(got), np.abs(want))
    ulp = np.where(m > 0, 2.0 ** (np.floor(np.log2(np.maximum(m, 1e-38))) - 7), 0.0)
    return bool((np.abs(got - want) <= ulp).all())


@pytest.mark.parametrize("paged,theta,head_dim,ps", [(True, 1e6, 128, 64), (True, 0.0, 128, 64), (False, 1e4, 64, 64),
                                                     (True, 1e4, 64, 64), (True, 1e6, 128, 128)])
def test_kv_append(o, paged, theta, head_dim, ps):
    print(f"[case] append paged={paged} theta={theta} d={head_dim} page_size={ps}", flush=True)
    _cuda()
    case = BASE.with_(batch=6, head_dim=head_dim, ragged=True, prefix_len=200, page_size=ps)
    inp = synth.make_inputs(case, parts=("attn", "paged"))
    B, S = case.block, 2 * case.block
    n_app = np.array([B, 0, 5, B, B, S + 1], np.int32)   # seq 5: more rows than the source holds
    if paged:
        kp, vp, table = inp["k_pages"], inp["v_pages"], inp["block_table"]
        ps, cap = case.page_size, case.page_size * table.shape[1]
        lens = inp["prefix_lens"].copy()
    else:   # contiguous, row stride 240
        ps = cap = 240
        kp = np.zeros((6, case.n_kvh, ps, head_dim), np.float32)
        vp = np.zeros_like(kp)
        kp[:, :, :200], vp[:, :, :200] = inp["k_cache"], inp["v_cache"]
        table, lens = None, inp["prefix_lens"].copy()
    lens[3] = cap - B          # exact fit
    lens[4] = cap - B + 1      # one row too many: nothing appended
    d = lambda a, dt=None: (lambda t: t.to(dt) if dt is not None else t)(torch.from_numpy(np.ascontiguousarray(a)).cuda())
    kr, vr = d(inp["k_new"], torch.bfloat16), d(inp["v_new"], torch.bfloat16)   # the D rows come first
    kpd, vpd = d(kp, torch.bfloat16), d(vp, torch.bfloat16)
    tb = d(table) if paged else None
    pl, na = d(lens), d(n_app)
    status = torch.empty(6, dtype=torch.int32, device="cuda")
    sv.spec_verify_kv_append(kr, vr, S, na, kpd, vpd, tb, pl, status, sv.SV_BF16, 6, ps,
                             table.shape[1] if paged else 0, kp.shape[0] if paged else 0, case.n_kvh, head_dim, theta)
    torch.cuda.synchronize()
    n_ok = n_app.copy()
    n_ok[5] = 0                # the oracle rejects n > stride outright; the kernel reports status 2
    kp_o, vp_o, lens_o, st_o = o.kv_append(inp["k_new"], inp["v_new"], n_ok, kp, vp, table, lens, ps, theta)
    st = status.cpu().numpy()
    assert st.tolist()[:5] == st_o.tolist()[:5] and st[5] == 2, (st, st_o)
    assert st[4] == 1 and st[3] == 0
    assert np.array_equal(pl.cpu().numpy(), lens_o)
    kg, vg = kpd.float().cpu().numpy(), vpd.float().cpu().numpy()
    assert np.array_equal(vg, vp_o)
    if theta > 0:
        assert _bf16_close(kg, kp_o)
    else:
        assert np.array_equal(kg, kp_o)
    assert np.array_equal(kg[kp_o == kp], kp[kp_o == kp])   # rows not appended are untouched
    print(f"[result] append: lengths {lens.tolist()} -> {lens_o.tolist()}", flush=True)


def test_kv_append_bad_page(o):
    """A block-table entry outside [0, n_pages) where an append would land:
    status 3, nothing written for that sequence and its length unchanged;
    the other sequences append as usual."""
    print("[case] append with planted bad page ids", flush=True)
    _cuda()
    case = BASE.with_(batch=6, ragged=True, prefix_len=200, page_size=64)
    inp = synth.make_inputs(case, parts=("attn", "paged"))
    B, S = case.block, 2 * case.block
    kp, vp, table = inp["k_pages"], inp["v_pages"], inp["block_table"].copy()
    ps, n_pages = case.page_size, kp.shape[0]
    lens = inp["prefix_lens"].copy()
    n_app = np.array([B, B, 5, 0, B, B], np.int32)
    table[0, (lens[0] + B - 1) // ps] = n_pages      # last page of the rows: one past the end
    table[2, lens[2] // ps] = -1                      # first page of the rows: negative
    table[3, lens[3] // ps] = n_pages + 7             # nothing to append: not looked at
    d = lambda a, dt=None: (lambda t: t.to(dt) if dt is not None else t)(torch.from_numpy(np.ascontiguousarray(a)).cuda())
    kr, vr = d(inp["k_new"], torch.bfloat16), d(inp["v_new"], torch.bfloat16)
    kpd, vpd = d(kp, torch.bfloat16), d(vp, torch.bfloat16)
    pl, na, tb = d(lens), d(n_app), d(table)
    status = torch.full((6,), -9, dtype=torch.int32, device="cuda")
    sv.spec_verify_kv_append(kr, vr, S, na, kpd, vpd, tb, pl, status, sv.SV_BF16, 6, ps, table.shape[1], n_pages,
                             case.n_kvh, case.head_dim, case.theta)
    torch.cuda.synchronize()
    st = status.cpu().numpy()
    assert st.tolist() == [3, 0, 3, 0, 0, 0], st
    n_ok = n_app.copy()
    n_ok[[0, 2]] = 0
    kp_o, vp_o, lens_o, _ = o.kv_append(inp["k_new"], inp["v_new"], n_ok, kp, vp, table, lens, ps, case.theta)
    assert np.array_equal(pl.cpu().numpy(), lens_o)
    assert lens_o[0] == lens[0] and lens_o[2] == lens[2]
    kg, vg = kpd.float().cpu().numpy(), vpd.float().cpu().numpy()
    assert np.array_equal(vg, vp_o)
    assert _bf16_close(kg, kp_o)
    assert np.array_equal(kg[kp_o == kp], kp[kp_o == kp])   # nothing else written
    print(f"[result] append bad pages: status {st.tolist()}", flush=True)


def test_step_chain(o):
    """Verification, commit and append in a row on the GPU, then the next
    verification attention over the grown cache: each stage vs the oracle."""
    _cuda()
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = BASE.with_(batch=4, block=8, gamma=8, prefix_len=130, vocab=64, ragged=True)
    inp = synth.make_inputs(case, parts=("attn", "accept", "paged"))
    # sequences 0 and 2 draft from the target's own distribution, so every
    # step is accepted (alpha = 1 up to float32 rounding) and their blocks
    # finish and are appended; the others keep their independent drafts
    for b in (0, 2):
        lt = inp["target_logits"][b].astype(np.float64)
        p = np.exp(lt - lt.max(axis=1, keepdims=True))
        inp["draft_probs"][b] = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    buf = StepBuffers(case, inp, parts=("attn", "accept", "paged"))
    buf.attn_paged()
    buf.accept()
    buf.commit(buf.out_tokens)
    # a finished block appends the D rows of this forward (positions P_b .. P_b + B - 1)
    buf.kv_append(buf.k_new, buf.v_new, 2 * case.block)
    torch.cuda.synchronize()
    L, ot = buf.accept_len.cpu().numpy(), buf.out_tokens.cpu().numpy()
    L_o, ot_o, _, _ = o.accept(inp["target_logits"], inp["draft_probs"], inp["draft_tokens"], inp["tau"],
                               inp["uniforms"], case.gamma)
    assert np.array_equal(L, L_o) and np.array_equal(ot, ot_o)
    bt_o, rem_o, st_o, na_o = o.commit(ot_o, inp["block_tokens"], case.gamma)
    assert np.array_equal(buf.block_tokens.cpu().numpy(), bt_o)
    assert np.array_equal(buf.n_append.cpu().numpy(), na_o)
    assert na_o[0] == case.block and na_o[2] == case.block, na_o
    kp_o, vp_o, lens_o, _ = o.kv_append(inp["k_new"], inp["v_new"], na_o, inp["k_pages"], inp["v_pages"],
                                        inp["block_table"], inp["prefix_lens"], case.page_size, case.theta)
    assert np.array_equal(buf.prefix_lens.cpu().numpy(), lens_o)
    # the next round's attention over the grown prompts (oracle on its own
    # cache); the longest prompt may now pass the case's prompt length
    buf.attn_paged(max_prefix=case.prefix_len + case.block)
    torch.cuda.synchronize()
    got = buf.out_paged.float().cpu().numpy()
    kp_g = buf.k_pages.float().cpu().numpy()
    assert _bf16_close(kp_g, kp_o)
    ref = o.attention_paged(inp["q"], inp["k_new"], inp["v_new"], kp_g, vp_o, inp["block_table"], lens_o,
                            inp["tau"], case.page_size, case.theta)
    for b in range(case.batch):
        parity.check_attn(got[b], ref[b], "bf16", f"chain seq {b}")
    print(f"[result] chain: accept_len {L.tolist()} n_append {na_o.tolist()} lengths {lens_o.tolist()}", flush=True)


# ------------------------------------------------------------------ tau validation
@pytest.mark.parametrize("B", [1, 7, 32, 64])
def test_check_tau(B):
    """Rows that are permutations of 1..B pass; rows with a label out of
    range (0, B + 1, negative) or a repeated label are flagged."""
    print(f"[case] check_tau B={B}", flush=True)
    _cuda()
    r = np.random.default_rng(2000 + B)
    n = 200
    tau = np.stack([r.permutation(B) + 1 for _ in range(n)]).astype(np.int32)
    for i in range(0, n, 2):
        k = int(r.integers(0, B))
        kind = (i // 2) % 4
        if kind == 0:
            tau[i, k] = 0
        elif kind == 1:
            tau[i, k] = B + 1
        elif kind == 2:
            tau[i, k] = -5
        elif B > 1:
            tau[i, k] = tau[i, (k + 1) % B]          # a repeated label
    want = np.array([0 if sorted(row.tolist()) == list(range(1, B + 1)) else 1 for row in tau], np.int32)
    t = torch.from_numpy(tau).cuda()
    bad = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    sv.spec_verify_check_tau(t, n, B, bad)
    torch.cuda.synchronize()
    assert np.array_equal(bad.cpu().numpy(), want)
    print(f"[result] check_tau B={B}: {int(want.sum())} bad rows found", flush=True)
