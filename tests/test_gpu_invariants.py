"""Invariants of the GPU attention that follow from the pages' definitions,
checked on the HIP path's own outputs without the oracle's attention.

- Rebuilt context ("SimSD: Simple Speculative Decoding in Diffusion Language
  Models", 关键设计 2: the masked single forward equals the autoregressive
  verification context): each D~_i row equals plain unmasked attention over
  [prompt; for every slot k, D_k if tau(k) < tau(i) else D~_k], each key at its
  true position; each D_i row likewise with <=.  The reference here is numpy
  float64 softmax attention over that explicit context; the keys are rotated
  with the (pinned) oracle's RoPE.
- Step-label equivariance: permuting the slots of pre-rotated inputs by sigma,
  with the labels permuted alike, permutes the output rows by sigma (the mask
  depends on the labels only, not on the slot order).
"""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _gpu_attn(case, inp, rope_theta=None):
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("attn",))
    buf.attn(rope_theta=rope_theta)
    torch.cuda.synchronize()
    return buf.out.float().cpu().numpy()


def _rebuilt_reference(o, case, inp, b):
    """Unmasked float64 attention of every response row over its explicit
    autoregressive context."""
    B, P, d, g = case.block, case.prefix_len, case.head_dim, case.n_qh // case.n_kvh
    pos = P + (np.arange(2 * B) % B).astype(np.float64)
    q = o.rope(inp["q"][b], pos, case.theta)            # [2B][Hq][d]
    k = o.rope(inp["k_new"][b], pos, case.theta)        # [2B][Hkv][d]
    v = inp["v_new"][b].astype(np.float64)
    kc, vc = inp["k_cache"][b].astype(np.float64), inp["v_cache"][b].astype(np.float64)  # [Hkv][P][d]
    tau = inp["tau"][b]
    out = np.empty((2 * B, case.n_qh, d))
    for r in range(2 * B):
        i, is_data = r % B, r < B
        ctx = [k2 if (tau[k2] <= tau[i] if is_data else tau[k2] < tau[i]) else B + k2 for k2 in range(B)]
        for h in range(case.n_qh):
            kv = h // g
            keys = np.concatenate([kc[kv], k[ctx, kv]])
            vals = np.concatenate([vc[kv], v[ctx, kv]])
            s = keys @ q[r, h] / np.sqrt(d)
            w = np.exp(s - s.max())
            out[r, h] = (w / w.sum()) @ vals
    return out


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict()),
    ("bf16", dict(batch=2, prefix_len=130, block=8, gamma=8, n_qh=8, n_kvh=2, head_dim=128, vocab=512,
                  dtype="bf16", theta=1e6)),
    ("bf16-B32", dict(batch=1, prefix_len=300, block=32, gamma=32, n_qh=4, n_kvh=1, head_dim=64, vocab=512,
                      dtype="bf16", theta=1e6)),
])
def test_rebuilt_context(o, name, kw):
    print(f"[case] rebuilt context {name}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = synth.config_by_name("tiny").with_(**kw)
    inp = synth.make_inputs(case, parts=("attn",))
    out = _gpu_attn(case, inp)
    for b in range(case.batch):
        parity.check_attn(out[b], _rebuilt_reference(o, case, inp, b), case.dtype, f"rebuilt context {name} seq {b}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_label_permutation_equivariance(o, dtype):
    print(f"[case] label permutation equivariance {dtype}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = synth.Case("equiv", 3, 70, 16, 16, 8, 2, 64, 64, dtype, 1e6, "iid", 2.0, 2.0, 0, seed=88)
    inp = synth.make_inputs(case, parts=("attn",))
    B = case.block
    pos = case.prefix_len + (np.arange(2 * B) % B).astype(np.float64)
    for key in ("q", "k_new"):   # pre-rotated at the slots' positions; the kernel then rotates nothing
        rot = np.stack([o.rope(inp[key][b], pos, case.theta) for b in range(case.batch)]).astype(np.float32)
        inp[key] = synth.round_bf16(rot) if dtype == "bf16" else rot
    out = _gpu_attn(case, inp, rope_theta=0.0)
    r = np.random.default_rng(5)
    sigma = np.stack([r.permutation(B) for _ in range(case.batch)])   # new slot j holds old slot sigma[j]
    perm = dict(inp)
    rows = np.stack([np.concatenate([s, B + s]) for s in sigma])      # D and D~ rows move together
    for key in ("q", "k_new", "v_new"):
        perm[key] = np.stack([inp[key][b][rows[b]] for b in range(case.batch)])
    perm["tau"] = np.stack([inp["tau"][b][sigma[b]] for b in range(case.batch)])
    out_p = _gpu_attn(case, perm, rope_theta=0.0)
    tol = 1e-5 if dtype == "f32" else 4e-3   # a few bf16 ulps of |o| < 1: only the summation order differs
    for b in range(case.batch):
        err = float(np.abs(out_p[b] - out[b][rows[b]]).max())
        assert err <= tol, (dtype, b, err)
    print(f"[result] permuted outputs equal the permuted rows", flush=True)
