"""The C ABI from a plain host program: tests/c/abi_step (built by
__graft_entry__.build()) allocates device memory with the HIP runtime, creates
its own stream and runs spec_verify_attn (RoPE fused) and spec_verify_accept
through include/spec_verify.h alone -- no Python, no torch.  Its outputs are
checked against the CPU oracle on the same seeded inputs."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c", "abi_step")


def _bf16_bits(a):
    """float32 values that are bfloat16 numbers -> their 16-bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert (u & 0xFFFF).max(initial=0) == 0, "inputs must be bfloat16 values"
    return (u >> 16).astype(np.uint16)


def _from_bf16_bits(u16, shape):
    return (u16.astype(np.uint32) << 16).view(np.float32).reshape(shape)


@pytest.mark.parametrize("kw", [dict(), dict(prefix_len=0), dict(batch=3, block=8, gamma=5, vocab=1001)])
def test_c_client_step(tmp_path, kw):
    case = synth.config_by_name("small").with_(**kw)
    print(f"[case] C client: {case}", flush=True)
    try:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("no GPU")
    except ImportError:
        pytest.skip("no torch")
    assert os.path.exists(CLIENT), "tests/c/abi_step is not built: run __graft_entry__.build()"
    inp = synth.make_inputs(case)
    d = str(tmp_path)
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(f"{case.batch} {case.block} {case.gamma} {case.prefix_len} {case.n_qh} {case.n_kvh} "
                f"{case.head_dim} {case.vocab} {case.theta!r}\n")
    for name in ("q", "k_new", "v_new", "k_cache", "v_cache"):
        _bf16_bits(inp[name]).tofile(os.path.join(d, name + ".bin"))
    for name, dt in (("tau", np.int32), ("draft_tokens", np.int32), ("target_logits", np.float32),
                     ("draft_probs", np.float32), ("uniforms", np.float32)):
        np.ascontiguousarray(inp[name], dt).tofile(os.path.join(d, name + ".bin"))
    r = subprocess.run([CLIENT, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "abi_step: ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
    out = _from_bf16_bits(np.fromfile(os.path.join(d, "out.bin"), np.uint16), inp["q"].shape)
    L = np.fromfile(os.path.join(d, "accept_len.bin"), np.int32)
    tok = np.fromfile(os.path.join(d, "out_tokens.bin"), np.int32).reshape(case.batch, case.block)
    al = np.fromfile(os.path.join(d, "alpha.bin"), np.float32).reshape(case.batch, case.gamma)
    o = oracle.Oracle()
    for b in range(case.batch):
        ref = o.attention(inp["q"][b], inp["k_new"][b], inp["v_new"][b], inp["k_cache"][b], inp["v_cache"][b],
                          inp["tau"][b], case.theta)
        parity.check_attn(out[b], ref, "bf16", f"C client seq {b}")
    ties = parity.check_accept(o, inp, case.gamma, L, tok, al)
    print(f"[result] C client ok: accept_len {L.tolist()}, ties {ties}", flush=True)
