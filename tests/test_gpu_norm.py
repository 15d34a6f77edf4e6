"""GPU parity of gdn_gated_rmsnorm (applied to gdn_prefill / gdn_decode outputs) against the
float64 oracle's scan followed by its gated RMSNorm (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def gate_dev(nrm):
    import torch
    if nrm.gate_bits is not None:
        return torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    return dev(nrm.gate)


def prefill_then_norm(gdn, oracle_lib, x, chunk, nrm, gated=True, pairs=None, label=""):
    q, k, v = qkv_dev(x)
    init = dev(x.s0) if x.s0 is not None else None
    o, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=chunk, scale=x.scale, write_final_state=False)
    gdn.gated_rmsnorm(o, dev(nrm.weight), gate_dev(nrm) if gated else None, eps=EPS)
    got = o.cpu().numpy()
    o_ref, _ = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, pairs=pairs)
    if pairs is not None:
        B, Hv = x.v.shape[:2]
        got = got.reshape(B * Hv, *got.shape[2:])[pairs]
        gate = nrm.gate.reshape(B * Hv, *nrm.gate.shape[2:])[pairs]
    else:
        gate = nrm.gate
    want = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=gate if gated else None, eps=EPS)
    err = rel_err(got, want)
    print(f"{label}: rel err {err:.3e}")
    return err


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_bf16_gated(gdn, oracle_lib, chunk):
    x = inputs.generate(2, 100, 2, 4, 128, "bf16", seed=41 + chunk, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=42)
    assert prefill_then_norm(gdn, oracle_lib, x, chunk, nrm, label=f"bf16 C{chunk}") <= TOL_BF16


def test_prefill_bf16_ungated(gdn, oracle_lib):
    x = inputs.generate(1, 200, 2, 4, 128, "bf16", seed=43, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=44)
    assert prefill_then_norm(gdn, oracle_lib, x, 64, nrm, gated=False, label="bf16 ungated") <= TOL_BF16


def test_prefill_4k_gated(gdn, oracle_lib):
    wl = inputs.WORKLOADS["prefill_4k"]
    x = inputs.generate_workload(wl)
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=45)
    assert prefill_then_norm(gdn, oracle_lib, x, wl.chunk, nrm, label="prefill_4k gated") <= TOL_BF16


def test_long_prefill_gated_sampled(gdn, oracle_lib):
    """T = 32768: a million output rows through the epilogue; 4 value heads checked in full."""
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=46)
    err = prefill_then_norm(gdn, oracle_lib, x, wl.chunk, nrm, pairs=np.array([0, 9, 22, 31]),
                            label="long_32k gated (4 heads)")
    assert err <= TOL_BF16


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_prefill_f32_gated(gdn, oracle_lib, d):
    x = inputs.generate(2, 70, 2, 4, d, "f32", seed=47 + d, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "f32", seed=48)
    assert prefill_then_norm(gdn, oracle_lib, x, 32, nrm, label=f"f32 d{d}") <= TOL_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_gated(gdn, oracle_lib, dtype):
    x = inputs.generate(8, 0, 2, 4, 128, dtype, seed=49, init_state="normal", decode_steps=3)
    nrm = inputs.generate_norm((3, 8, 4, 128), dtype, seed=50)
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    state = dev(x.s0)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    for step in range(3):
        o = gdn.decode(q[step], k[step], v[step], g[step], beta[step], state, scale=x.scale)
        sub = inputs.NormInputs(gate=nrm.gate[step], weight=nrm.weight,
                                gate_bits=None if nrm.gate_bits is None else nrm.gate_bits[step])
        gdn.gated_rmsnorm(o, dev(nrm.weight), gate_dev(sub), eps=EPS)
        o_ref = oracle_lib.decode_step(x.q[step], x.k[step], x.v[step], x.g[step], x.beta[step], ref_state,
                                       scale=x.scale)
        want = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=nrm.gate[step], eps=EPS)
        err = rel_err(o.cpu().numpy(), want)
        print(f"decode {dtype} step {step}: rel err {err:.3e}")
        assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32)
