"""float16 outputs (GDN_OUT_F16). The recurrence is unchanged and only the stored o is
rounded, so the float16 o of every call equals the float32 o of the same call rounded to
nearest even, bit for bit; against the float64 oracle the bfloat16 bar (2e-3 of max|o|)
still holds, since the rounding adds at most 2^-11 of a value. The gated RMSNorm on float16
rows is checked against the oracle's norm of the same float16 values, to one float16
rounding per element (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


@pytest.mark.parametrize("chunk", [64, 32])
def test_prefill_f16_o(gdn, oracle_lib, chunk):
    import torch
    x = inputs.generate(2, 300, 2, 4, 128, "bf16", seed=110 + chunk, init_state="normal")
    q, k, v = qkv_dev(x)
    args = (q, k, v, dev(x.g), dev(x.beta), dev(x.s0))
    o32, s32 = gdn.prefill(*args, chunk=chunk, scale=x.scale)
    o16, s16 = gdn.prefill(*args, chunk=chunk, scale=x.scale, o_dtype=torch.float16)
    assert o16.dtype == torch.float16
    assert torch.equal(o16, o32.half()) and torch.equal(s16, s32)
    o_ref, _ = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    err = rel_err(o16.float().cpu().numpy(), o_ref)
    print(f"prefill C{chunk}, float16 o: rel err {err:.3e}")
    assert err <= TOL_BF16


def test_long_prefill_f16_o_sampled(gdn, oracle_lib):
    """T = 32768 at the benchmarked shape with float16 o; 2 value heads against the oracle."""
    import torch
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    q, k, v = qkv_dev(x)
    o16, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), None, chunk=wl.chunk, scale=x.scale,
                         o_dtype=torch.float16, write_final_state=False)
    pairs = np.array([3, 28])
    o_ref, _ = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, pairs=pairs)
    got = o16.reshape(-1, *o16.shape[2:])[torch.from_numpy(pairs).cuda()].float().cpu().numpy()
    err = rel_err(got, o_ref)
    print(f"long_32k float16 o (2 heads): rel err {err:.3e}")
    assert err <= TOL_BF16


def test_segmented_and_packed_f16_o(gdn):
    """Four segments (the preferred workspace at B=2, Hv=32, T=2000) and packed sequences write
    the float32 run's o rounded to float16."""
    import torch
    x = inputs.generate(2, 2000, 16, 32, 128, "bf16", seed=113, init_state="normal")
    q, k, v = qkv_dev(x)
    args = (q, k, v, dev(x.g), dev(x.beta), dev(x.s0))
    o32, _ = gdn.prefill(*args, chunk=64, scale=x.scale)
    o16, _ = gdn.prefill(*args, chunk=64, scale=x.scale, o_dtype=torch.float16)
    assert torch.equal(o16, o32.half())
    cu = torch.tensor([0, 700, 700, 2000], dtype=torch.int32, device="cuda")
    vargs = (q[0], k[0], v[0], dev(x.g[0]), dev(x.beta[0]), cu)
    p32, _ = gdn.prefill_varlen(*vargs, chunk=64, scale=x.scale)
    p16, _ = gdn.prefill_varlen(*vargs, chunk=64, scale=x.scale, o_dtype=torch.float16)
    assert torch.equal(p16, p32.half())


def test_decode_f16_o(gdn):
    import torch
    x = inputs.generate(8, 1, 2, 4, 128, "bf16", seed=114, init_state="normal", decode_steps=1)
    q, k, v = (t[0] for t in qkv_dev(x))
    s_a, s_b = dev(x.s0), dev(x.s0)
    o32 = gdn.decode(q, k, v, dev(x.g[0]), dev(x.beta[0]), s_a, scale=x.scale)
    o16 = gdn.decode(q, k, v, dev(x.g[0]), dev(x.beta[0]), s_b, scale=x.scale, o_dtype=torch.float16)
    assert torch.equal(o16, o32.half()) and torch.equal(s_a, s_b)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("gate_dtype", ["bf16", "f32", None])
def test_gated_rmsnorm_f16_rows(gdn, oracle_lib, d, gate_dtype):
    """float16 rows (8 values per lane: rows of 2, 4, 8 or 16 lanes), bfloat16, float32 or no gate."""
    import torch
    rng = np.random.default_rng(115 + d)
    o = (rng.standard_normal((2, 4, 300, d)) * 0.05).astype(np.float16)
    nrm = inputs.generate_norm(o.shape, gate_dtype or "bf16", seed=116 + d)
    t = torch.from_numpy(o).cuda()
    if gate_dtype == "bf16":
        gate = torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    elif gate_dtype == "f32":
        gate = dev(nrm.gate)
    else:
        gate = None
    gdn.gated_rmsnorm(t, dev(nrm.weight), gate, eps=1e-6)
    want = oracle_lib.gated_rmsnorm(o.astype(np.float64), nrm.weight, gate=nrm.gate if gate_dtype else None,
                                    eps=1e-6)
    got = t.float().cpu().numpy()
    bound = 2.0 ** -11 * np.abs(want) + 1e-5 * np.max(np.abs(want))
    assert np.max(np.abs(got - want) - bound) <= 0.0


def test_chain_f16_o(gdn, oracle_lib):
    """prefill with float16 o, then the gated RMSNorm on those rows, against the oracle's chain."""
    import torch
    x = inputs.generate(1, 500, 16, 32, 128, "bf16", seed=117, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=118)
    q, k, v = qkv_dev(x)
    o16, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale,
                         o_dtype=torch.float16, write_final_state=False)
    gate = torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    gdn.gated_rmsnorm(o16, dev(nrm.weight), gate, eps=1e-6)
    o_ref, _ = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    y_ref = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=nrm.gate, eps=1e-6)
    err = rel_err(o16.float().cpu().numpy(), y_ref)
    print(f"chain with float16 o: rel err {err:.3e}")
    assert err <= TOL_BF16
