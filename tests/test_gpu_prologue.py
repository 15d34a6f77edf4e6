"""GPU parity of gdn_qkv_prologue against the float64 oracle, and of the whole chain
prologue -> prefill -> gated RMSNorm against the oracle's chain (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, rel_err  # noqa: F401

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def make_inputs(B, T, Hk, Hv, d, dtype, seed, state=True):
    """Raw projections x ~ N(0, 1) (bf16-rounded for bf16), conv weights ~ N(0, 0.5) and a
    conv state ~ N(0, 1) (or none)."""
    rng = np.random.default_rng(seed)
    C = (2 * Hk + Hv) * d
    x = rng.standard_normal((B, T, C))
    xf, xb = inputs._store(x, dtype)
    w = (rng.standard_normal((C, 4)) * 0.5).astype(np.float32)
    st = rng.standard_normal((B, 3, C)).astype(np.float32) if state else None
    return xf, xb, w, st


def x_dev(xf, xb):
    import torch
    if xb is not None:
        return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()
    return dev(xf)


def to_np(t):
    import torch
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [1, 3, 50, 200])
def test_prologue_parity(gdn, oracle_lib, dtype, d, T):
    Hk, Hv = 2, 4
    for state in (True, False):
        xf, xb, w, st = make_inputs(2, T, Hk, Hv, d, dtype, seed=60 + T + d, state=state)
        st_dev = dev(st) if st is not None else None
        q, k, v = gdn.qkv_prologue(x_dev(xf, xb), dev(w), st_dev, num_k_heads=Hk, num_v_heads=Hv, head_dim=d,
                                   eps=EPS)
        rq, rk, rv, rst = oracle_lib.qkv_prologue(xf, w, Hk, Hv, d, state=st, eps=EPS)
        for name, got, want in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
            g_ = to_np(got)
            if dtype == "bf16":
                # bf16 outputs: the stored value is a rounding of the fp32 result, so the bar is one
                # bf16 step (2^-8 of the value) per element, plus fp32 arithmetic noise
                bound = 2.0 ** -8 * np.abs(want) + 1e-5 * np.max(np.abs(want))
                worst = float(np.max(np.abs(g_ - want) - bound))
                assert worst <= 0.0, (name, dtype, d, T, state, worst)
            else:
                err = rel_err(g_, want)
                assert err <= TOL_F32, (name, dtype, d, T, state, err)
        if st is not None:  # the new state is input rows, copied exactly
            assert np.array_equal(st_dev.cpu().numpy(), rst.astype(np.float32)), (dtype, d, T)


def test_prologue_continuation(gdn):
    """One call over 300 tokens equals calls over 130 then 170 tokens with the state carried."""
    Hk, Hv, d = 2, 4, 128
    xf, xb, w, st = make_inputs(2, 300, Hk, Hv, d, "bf16", seed=70)
    x = x_dev(xf, xb)
    s_full = dev(st)
    full = gdn.qkv_prologue(x, dev(w), s_full, num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    s_part = dev(st)
    a = gdn.qkv_prologue(x[:, :130].contiguous(), dev(w), s_part, num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    b = gdn.qkv_prologue(x[:, 130:].contiguous(), dev(w), s_part, num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    import torch
    for f, p1, p2 in zip(full, a, b):
        assert torch.equal(f, torch.cat([p1, p2], dim=2))
    assert torch.equal(s_full, s_part)


def test_chain_prologue_prefill_norm(gdn, oracle_lib):
    """Raw projections -> prologue -> chunked prefill -> gated RMSNorm, against the same chain in
    the oracle (B=1, Hk=16, Hv=32, T=1000, d=128, bf16)."""
    Hk, Hv, d, T = 16, 32, 128, 1000
    xf, xb, w, st = make_inputs(1, T, Hk, Hv, d, "bf16", seed=71)
    rng = np.random.default_rng(72)
    g = (-np.log1p(np.exp(rng.standard_normal((1, Hv, T))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((1, Hv, T))))).astype(np.float32)
    nrm = inputs.generate_norm((1, Hv, T, d), "bf16", seed=73)
    scale = d ** -0.5
    q, k, v = gdn.qkv_prologue(x_dev(xf, xb), dev(w), dev(st), num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    o, _ = gdn.prefill(q, k, v, dev(g), dev(beta), None, chunk=64, scale=scale, write_final_state=False)
    import torch
    gate = torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    gdn.gated_rmsnorm(o, dev(nrm.weight), gate, eps=EPS)
    rq, rk, rv, _ = oracle_lib.qkv_prologue(xf, w, Hk, Hv, d, state=st, eps=EPS)
    # the oracle's scan reads the GPU path's input precision: q, k, v rounded to bfloat16
    rb = [inputs.bf16_to_f32(inputs.bf16_round(a.astype(np.float32))) for a in (rq, rk, rv)]
    o_ref, _ = oracle_lib.prefill(rb[0], rb[1], rb[2], g, beta, None, scale=scale)
    y_ref = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=nrm.gate, eps=EPS)
    err = rel_err(o.cpu().numpy(), y_ref)
    print(f"chain: rel err {err:.3e}")
    assert err <= TOL_BF16
