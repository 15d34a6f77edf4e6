"""GPU parity of gdn_prefill against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def run_prefill(gdn, x, chunk, head_map=0, s0=True, **kw):
    q, k, v = qkv_dev(x)
    init = dev(x.s0) if (s0 and x.s0 is not None) else None
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=chunk, head_map=head_map,
                        scale=x.scale, **kw)
    return o.cpu().numpy(), sf.cpu().numpy()


def check(oracle_lib, x, o, sf, head_map=0, tol=None, pairs=None, label=""):
    tol = tol or tol_for(x)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, head_map=head_map,
                                      pairs=pairs)
    if pairs is not None:
        B, Hv = x.v.shape[:2]
        o = o.reshape(B * Hv, *o.shape[2:])[pairs]
        sf = sf.reshape(B * Hv, *sf.shape[2:])[pairs]
    eo, es = rel_err(o, o_ref), rel_err(sf, s_ref)
    print(f"{label}: rel err o {eo:.3e} state {es:.3e} (bar {tol:g})")
    assert eo <= tol, (label, eo)
    assert es <= tol, (label, es)
    return o_ref, s_ref


# ---------------------------------------------------------------- float32 path
def test_tiny_fp32_workload(gdn, oracle_lib):
    wl = inputs.WORKLOADS["tiny_fp32"]
    x = inputs.generate_workload(wl)
    o, sf = run_prefill(gdn, x, wl.chunk)
    check(oracle_lib, x, o, sf, tol=TOL_F32, label="tiny_fp32")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_shapes(gdn, oracle_lib, d, chunk):
    x = inputs.generate(2, 100, 2, 4, d, "f32", seed=d + chunk, init_state="normal")
    for head_map in (0, 1):
        o, sf = run_prefill(gdn, x, chunk, head_map=head_map)
        check(oracle_lib, x, o, sf, head_map=head_map, tol=TOL_F32, label=f"f32 d{d} C{chunk} map{head_map}")


# ---------------------------------------------------------------- bfloat16 MFMA path
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 64, 100, 200])
def test_bf16_small(gdn, oracle_lib, chunk, T):
    for head_map, s0 in ((0, "normal"), (1, "zero")):
        x = inputs.generate(2, T, 2, 4, 128, "bf16", seed=1000 + T + chunk, init_state=s0)
        o, sf = run_prefill(gdn, x, chunk, head_map=head_map)
        check(oracle_lib, x, o, sf, head_map=head_map, label=f"bf16 T{T} C{chunk} map{head_map} s0={s0}")


def test_prefill_4k_workload(gdn, oracle_lib):
    wl = inputs.WORKLOADS["prefill_4k"]
    x = inputs.generate_workload(wl)
    o, sf = run_prefill(gdn, x, wl.chunk)
    check(oracle_lib, x, o, sf, label="prefill_4k")


@pytest.mark.parametrize("chunk", [64, 32])
@pytest.mark.parametrize("head_map", [0, 1])
def test_ragged_continuation_workload(gdn, oracle_lib, chunk, head_map):
    wl = inputs.WORKLOADS["ragged_continuation"]
    x = inputs.generate_workload(wl)
    o, sf = run_prefill(gdn, x, chunk, head_map=head_map)
    check(oracle_lib, x, o, sf, head_map=head_map, label=f"ragged C{chunk} map{head_map}")
    # padded steps produce exactly zero output (q = 0 there)
    for b, length in enumerate(x.lengths):
        assert np.all(o[b, :, length:] == 0.0)


def test_long_prefill_32k_full(gdn, oracle_lib):
    """T = 32768 at the benchmarked launch shape (chunk 64, fp32 o): every output and the final
    state of all 32 value heads against the oracle (about a second of oracle time on 16 cores)."""
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    o, sf = run_prefill(gdn, x, wl.chunk)
    assert np.isfinite(o).all() and np.isfinite(sf).all()
    check(oracle_lib, x, o, sf, label="long_32k (all heads)")


# ---------------------------------------------------------------- semantics
def test_zero_length_copies_state(gdn):
    import torch
    x = inputs.generate(2, 0, 2, 4, 128, "bf16", seed=5, init_state="normal")
    q, k, v = qkv_dev(x)
    init = dev(x.s0)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=64, scale=x.scale)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(sf.cpu().numpy(), x.s0)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), None, chunk=64, scale=x.scale)
    assert np.all(sf.cpu().numpy() == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place_state_and_poisoned_output(gdn, oracle_lib, dtype):
    import torch
    x = inputs.generate(2, 77, 2, 4, 128, dtype, seed=6, init_state="normal")
    q, k, v = qkv_dev(x)
    state = dev(x.s0)
    o = torch.full((2, 4, 77, 128), float("nan"), dtype=torch.float32, device="cuda")
    gdn.prefill(q, k, v, dev(x.g), dev(x.beta), state, chunk=32, scale=x.scale, o=o, final_state=state)
    o_np, s_np = o.cpu().numpy(), state.cpu().numpy()
    assert np.isfinite(o_np).all()
    check(oracle_lib, x, o_np, s_np, label=f"in place {dtype}")


def test_continuation_split(gdn, oracle_lib):
    """prefill(T) vs prefill(m) then prefill(T - m) from the GPU state, at aligned and unaligned m."""
    x = inputs.generate(1, 300, 2, 4, 128, "bf16", seed=8, init_state="normal")
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    o_full, s_full = gdn.prefill(q, k, v, g, beta, dev(x.s0), chunk=64, scale=x.scale)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    for m in (64, 100, 1, 299):
        sl = lambda t, a, b_: t[:, :, a:b_].contiguous()
        o1, s1 = gdn.prefill(sl(q, 0, m), sl(k, 0, m), sl(v, 0, m), sl(g, 0, m), sl(beta, 0, m), dev(x.s0),
                             chunk=64, scale=x.scale)
        o2, s2 = gdn.prefill(sl(q, m, 300), sl(k, m, 300), sl(v, m, 300), sl(g, m, 300), sl(beta, m, 300), s1,
                             chunk=64, scale=x.scale)
        o_cat = np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], axis=2)
        assert rel_err(o_cat, o_ref) <= TOL_BF16, m
        assert rel_err(s2.cpu().numpy(), s_ref) <= TOL_BF16, m
    assert rel_err(o_full.cpu().numpy(), o_ref) <= TOL_BF16


def test_prefill_matches_decode_steps(gdn):
    """A T-token prefill equals T single-token decode calls (both within rounding)."""
    import torch
    x = inputs.generate(2, 40, 2, 4, 128, "bf16", seed=9, init_state="normal")
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    o_pf, s_pf = gdn.prefill(q, k, v, g, beta, dev(x.s0), chunk=16, scale=x.scale)
    state = dev(x.s0)
    outs = []
    for t in range(40):
        outs.append(gdn.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                               g[:, :, t].contiguous(), beta[:, :, t].contiguous(), state, scale=x.scale))
    o_dec = torch.stack(outs, dim=2)
    assert rel_err(o_pf.cpu().numpy(), o_dec.cpu().numpy()) <= TOL_BF16
    assert rel_err(s_pf.cpu().numpy(), state.cpu().numpy()) <= TOL_BF16


def test_prefill_repeatable(gdn):
    x = inputs.generate(1, 500, 2, 4, 128, "bf16", seed=10, init_state="normal")
    a = run_prefill(gdn, x, 64)
    b = run_prefill(gdn, x, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
