"""GPU parity of gdn_decode against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def _step_inputs(x, s):
    """Inputs of decode step s as a ScanInputs-like object with per-step arrays."""
    class Step:
        pass
    st = Step()
    st.qkv_dtype = x.qkv_dtype
    st.q, st.k, st.v = x.q[s], x.k[s], x.v[s]
    if x.qkv_dtype == "bf16":
        st.q_bits, st.k_bits, st.v_bits = x.q_bits[s], x.k_bits[s], x.v_bits[s]
    st.g, st.beta = x.g[s], x.beta[s]
    return st


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_map", [0, 1])
def test_decode_small(gdn, oracle_lib, d, dtype, head_map):
    import torch
    steps, B, Hk, Hv = 3, 3, 2, 6
    x = inputs.generate(B, 1, Hk, Hv, d, dtype, seed=40 + d, init_state="normal", decode_steps=steps)
    state = dev(x.s0)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    for s in range(steps):
        st = _step_inputs(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, head_map=head_map, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref_state, scale=x.scale,
                                       head_map=head_map)
        torch.cuda.synchronize()
        eo = rel_err(o.cpu().numpy(), o_ref)
        assert eo <= TOL_F32, (s, eo)
    es = rel_err(state.cpu().numpy(), ref_state)
    assert es <= TOL_F32, es


def test_decode_batched_full(gdn, oracle_lib):
    """B=256, Hk=16, Hv=32, d=128, 64 in-place steps on a 537 MB fp32 state, as the benchmark
    runs them: every output of every step and the whole final state against the oracle."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    state = dev(x.s0)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    worst = 0.0
    for s in range(wl.decode_steps):
        st = _step_inputs(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref_state, scale=x.scale)
        worst = max(worst, rel_err(o.cpu().numpy(), o_ref))
    assert torch.isfinite(state).all()
    es = rel_err(state.cpu().numpy(), ref_state)
    print(f"batched decode: max rel err o {worst:.3e}, state {es:.3e}")
    assert worst <= TOL_BF16 and es <= TOL_BF16
    assert worst <= 1e-4 and es <= 1e-4  # fp32 arithmetic: far inside the bf16 bar


def test_decode_repeatable(gdn):
    import torch
    x = inputs.generate(4, 1, 2, 4, 128, "bf16", seed=77, init_state="normal", decode_steps=1)
    st = _step_inputs(x, 0)
    q, k, v = qkv_dev(st)
    outs = []
    for _ in range(2):
        state = dev(x.s0)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, scale=x.scale)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), state.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("state16", [False, True])
@pytest.mark.parametrize("kda", [False, True])
def test_decode_row_split_is_exact(gdn, state16, kda):
    """Fewer (b, h) pairs than compute units split each pair's rows over several workgroups; the
    arithmetic of a row does not change, so one sequence alone (32 pairs, split) and the same
    sequence first in a batch of 8 (256 pairs, not split) agree bit for bit."""
    import torch
    B, Hk, Hv, d = 8, 16, 32, 128
    x = inputs.generate(B, 1, Hk, Hv, d, "bf16", seed=91, init_state="normal", decode_steps=1)
    st = _step_inputs(x, 0)
    q, k, v = qkv_dev(st)
    beta = dev(st.beta)
    g = dev(inputs.generate_channel_decay((B, Hv, d), seed=92)) if kda else dev(st.g)
    sdt = torch.float16 if state16 else torch.float32
    full = dev(x.s0).to(sdt)
    one = full[:1].clone()
    call = gdn.kda_decode if kda else gdn.decode
    o_full = call(q, k, v, g, beta, full, scale=x.scale)
    o_one = call(q[:1], k[:1], v[:1], g[:1], beta[:1], one, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_one[0], o_full[0])
    assert torch.equal(one[0], full[0])

