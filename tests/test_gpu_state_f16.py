"""float16 state storage (GDN_STATE_F16): decode and prefill against the float64 oracle, which
starts from the same float16 initial state and keeps its own state exact (needs an MI355X).

Bars: the recurrence runs in float32 and only the stored state is rounded, by at most 2^-11
of its value per write, so the bfloat16 bar (2e-3 of the largest value) holds for the bf16
paths and for the decode sequences (the emulated error of 64 float16-stored steps of the
batched workload is 3e-4); the float32 q/k/v path keeps its 1e-4 bar on o, and its float16
final state one rounding (2^-11) above that."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu
F16_ROUND = 2.0 ** -11


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def f16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()


def _step(x, s):
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
def test_decode_f16_state(gdn, oracle_lib, d, dtype, head_map):
    import torch
    steps = 4
    x = inputs.generate(3, 1, 2, 6, d, dtype, seed=90 + d, init_state="normal", decode_steps=steps)
    s16 = x.s0.astype(np.float16)
    state = f16_dev(s16)
    state32 = dev(s16.astype(np.float32))
    ref = np.ascontiguousarray(s16.astype(np.float64))
    for s in range(steps):
        st = _step(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, head_map=head_map, scale=x.scale)
        o32 = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state32, head_map=head_map, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref, scale=x.scale, head_map=head_map)
        torch.cuda.synchronize()
        assert rel_err(o.cpu().numpy(), o_ref) <= TOL_BF16, s
        if s == 0:
            # one step from the same state: the float16 state is the float32 one rounded, within
            # one float16 step (the two kernels sum their dot products in different orders)
            got, want = state.float().cpu().numpy(), state32.cpu().numpy()
            ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float32)
            assert np.all(np.abs(got - want) <= ulp + 1e-6 * np.abs(want).max()), (d, dtype)
            assert np.array_equal(o.cpu().numpy(), o32.cpu().numpy()) or \
                rel_err(o.cpu().numpy(), o32.cpu().numpy()) <= 1e-5
    es = rel_err(state.float().cpu().numpy(), ref)
    print(f"decode f16 state d{d} {dtype}: state rel err {es:.3e}")
    assert es <= TOL_BF16


def test_decode_f16_state_batched(gdn, oracle_lib):
    """B=256, Hk=16, Hv=32, d=128: 64 in-place steps on a 268 MB float16 state; 256 sampled
    (b, h) pairs checked at every step and at the end."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    B, Hv, d = wl.batch, wl.num_v_heads, wl.head_dim
    pairs = np.sort(np.random.default_rng(98).choice(B * Hv, size=256, replace=False))
    s16 = x.s0.astype(np.float16)
    state = f16_dev(s16)
    ref = np.ascontiguousarray(s16.reshape(B * Hv, d, d)[pairs].astype(np.float64))
    idx = torch.from_numpy(pairs).cuda()
    worst = 0.0
    for s in range(wl.decode_steps):
        st = _step(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref, scale=x.scale, pairs=pairs)
        worst = max(worst, rel_err(o.reshape(B * Hv, d)[idx].cpu().numpy(), o_ref))
    es = rel_err(state.reshape(B * Hv, d, d)[idx].float().cpu().numpy(), ref)
    print(f"batched decode, float16 state: max rel err o {worst:.3e}, state {es:.3e}")
    assert worst <= TOL_BF16 and es <= TOL_BF16
    assert torch.isfinite(state).all()


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("bf16", 32), ("bf16", 16), ("f32", 32)])
def test_prefill_f16_state(gdn, oracle_lib, dtype, chunk):
    import torch
    x = inputs.generate(2, 150, 2, 4, 128, dtype, seed=95 + chunk, init_state="normal")
    s16 = x.s0.astype(np.float16)
    q, k, v = qkv_dev(x)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), f16_dev(s16), chunk=chunk, scale=x.scale)
    assert sf.dtype == torch.float16
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, s16.astype(np.float64), scale=x.scale)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(sf.float().cpu().numpy(), s_ref)
    print(f"prefill {dtype} C{chunk}, float16 states: o {eo:.3e} state {es:.3e}")
    if dtype == "bf16":
        assert eo <= TOL_BF16 and es <= TOL_BF16
    else:
        assert eo <= TOL_F32 and es <= TOL_F32 + F16_ROUND
    # the same call with float32 states: o identical (the float16 initial state widens exactly),
    # the final state its float16 rounding
    o32, sf32 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(s16.astype(np.float32)), chunk=chunk,
                            scale=x.scale)
    assert torch.equal(o, o32)
    assert torch.equal(sf, sf32.half())


def test_prefill_f16_state_in_place_and_segmented(gdn, oracle_lib):
    """float16 state updated in place, over four segments (B=2, Hv=32, T=2000 at chunk 64 with
    the preferred workspace): segment starts are kept in float32 in the workspace and the final
    state is rounded once."""
    import torch
    assert gdn.prefill_segments(2, 2000, 16, 32, 128, 1 << 40, chunk=64) == 4
    x = inputs.generate(2, 2000, 16, 32, 128, "bf16", seed=97, init_state="normal")
    s16 = x.s0.astype(np.float16)
    q, k, v = qkv_dev(x)
    state = f16_dev(s16)
    o, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), state, chunk=64, scale=x.scale, final_state=state)
    s32 = dev(s16.astype(np.float32))
    o32, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s32, chunk=64, scale=x.scale, final_state=s32)
    torch.cuda.synchronize()
    assert torch.equal(o, o32)
    assert torch.equal(state, s32.half())  # carried in float32, rounded once at the end
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, s16.astype(np.float64), scale=x.scale)
    assert rel_err(o.cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_err(state.float().cpu().numpy(), s_ref) <= TOL_BF16


def test_zero_length_f16_state(gdn):
    import torch
    x = inputs.generate(2, 0, 2, 4, 128, "bf16", seed=96, init_state="normal")
    q, k, v = qkv_dev(x)
    s16 = x.s0.astype(np.float16)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), f16_dev(s16), chunk=64, scale=x.scale)
    torch.cuda.synchronize()
    assert o.numel() == 0 and sf.dtype == torch.float16
    assert np.array_equal(sf.cpu().numpy(), s16)


def test_binding_rejects_mixed_state_types(gdn):
    import torch
    x = inputs.generate(1, 8, 2, 4, 128, "bf16", seed=3, init_state="normal")
    q, k, v = qkv_dev(x)
    s16 = f16_dev(x.s0.astype(np.float16))
    with pytest.raises(TypeError, match="same type"):
        gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s16, final_state=torch.empty(s16.shape, device="cuda"),
                    scale=x.scale)
    with pytest.raises(TypeError):
        gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s16, state_dtype=torch.float32, scale=x.scale)
