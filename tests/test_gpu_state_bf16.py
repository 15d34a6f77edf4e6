"""bfloat16 state storage (GDN_STATE_BF16): decode, prefill and the per-channel-decay prefill
(needs an MI355X).

Decode writes the state every step, rounded to bfloat16 (up to 2^-8 of a value), so its
reference is the float64 oracle step with the state rounded to bfloat16 after every step (the
storage emulated): outputs within the bfloat16 bar, the first step's state within one bfloat16
rounding of it and later states within a few spacings of their largest value (the float32 and
float64 recurrences can round a value to neighbouring bfloat16 numbers, and the next step carries
that difference). The prefill carries its state in float32 and rounds once: o equals the
float32-state call from the widened initial state, and the final state is its float32 final
state rounded to bfloat16."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu
BF16_ULP = 2.0 ** -8  # a bfloat16 spacing is 2^-8 .. 2^-7 of a value; one rounding moves it by <= 2^-8


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def bf16_dev(a32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).cuda()


def bf16_values(a):
    """float64 -> float32 -> bfloat16 (round to nearest even) -> float64: what a stored state holds."""
    return inputs.bf16_to_f32(inputs.bf16_round(np.asarray(a, dtype=np.float32))).reshape(np.shape(a)).astype(np.float64)


def bf16_spacing(w):
    """The distance between neighbouring bfloat16 numbers at |w|: 2^(e - 8) for |w| in
    [2^(e-1), 2^e) (8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(w, dtype=np.float64)))
    return np.ldexp(1.0, e - 8)


def within_rounding(got, want, ulps=1.0):
    """How far |got - want| exceeds `ulps` bfloat16 spacings at want (plus a float32 floor);
    <= 0 when within."""
    got = np.asarray(got, dtype=np.float64)
    tol = ulps * bf16_spacing(want) + 1e-6 * np.abs(want).max()
    return float(np.max(np.abs(got - want) - tol))


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
def test_decode_bf16_state(gdn, oracle_lib, d, dtype, head_map):
    import torch
    steps = 4
    x = inputs.generate(3, 1, 2, 6, d, dtype, seed=300 + d, init_state="normal", decode_steps=steps)
    state = bf16_dev(x.s0)
    ref = np.ascontiguousarray(bf16_values(x.s0))
    for s in range(steps):
        st = _step(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, head_map=head_map, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref, scale=x.scale, head_map=head_map)
        ref[...] = bf16_values(ref)  # the stored state
        torch.cuda.synchronize()
        # o reads the state the previous step stored: a value rounded to the other neighbouring
        # bfloat16 number moves o by up to 2^-7 of that term, so the bar is the bf16 one
        assert rel_err(o.cpu().numpy(), o_ref) <= TOL_BF16, s
        got = state.float().cpu().numpy()
        if s == 0:
            # same stored input state: every value within one rounding of the reference's
            excess = within_rounding(got, ref, ulps=1.0)
            assert excess <= 0, (s, excess)
        else:
            # a neighbouring rounding carried from an earlier step can sit in a larger binade
            # than the decayed value: bound it by spacings of the largest value instead
            assert rel_err(got, ref) <= 2 * (s + 1) * BF16_ULP, s
    assert state.dtype == torch.bfloat16


def test_decode_bf16_state_batched(gdn, oracle_lib):
    """B=256, Hk=16, Hv=32, d=128: 64 in-place steps on a 268 MB bfloat16 state; 256 sampled
    (b, h) pairs against the storage-emulating reference at every step."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    B, Hv, d = wl.batch, wl.num_v_heads, wl.head_dim
    pairs = np.sort(np.random.default_rng(301).choice(B * Hv, size=256, replace=False))
    state = bf16_dev(x.s0)
    ref = np.ascontiguousarray(bf16_values(x.s0.reshape(B * Hv, d, d)[pairs]))
    idx = torch.from_numpy(pairs).cuda()
    worst_o = worst_s = 0.0
    for s in range(wl.decode_steps):
        st = _step(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref, scale=x.scale, pairs=pairs)
        ref[...] = bf16_values(ref)
        worst_o = max(worst_o, rel_err(o.reshape(B * Hv, d)[idx].cpu().numpy(), o_ref))
        worst_s = max(worst_s, rel_err(state.reshape(B * Hv, d, d)[idx].float().cpu().numpy(), ref))
    print(f"batched decode, bfloat16 state: max rel err o {worst_o:.3e}, state {worst_s:.3e}")
    # neighbouring-rounding differences stay within a few bfloat16 spacings of the largest value
    assert worst_o <= TOL_BF16 and worst_s <= 4 * BF16_ULP
    assert torch.isfinite(state.float()).all()


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("bf16", 32), ("bf16", 16), ("f32", 32)])
def test_prefill_bf16_state(gdn, oracle_lib, dtype, chunk):
    import torch
    x = inputs.generate(2, 150, 2, 4, 128, dtype, seed=302 + chunk, init_state="normal")
    s_bf = bf16_dev(x.s0)
    q, k, v = qkv_dev(x)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s_bf, chunk=chunk, scale=x.scale)
    assert sf.dtype == torch.bfloat16
    o32, sf32 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s_bf.float(), chunk=chunk, scale=x.scale)
    assert torch.equal(o, o32)
    assert torch.equal(sf, sf32.to(torch.bfloat16))
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, bf16_values(x.s0), scale=x.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert rel_err(o.cpu().numpy(), o_ref) <= tol
    assert rel_err(sf.float().cpu().numpy(), s_ref) <= tol + BF16_ULP  # one rounding


def test_prefill_bf16_state_in_place_and_segmented(gdn):
    """In place over four segments (B=2, Hv=32, T=2000, chunk 64, preferred workspace)."""
    import torch
    assert gdn.prefill_segments(2, 2000, 16, 32, 128, 1 << 40, chunk=64) == 4
    x = inputs.generate(2, 2000, 16, 32, 128, "bf16", seed=303, init_state="normal")
    q, k, v = qkv_dev(x)
    state = bf16_dev(x.s0)
    s32 = state.float()
    o, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), state, chunk=64, scale=x.scale, final_state=state)
    o32, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s32, chunk=64, scale=x.scale, final_state=s32)
    torch.cuda.synchronize()
    assert torch.equal(o, o32)
    assert torch.equal(state, s32.to(torch.bfloat16))


@pytest.mark.parametrize("chunk", [32, 16])
def test_kda_prefill_bf16_state(gdn, chunk):
    """The per-channel-decay prefill, chunked and token by token, with bfloat16 states."""
    import torch
    x = inputs.generate(1, 90, 2, 4, 128, "bf16", seed=304, init_state="normal")
    g = dev(inputs.generate_channel_decay((1, 4, 90, 128), seed=305))
    q, k, v = qkv_dev(x)
    s_bf = bf16_dev(x.s0)
    o, sf = gdn.kda_prefill(q, k, v, g, dev(x.beta), s_bf, chunk=chunk, scale=x.scale)
    o32, sf32 = gdn.kda_prefill(q, k, v, g, dev(x.beta), s_bf.float(), chunk=chunk, scale=x.scale)
    assert torch.equal(o, o32) and torch.equal(sf, sf32.to(torch.bfloat16))


def test_zero_length_bf16_state(gdn):
    import torch
    x = inputs.generate(2, 0, 2, 4, 128, "bf16", seed=306, init_state="normal")
    q, k, v = qkv_dev(x)
    s_bf = bf16_dev(x.s0)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s_bf, chunk=64, scale=x.scale)
    torch.cuda.synchronize()
    assert o.numel() == 0 and sf.dtype == torch.bfloat16 and torch.equal(sf, s_bf)
