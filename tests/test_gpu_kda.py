"""GPU parity of the per-channel-decay variant (gdn_kda_prefill, gdn_kda_decode) against the
float64 oracle's per-channel recurrence (needs an MI355X). The bf16 prefill runs the chunked form
(chunk 32 or 64: 32-token chunks, segment-parallel) or, with chunk 16, token by token."""
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


def check(oracle_lib, x, g, o, sf, tol, head_map=0, pairs=None, label=""):
    o_ref, s_ref = oracle_lib.kda_prefill(x.q, x.k, x.v, g, x.beta, x.s0, scale=x.scale, head_map=head_map,
                                          pairs=pairs)
    if pairs is not None:
        B, Hv = x.v.shape[:2]
        o = o.reshape(B * Hv, *o.shape[2:])[pairs]
        sf = sf.reshape(B * Hv, *sf.shape[2:])[pairs]
    eo, es = rel_err(o, o_ref), rel_err(sf, s_ref)
    print(f"{label}: rel err o {eo:.3e} state {es:.3e}")
    assert eo <= tol and es <= tol, (label, eo, es)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 32), ("bf16", 16), ("f32", 32)])
# one, two, three and four 16-token blocks and 32-token chunks, whole and ragged
@pytest.mark.parametrize("T", [1, 16, 37, 48, 64, 200])
@pytest.mark.parametrize("head_map", [0, 1])
def test_kda_prefill_small(gdn, oracle_lib, dtype, chunk, T, head_map):
    x = inputs.generate(2, T, 2, 4, 128, dtype, seed=120 + T, init_state="normal")
    g = inputs.generate_channel_decay((2, 4, T, 128), seed=121 + T)
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), dev(x.s0), chunk=chunk, head_map=head_map, scale=x.scale)
    check(oracle_lib, x, g, o.cpu().numpy(), sf.cpu().numpy(), tol_for(x), head_map=head_map,
          label=f"kda {dtype} C{chunk} T{T} map{head_map}")


@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_kda_chunked_segments(gdn, oracle_lib, P):
    """The chunked form split into P segments by the workspace size (maps, combine, output)."""
    import torch
    B, Hk, Hv, T = 1, 2, 4, 700
    x = inputs.generate(B, T, Hk, Hv, 128, "bf16", seed=140 + P, init_state="normal")
    g = inputs.generate_channel_decay((B, Hv, T, 128), seed=141 + P)
    nbytes = 3 * B * Hv * P * 128 * 128 * 4 if P > 1 else 0
    assert gdn.prefill_segments(B, T, Hk, Hv, 128, nbytes, chunk=32) == P
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), dev(x.s0), scale=x.scale, workspace=ws)
    check(oracle_lib, x, g, o.cpu().numpy(), sf.cpu().numpy(), TOL_BF16, label=f"kda chunked P{P}")


@pytest.mark.parametrize("mult", [3.0, 10.0])
def test_kda_chunked_strong_decay(gdn, oracle_lib, mult):
    """Per-channel decays three and ten times the workload's: at x10 a fifth of the steps fall
    below -10, which the chunked form takes as -10 (a difference below e^-10 of the state)."""
    x = inputs.generate(1, 200, 2, 4, 128, "bf16", seed=150, init_state="normal")
    g = inputs.generate_channel_decay((1, 4, 200, 128), seed=151, factor=mult)
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), dev(x.s0), scale=x.scale)
    check(oracle_lib, x, g, o.cpu().numpy(), sf.cpu().numpy(), TOL_BF16, label=f"kda chunked decay x{mult}")


def test_kda_chunk_64_runs_chunked(gdn):
    """chunk 64 is served by the 32-token chunked form: bit-equal to chunk 32."""
    import torch
    x = inputs.generate(1, 150, 2, 4, 128, "bf16", seed=152, init_state="normal")
    g = dev(inputs.generate_channel_decay((1, 4, 150, 128), seed=153))
    q, k, v = qkv_dev(x)
    o32, s32 = gdn.kda_prefill(q, k, v, g, dev(x.beta), dev(x.s0), chunk=32, scale=x.scale)
    o64, s64 = gdn.kda_prefill(q, k, v, g, dev(x.beta), dev(x.s0), chunk=64, scale=x.scale)
    assert torch.equal(o32, o64) and torch.equal(s32, s64)


def test_kda_prefill_empty(gdn):
    """No tokens: o is empty and the final state is the initial state, bit for bit."""
    import torch
    x = inputs.generate(2, 0, 2, 4, 128, "bf16", seed=126, init_state="normal")
    g = inputs.generate_channel_decay((2, 4, 0, 128), seed=127)
    q, k, v = qkv_dev(x)
    s0 = dev(x.s0)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), s0, scale=x.scale)
    assert o.shape == (2, 4, 0, 128)
    assert torch.equal(sf, s0)


def test_kda_uniform_decay_is_gdn(gdn):
    """Every channel of g_t equal: the per-channel prefill agrees with gdn_prefill."""
    x = inputs.generate(1, 300, 2, 4, 128, "bf16", seed=122, init_state="normal")
    q, k, v = qkv_dev(x)
    gc = np.repeat(x.g[..., None], 128, axis=-1)
    o1, s1 = gdn.kda_prefill(q, k, v, dev(gc), dev(x.beta), dev(x.s0), scale=x.scale)
    o2, s2 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale)
    assert rel_err(o1.cpu().numpy(), o2.cpu().numpy()) <= TOL_BF16
    assert rel_err(s1.cpu().numpy(), s2.cpu().numpy()) <= TOL_BF16


def test_kda_long_full(gdn, oracle_lib):
    """T = 32768 at the long workload's shape, per-channel decays -softplus(N(0,1)) * 0.1; every
    output and the final state of all 32 value heads against the oracle."""
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    g = inputs.generate_channel_decay(x.v.shape, seed=123, factor=0.1)
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), None, scale=x.scale)
    check(oracle_lib, x, g, o.cpu().numpy(), sf.cpu().numpy(), TOL_BF16, label="kda long_32k (all heads)")


def test_kda_prefill_equals_decode_steps(gdn):
    """A prefill of T tokens and T decode steps from the same state agree."""
    import torch
    T = 24
    x = inputs.generate(2, T, 2, 4, 128, "bf16", seed=124, init_state="normal")
    g = inputs.generate_channel_decay((2, 4, T, 128), seed=125)
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), dev(x.s0), chunk=16, scale=x.scale)  # token by token
    state = dev(x.s0)
    gd, bd = dev(g), dev(x.beta)
    for t in range(T):
        od = gdn.kda_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                            gd[:, :, t].contiguous(), bd[:, :, t].contiguous(), state, scale=x.scale)
        assert rel_err(od.cpu().numpy(), o[:, :, t].cpu().numpy()) <= 1e-5, t
    torch.cuda.synchronize()
    assert rel_err(state.cpu().numpy(), sf.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("state16", [False, True])
def test_kda_decode(gdn, oracle_lib, d, dtype, state16):
    import torch
    steps = 3
    x = inputs.generate(3, 1, 2, 6, d, dtype, seed=126 + d, init_state="normal", decode_steps=steps)
    g = inputs.generate_channel_decay((steps, 3, 6, d), seed=127 + d)
    s0 = x.s0.astype(np.float16) if state16 else x.s0
    state = torch.from_numpy(np.ascontiguousarray(s0)).cuda()
    ref = np.ascontiguousarray(s0.astype(np.float64))
    q, k, v = qkv_dev(x)
    bar = TOL_BF16 if (dtype == "bf16" or state16) else TOL_F32
    for s in range(steps):
        o = gdn.kda_decode(q[s], k[s], v[s], dev(g[s]), dev(x.beta[s]), state, scale=x.scale)
        o_ref = oracle_lib.kda_decode_step(x.q[s], x.k[s], x.v[s], g[s], x.beta[s], ref, scale=x.scale)
        assert rel_err(o.cpu().numpy(), o_ref) <= bar, s
    assert rel_err(state.float().cpu().numpy(), ref) <= bar


def test_kda_decode_batched(gdn, oracle_lib):
    """B=256, Hk=16, Hv=32, d=128: 64 in-place steps; every output of every step and the whole
    final state against the oracle."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    B, Hv, d = wl.batch, wl.num_v_heads, wl.head_dim
    g = inputs.generate_channel_decay((wl.decode_steps, B, Hv, d), seed=128)
    state = dev(x.s0)
    ref = np.ascontiguousarray(x.s0.astype(np.float64))
    q, k, v = qkv_dev(x)
    worst = 0.0
    for s in range(wl.decode_steps):
        o = gdn.kda_decode(q[s], k[s], v[s], dev(g[s]), dev(x.beta[s]), state, scale=x.scale)
        o_ref = oracle_lib.kda_decode_step(x.q[s], x.k[s], x.v[s], g[s], x.beta[s], ref, scale=x.scale)
        worst = max(worst, rel_err(o.cpu().numpy(), o_ref))
    assert torch.isfinite(state).all()
    es = rel_err(state.cpu().numpy(), ref)
    print(f"kda batched decode: o {worst:.3e} state {es:.3e}")
    assert worst <= 1e-4 and es <= 1e-4


def test_kda_storage_options(gdn):
    """float16 o equals the float32 o rounded; float16 states widen and round as stored."""
    import torch
    x = inputs.generate(1, 90, 2, 4, 128, "bf16", seed=130, init_state="normal")
    g = dev(inputs.generate_channel_decay((1, 4, 90, 128), seed=131))
    q, k, v = qkv_dev(x)
    s16 = torch.from_numpy(x.s0.astype(np.float16)).cuda()
    o32, f32 = gdn.kda_prefill(q, k, v, g, dev(x.beta), s16.float(), scale=x.scale)
    o16, f16 = gdn.kda_prefill(q, k, v, g, dev(x.beta), s16, scale=x.scale, o_dtype=torch.float16)
    assert torch.equal(o16, o32.half()) and torch.equal(f16, f32.half())
