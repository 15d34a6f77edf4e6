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


def test_segmented_prefill(gdn, oracle_lib, monkeypatch):
    """A prefill run as several token segments (B=2, Hv=32, T=2000 at chunk 64 under a 160 MiB
    segment budget: two segments of 16 chunks, the last ragged), with the carried state in the
    caller's final_state, in the workspace (no final state asked for), and in place."""
    import torch
    monkeypatch.setenv("GDN_PREFILL_SEGMENT_BYTES", str(160 << 20))
    x = inputs.generate(2, 2000, 16, 32, 128, "bf16", seed=12, init_state="normal")
    shape = gdn.make_shape(batch=2, seq_len=2000, num_k_heads=16, num_v_heads=32, head_dim=128, chunk=64,
                           qkv_dtype=gdn.GDN_DTYPE_BF16, head_map=0, scale=x.scale)
    lib = gdn.load_library()
    import ctypes
    ws = lib.gdn_prefill_workspace_bytes(ctypes.byref(shape))
    full = 2 * (2 * 32 * 32 * (2 * 64 * 64 + 6 * 64) + 2 * 16 * 32 * 64 * 256)
    assert 0 < ws < full  # smaller than one workspace for the whole sequence
    o, sf = run_prefill(gdn, x, 64)
    o_ref, s_ref = check(oracle_lib, x, o, sf, label="segmented, state via final_state")
    q, k, v = qkv_dev(x)
    o2, none = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale,
                           write_final_state=False)
    assert none is None
    assert rel_err(o2.cpu().numpy(), o_ref) <= TOL_BF16
    state = dev(x.s0)
    o3, s3 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), state, chunk=64, scale=x.scale, final_state=state)
    torch.cuda.synchronize()
    assert rel_err(o3.cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_err(state.cpu().numpy(), s_ref) <= TOL_BF16


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
