"""GPU parity of gdn_gated_rmsnorm (applied to gdn_prefill / gdn_decode outputs) against the
float64 oracle's scan followed by its gated RMSNorm (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err, with_values

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


# ---- the norm as an argument of gdn_prefill / gdn_decode (gdn_norm): fused into the output
# store of the segmented bf16 prefill and of decode with >= 256 (b, h) pairs, a pass over o
# after the scan elsewhere; every path against the oracle's scan followed by its norm

# (q/k/v dtype, chunk, segments asked for): the segmented path with one and several segments at
# both chunk lengths (fused), the chunk-16 MFMA kernel and the float32 kernel (separate pass)
FUSED_PATHS = [("bf16", 64, 1), ("bf16", 64, 4), ("bf16", 32, 3), ("bf16", 16, 1), ("f32", 64, 1), ("f32", 16, 1)]
FUSED_IDS = [f"{d}-C{c}-P{p}" for d, c, p in FUSED_PATHS]


def prefill_fused(gdn, x, chunk, P, nrm, gated=True, o_dtype="f32", pairs=None):
    """gdn_prefill with the norm argument; returns (o, final state) as float32 numpy arrays
    (o restricted to the listed flattened pairs when given)."""
    import torch
    B, Hk, T, d = x.q.shape
    Hv = x.v.shape[1]
    nbytes = 3 * B * Hv * P * d * d * 4 if P > 1 else 0
    if x.qkv_dtype == "bf16" and chunk in (32, 64) and T > 0:
        used = gdn.prefill_segments(B, T, Hk, Hv, d, nbytes, chunk=chunk)
        assert (used > 1) == (P > 1) and used <= P, (used, P)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    q, k, v = qkv_dev(x)
    s0 = dev(x.s0) if x.s0 is not None else None
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s0, chunk=chunk, scale=x.scale, workspace=ws,
                        o_dtype=torch.float16 if o_dtype == "f16" else torch.float32,
                        norm_weight=dev(nrm.weight), norm_gate=gate_dev(nrm) if gated else None, norm_eps=EPS)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    if pairs is not None:
        o = o.reshape(B * Hv, T, d)[pairs]
    return o, sf.float().cpu().numpy()


def want_fused(oracle_lib, x, nrm, gated=True, pairs=None):
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, pairs=pairs)
    gate = nrm.gate
    if pairs is not None:
        B, Hv, T, d = gate.shape
        gate = gate.reshape(B * Hv, T, d)[pairs]
    return oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=gate if gated else None, eps=EPS), s_ref


def check_fused(got, want, label, tol, state=None):
    assert np.isfinite(got).all(), label
    err = rel_err(got, want)
    msg = f"{label}: rel err o {err:.3e}"
    if state is not None:
        es = rel_err(*state)
        msg += f" state {es:.3e}"
        assert es <= tol, (label, es)
    print(msg, flush=True)
    assert err <= tol, (label, err)


@pytest.mark.parametrize("gated", [True, False], ids=["gated", "ungated"])
@pytest.mark.parametrize("dtype,chunk,P", FUSED_PATHS, ids=FUSED_IDS)
def test_fused_prefill(gdn, oracle_lib, dtype, chunk, P, gated):
    """T = 300: several chunks and a ragged last one; the final state is unaffected by the norm."""
    x = inputs.generate(2, 300, 2, 4, 128, dtype, seed=71 + chunk + P, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, dtype, seed=72)
    o, sf = prefill_fused(gdn, x, chunk, P, nrm, gated)
    want, s_ref = want_fused(oracle_lib, x, nrm, gated)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    check_fused(o, want, f"fused {dtype} C{chunk} P{P} {'gated' if gated else 'ungated'}", tol, (sf, s_ref))


@pytest.mark.parametrize("dtype,chunk,P", [("bf16", 64, 4), ("bf16", 32, 1), ("f32", 16, 1)],
                         ids=["bf16-C64-P4", "bf16-C32-P1", "f32-C16-P1"])
def test_fused_prefill_f16_out(gdn, oracle_lib, dtype, chunk, P):
    x = inputs.generate(1, 200, 2, 4, 128, dtype, seed=73, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, dtype, seed=74)
    o, _ = prefill_fused(gdn, x, chunk, P, nrm, o_dtype="f16")
    want, _ = want_fused(oracle_lib, x, nrm)
    check_fused(o, want, f"fused f16 out {dtype} C{chunk} P{P}", TOL_BF16)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65])
def test_fused_prefill_short(gdn, oracle_lib, T):
    """Sequences of one partial chunk, exactly one chunk, and one token past it (segmented path)."""
    x = inputs.generate(1, T, 2, 4, 128, "bf16", seed=75 + T, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=76)
    o, sf = prefill_fused(gdn, x, 64, 1, nrm)
    want, s_ref = want_fused(oracle_lib, x, nrm)
    check_fused(o, want, f"fused T={T}", TOL_BF16, (sf, s_ref))


def test_fused_prefill_empty(gdn):
    """T = 0: no output rows; the call only copies the initial state to the final one."""
    import torch
    x = inputs.generate(1, 0, 2, 4, 128, "bf16", seed=77, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=78)
    q, k, v = qkv_dev(x)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale,
                        norm_weight=dev(nrm.weight), norm_gate=gate_dev(nrm), norm_eps=EPS)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(sf.cpu().numpy(), x.s0)


@pytest.mark.parametrize("mult", [1e-3, 30.0])
def test_fused_prefill_magnitudes(gdn, oracle_lib, mult):
    """Output rows far below and above unit size (v scaled): the norm takes them to unit size,
    so the staged values must keep their relative precision at any magnitude."""
    x = inputs.generate(1, 256, 2, 4, 128, "bf16", seed=79)
    x = with_values(x, v=x.v.astype(np.float64) * mult)
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=80)
    o, sf = prefill_fused(gdn, x, 64, 4, nrm)
    want, s_ref = want_fused(oracle_lib, x, nrm)
    check_fused(o, want, f"fused v x {mult}", TOL_BF16, (sf, s_ref))


def test_fused_prefill_4k(gdn, oracle_lib):
    wl = inputs.WORKLOADS["prefill_4k"]
    x = inputs.generate_workload(wl)
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=81)
    P = gdn.prefill_segments(1, x.q.shape[2], x.q.shape[1], x.v.shape[1], 128, 1 << 40, chunk=wl.chunk)
    o, _ = prefill_fused(gdn, x, wl.chunk, P, nrm)
    want, _ = want_fused(oracle_lib, x, nrm)
    check_fused(o, want, f"fused prefill_4k P{P}", TOL_BF16)


def test_fused_long_prefill_sampled(gdn, oracle_lib):
    """T = 32768 at its preferred segment count (the timed launch): 4 value heads in full."""
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=82)
    B, Hk, T, d = x.q.shape
    Hv = x.v.shape[1]
    P = gdn.prefill_segments(B, T, Hk, Hv, d, 1 << 40, chunk=wl.chunk)
    pairs = np.array([0, 9, 22, 31])
    o, _ = prefill_fused(gdn, x, wl.chunk, P, nrm, pairs=pairs)
    want, _ = want_fused(oracle_lib, x, nrm, pairs=pairs)
    check_fused(o, want, f"fused long_32k P{P} (4 heads)", TOL_BF16)


@pytest.mark.parametrize("B", [64, 8], ids=["fused-256pairs", "split-32pairs"])
@pytest.mark.parametrize("dtype,state,out", [("bf16", "f32", "f32"), ("f32", "f32", "f32"),
                                             ("bf16", "f16", "f16"), ("f32", "f16", "f32")])
def test_fused_decode(gdn, oracle_lib, B, dtype, state, out):
    """Three decode steps with the norm argument, state and outputs against the oracle."""
    import torch
    steps = 3
    x = inputs.generate(B, 0, 2, 4, 128, dtype, seed=83 + B, init_state="normal", decode_steps=steps)
    nrm = inputs.generate_norm((steps, B, 4, 128), dtype, seed=84)
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    st = dev(x.s0).to(torch.float16 if state == "f16" else torch.float32)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    if state == "f16":  # the device starts from the float16 rounding of the state
        ref_state = np.ascontiguousarray(x.s0.astype(np.float16).astype(np.float64))
    gated = dtype == "bf16"
    tol = TOL_BF16 if (dtype == "bf16" or state == "f16" or out == "f16") else TOL_F32
    for step in range(steps):
        sub = inputs.NormInputs(gate=nrm.gate[step], weight=nrm.weight,
                                gate_bits=None if nrm.gate_bits is None else nrm.gate_bits[step])
        o = gdn.decode(q[step], k[step], v[step], g[step], beta[step], st, scale=x.scale,
                       o_dtype=torch.float16 if out == "f16" else torch.float32,
                       norm_weight=dev(nrm.weight), norm_gate=gate_dev(sub) if gated else None, norm_eps=EPS)
        o_ref = oracle_lib.decode_step(x.q[step], x.k[step], x.v[step], x.g[step], x.beta[step], ref_state,
                                       scale=x.scale)
        want = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=nrm.gate[step] if gated else None, eps=EPS)
        torch.cuda.synchronize()
        check_fused(o.float().cpu().numpy(), want, f"fused decode B{B} {dtype} state {state} o {out} step {step}",
                    tol, (st.float().cpu().numpy(), ref_state))


def test_fused_decode_workload(gdn, oracle_lib):
    """The batched decode workload (256 x 32 pairs), four steps in place, all outputs."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    steps = 4
    nrm = inputs.generate_norm((steps,) + x.v.shape[1:], "bf16", seed=85)
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    st = dev(x.s0)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    for step in range(steps):
        sub = inputs.NormInputs(gate=nrm.gate[step], weight=nrm.weight, gate_bits=nrm.gate_bits[step])
        o = gdn.decode(q[step], k[step], v[step], g[step], beta[step], st, scale=x.scale,
                       norm_weight=dev(nrm.weight), norm_gate=gate_dev(sub), norm_eps=EPS)
        o_ref = oracle_lib.decode_step(x.q[step], x.k[step], x.v[step], x.g[step], x.beta[step], ref_state,
                                       scale=x.scale)
        want = oracle_lib.gated_rmsnorm(o_ref, nrm.weight, gate=nrm.gate[step], eps=EPS)
        torch.cuda.synchronize()
        check_fused(o.cpu().numpy(), want, f"fused decode workload step {step}", TOL_BF16)
