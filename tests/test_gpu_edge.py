"""GPU parity at the method's edge cases, element by element against the float64 oracle, on
every prefill path and on decode (needs an MI355X):

* strong decay: g ten times the workload's (G falls by ~450 inside one 64-token chunk, so
  exp(G) underflows within the chunk);
* recall: beta = 1, g = 0, one-hot keys (k_t = e_{t mod d}) and q_t = k_t, so that every
  step overwrites one state column with its value: S e_j holds the last value written to key
  j, and o_t = scale * v_t;
* pure decay: beta = 0, so o_t = exp(G_t) S0 (scale q_t) and the final state is exp(G_T) S0
  (a weak decay, g / 50, so that exp(G_T) stays far from float32 underflow);
* magnitudes near the float16 operand limit of the bf16 MFMA paths (v ~ 4e3 N(0,1), initial
  state ~ N(0, 1.5e3^2): every operand within a factor ~3 of 65504), and the documented
  behaviour beyond it (an initial state with entries ~1e5 gives non-finite outputs on those
  paths, finite and exact ones on the float32 path and on decode);
* a prefill on a stream other than the current one, its workspace allocated by the binding.
"""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err, with_values

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


# (q/k/v dtype, chunk, segments): the segmented bf16 path with one and several segments at
# both chunk lengths, the fused chunk-16 MFMA kernel, the float32 VALU kernel
PATHS = [("bf16", 64, 1), ("bf16", 64, 4), ("bf16", 32, 3), ("bf16", 16, 1), ("f32", 64, 1), ("f32", 16, 1)]
PATH_IDS = [f"{d}-C{c}-P{p}" for d, c, p in PATHS]


def run_prefill(gdn, x, chunk, P):
    import torch
    B, Hk, T, d = x.q.shape
    Hv = x.v.shape[1]
    nbytes = 3 * B * Hv * P * d * d * 4 if P > 1 else 0
    if x.qkv_dtype == "bf16" and chunk in (32, 64):
        # the library evens out the segment lengths, which can lower the count asked for
        used = gdn.prefill_segments(B, T, Hk, Hv, d, nbytes, chunk=chunk)
        assert (used > 1) == (P > 1) and used <= P, (used, P)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    q, k, v = qkv_dev(x)
    s0 = dev(x.s0) if x.s0 is not None else None
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s0, chunk=chunk, scale=x.scale, workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), sf.float().cpu().numpy()


def check(oracle_lib, x, o, sf, label, tol=None):
    tol = tol if tol is not None else (TOL_BF16 if x.qkv_dtype == "bf16" else TOL_F32)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    assert np.isfinite(o).all() and np.isfinite(sf).all(), label
    eo, es = rel_err(o, o_ref), rel_err(sf, s_ref)
    print(f"{label}: rel err o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= tol and es <= tol, (label, eo, es)
    return o_ref, s_ref


@pytest.mark.parametrize("dtype,chunk,P", PATHS, ids=PATH_IDS)
def test_strong_decay(gdn, oracle_lib, dtype, chunk, P):
    x = inputs.generate(1, 300, 2, 4, D, dtype, seed=61, decay_mult=10.0, init_state="normal")
    assert x.g.sum(axis=-1).min() < -500  # G reaches below -500 within the sequence
    o, sf = run_prefill(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, f"strong decay {dtype} C{chunk} P{P}")


def _recall_inputs(dtype, T, seed):
    x = inputs.generate(1, T, 2, 4, D, dtype, seed=seed)
    k = np.zeros(x.k.shape)
    t = np.arange(T)
    for h in range(x.k.shape[1]):
        k[0, h, t, (t + 17 * h) % D] = 1.0  # one-hot keys, a different order per key head
    return with_values(x, q=k, k=k, g=np.zeros_like(x.g), beta=np.ones_like(x.beta), s0=None)


@pytest.mark.parametrize("dtype,chunk,P", PATHS, ids=PATH_IDS)
def test_recall_one_hot(gdn, oracle_lib, dtype, chunk, P):
    T = 200  # keys repeat after 128 tokens: later writes overwrite earlier ones
    x = _recall_inputs(dtype, T, seed=62)
    o, sf = run_prefill(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, f"recall {dtype} C{chunk} P{P}")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    vmax = np.abs(x.v).max()
    # o_t = scale * v_t: the step writes v_t into column key_t and reads that column back
    assert np.abs(o - x.scale * x.v).max() <= tol * x.scale * vmax
    # S e_j = the last value written to key j (value heads read key head h % 2)
    for h in range(4):
        kh = h % 2
        for j in range(D):
            ts = [t for t in range(T) if (t + 17 * kh) % D == j]
            want = x.v[0, h, ts[-1]] if ts else np.zeros(D)
            assert np.abs(sf[0, h, :, j] - want).max() <= tol * vmax, (h, j)


@pytest.mark.parametrize("dtype,chunk,P", PATHS, ids=PATH_IDS)
def test_pure_decay(gdn, oracle_lib, dtype, chunk, P):
    x = inputs.generate(1, 150, 2, 4, D, dtype, seed=63, init_state="normal", decay_mult=0.02)
    x = with_values(x, beta=np.zeros_like(x.beta))
    assert -10 < x.g.sum(axis=-1).min() < -0.5
    o, sf = run_prefill(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, f"pure decay {dtype} C{chunk} P{P}")
    # closed form: o_t = exp(G_t) S0 (scale q_t), S_T = exp(G_T) S0
    G = np.cumsum(x.g.astype(np.float64), axis=-1)
    s0 = x.s0.astype(np.float64)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for h in range(4):
        q = x.q[0, h % 2].astype(np.float64)                      # [T][d]
        o_cf = np.exp(G[0, h])[:, None] * (q @ s0[0, h].T) * x.scale
        assert rel_err(o[0, h], o_cf) <= tol
        assert rel_err(sf[0, h], np.exp(G[0, h, -1]) * s0[0, h]) <= tol


@pytest.mark.parametrize("dtype,chunk,P", PATHS, ids=PATH_IDS)
def test_near_fp16_limit(gdn, oracle_lib, dtype, chunk, P):
    x = inputs.generate(1, 256, 2, 4, D, dtype, seed=71, init_state="normal")
    x = with_values(x, v=x.v.astype(np.float64) * 4000.0, s0=x.s0 * 15000.0)  # S0 ~ N(0, 1500^2)
    assert 1.2e4 < np.abs(x.v).max() < 6.5e4 and np.abs(x.s0).max() > 5e3
    o, sf = run_prefill(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, f"near fp16 limit {dtype} C{chunk} P{P}")


@pytest.mark.parametrize("dtype,chunk,P", PATHS, ids=PATH_IDS)
def test_beyond_fp16_range(gdn, oracle_lib, dtype, chunk, P):
    """The documented contract: a state beyond +-65504 overflows the float16 operands of the
    bf16 MFMA paths (non-finite outputs, no error); the float32 path stays exact."""
    x = inputs.generate(1, 100, 2, 4, D, dtype, seed=72, init_state="normal")
    x = with_values(x, s0=x.s0 * 1e6)  # S0 ~ N(0, 1e5^2)
    assert np.abs(x.s0).max() > 65504
    o, sf = run_prefill(gdn, x, chunk, P)
    if dtype == "bf16":
        assert not np.isfinite(o).all()
    else:
        check(oracle_lib, x, o, sf, f"beyond fp16 range {dtype} C{chunk}")


def _decode_run(gdn, x, steps):
    import torch
    from tests.gpu_util import bf16_dev
    state = dev(x.s0)
    os_ = []
    for s in range(steps):
        if x.qkv_dtype == "bf16":
            q, k, v = bf16_dev(x.q_bits[s]), bf16_dev(x.k_bits[s]), bf16_dev(x.v_bits[s])
        else:
            q, k, v = dev(x.q[s]), dev(x.k[s]), dev(x.v[s])
        os_.append(gdn.decode(q, k, v, dev(x.g[s]), dev(x.beta[s]), state, scale=x.scale).cpu().numpy())
    torch.cuda.synchronize()
    return np.stack(os_), state.cpu().numpy()


def _decode_ref(oracle_lib, x, steps):
    st = np.ascontiguousarray(x.s0.astype(np.float64))
    outs = []
    for s in range(steps):
        outs.append(oracle_lib.decode_step(x.q[s], x.k[s], x.v[s], x.g[s], x.beta[s], st, scale=x.scale))
    return np.stack(outs), st


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["strong_decay", "pure_decay", "recall", "beyond_fp16"])
def test_decode_edges(gdn, oracle_lib, dtype, case):
    steps, B = 16, 3
    x = inputs.generate(B, 1, 2, 4, D, dtype, seed=80, init_state="normal", decode_steps=steps,
                        decay_mult=10.0 if case == "strong_decay" else 1.0)
    if case == "pure_decay":
        x = with_values(x, beta=np.zeros_like(x.beta))
    elif case == "recall":
        k = np.zeros(x.k.shape)
        for s in range(steps):
            k[s, :, :, (5 * s) % D] = 1.0
        x = with_values(x, q=k, k=k, g=np.zeros_like(x.g), beta=np.ones_like(x.beta))
    elif case == "beyond_fp16":
        x = with_values(x, s0=x.s0 * 1e6)
    o, st = _decode_run(gdn, x, steps)
    o_ref, s_ref = _decode_ref(oracle_lib, x, steps)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert np.isfinite(o).all() and np.isfinite(st).all()
    assert rel_err(o, o_ref) <= tol and rel_err(st, s_ref) <= tol, (case, rel_err(o, o_ref), rel_err(st, s_ref))
    if case == "recall":
        assert np.abs(o - x.scale * x.v).max() <= tol * x.scale * np.abs(x.v).max()


def test_prefill_on_side_stream(gdn, oracle_lib):
    """A prefill enqueued on a stream that is not the current one, with the workspace the
    binding allocates: the block must not be handed to work on the current stream while the
    prefill still runs (allocations on the current stream follow it at once)."""
    import torch
    x = inputs.generate(2, 2000, 16, 32, D, "bf16", seed=90, init_state="normal")
    q, k, v = qkv_dev(x)
    g, beta, s0 = dev(x.g), dev(x.beta), dev(x.s0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, sf = gdn.prefill(q, k, v, g, beta, s0, chunk=64, scale=x.scale, stream=side)
    junk = [torch.full((1 << 24,), 7.0, device="cuda") for _ in range(4)]  # current stream
    torch.cuda.synchronize()
    del junk
    check(oracle_lib, x, o.cpu().numpy(), sf.cpu().numpy(), "side stream")
