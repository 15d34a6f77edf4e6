"""Full-size parity of the option legs the benchmark times beside the headline calls: the long
prefill with float16 o, the input prologue on raw projections of the long workload's shape, the
gated RMSNorm epilogue over all 1,048,576 output rows, and the batched decode with the state
stored in float16 (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, dev, qkv_dev, rel_err
from tests.test_gpu_decode import _step_inputs
from tests.test_gpu_prologue import make_inputs, to_np, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def test_long_prefill_f16_o_full(gdn):
    """T = 32768, chunk 64: the float16-o call equals the float32-o call rounded to nearest even,
    bit for bit, over every output (the float32-o call is checked against the oracle in full)."""
    import torch
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    q, k, v = qkv_dev(x)
    args = (q, k, v, dev(x.g), dev(x.beta), None)
    o32, s32 = gdn.prefill(*args, chunk=wl.chunk, scale=x.scale)
    o16, s16 = gdn.prefill(*args, chunk=wl.chunk, scale=x.scale, o_dtype=torch.float16)
    assert torch.equal(o16, o32.half()) and torch.equal(s16, s32)


def test_prologue_full_shape(gdn, oracle_lib):
    """x [1][32768][8192] bf16 (Hk=16, Hv=32, d=128) with a conv state: every q, k and v value and
    the new state against the oracle, to one bf16 step per element."""
    Hk, Hv, d, T = 16, 32, 128, 32768
    xf, xb, w, st = make_inputs(1, T, Hk, Hv, d, "bf16", seed=80)
    st_dev = dev(st)
    q, k, v = gdn.qkv_prologue(x_dev(xf, xb), dev(w), st_dev, num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    rq, rk, rv, rst = oracle_lib.qkv_prologue(xf, w, Hk, Hv, d, state=st)
    del xf, xb
    for name, got, want in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        g_ = to_np(got)
        bound = 2.0 ** -8 * np.abs(want) + 1e-5 * np.max(np.abs(want))
        worst = float(np.max(np.abs(g_ - want) - bound))
        assert worst <= 0.0, (name, worst)
    assert np.array_equal(st_dev.cpu().numpy(), rst.astype(np.float32))


def test_gated_rmsnorm_full_rows(gdn, oracle_lib):
    """All 1,048,576 rows of 128 of the long prefill's output shape, float32 o, bf16 gate."""
    import torch
    rng = np.random.default_rng(81)
    o = (rng.standard_normal((1, 32, 32768, 128), dtype=np.float32) * 0.05)
    nrm = inputs.generate_norm(o.shape, "bf16", seed=82)
    t = torch.from_numpy(o).cuda()
    gate = torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    gdn.gated_rmsnorm(t, dev(nrm.weight), gate, eps=1e-6)
    want = oracle_lib.gated_rmsnorm(o, nrm.weight, gate=nrm.gate, eps=1e-6)
    err = rel_err(t.cpu().numpy(), want)
    print(f"gated rmsnorm, 1M rows: rel err {err:.3e}")
    assert err <= 1e-5  # float32 arithmetic on float32 rows


def test_decode_f16_state_full(gdn, oracle_lib):
    """B=256, Hk=16, Hv=32, d=128, the 64 benchmark steps on a float16 state: every output and the
    whole final state against the oracle started from the same float16 state (the storage
    rounding of 64 stored steps stays inside the bf16 bar)."""
    import torch
    wl = inputs.WORKLOADS["batched_decode"]
    x = inputs.generate_workload(wl)
    s16 = x.s0.astype(np.float16)
    state = torch.from_numpy(s16).cuda()
    ref_state = np.ascontiguousarray(s16.astype(np.float64))
    worst = 0.0
    for s in range(wl.decode_steps):
        st = _step_inputs(x, s)
        q, k, v = qkv_dev(st)
        o = gdn.decode(q, k, v, dev(st.g), dev(st.beta), state, scale=x.scale)
        o_ref = oracle_lib.decode_step(st.q, st.k, st.v, st.g, st.beta, ref_state, scale=x.scale)
        worst = max(worst, rel_err(o.cpu().numpy(), o_ref))
    es = rel_err(state.float().cpu().numpy(), ref_state)
    print(f"float16-state batched decode: max rel err o {worst:.3e}, state {es:.3e}")
    assert worst <= TOL_BF16 and es <= TOL_BF16
