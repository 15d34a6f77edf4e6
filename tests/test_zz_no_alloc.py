"""gdn_prefill_static, the prefill that allocates nothing, against gdn_prefill through the C ABI
(needs an MI355X). Both run the same kernels; the static call keeps its workspace in the
library's static device scratch instead of a caller's buffer, so at the same workspace size
(the same segment count) outputs and final states must agree bit for bit. Two calls in a row,
the second on a smaller input (the scratch then holds the first call's values), each also
against the float64 oracle within the bf16 bar; the 32768-token workload at its preferred
workspace; the fused norm; and no workspace at all."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def run(gdn, x, chunk, nbytes, static, norm=None):
    """One prefill into NaN-filled o and final state; returns them as numpy arrays."""
    import torch
    B, Hk, T, d = x.q.shape
    Hv = x.v.shape[1]
    q, k, v = qkv_dev(x)
    s0 = dev(x.s0) if x.s0 is not None else None
    o = torch.full((B, Hv, T, d), float("nan"), device="cuda")
    sf = torch.full((B, Hv, d, d), float("nan"), device="cuda")
    kw = dict(chunk=chunk, scale=x.scale, o=o, final_state=sf)
    if norm is not None:
        kw.update(norm_weight=norm[0], norm_gate=norm[1])
    print(f"{'static' if static else 'regular'} prefill B{B} Hk{Hk} Hv{Hv} T{T} C{chunk} ws {nbytes}", flush=True)
    if static:
        gdn.prefill_static(q, k, v, dev(x.g), dev(x.beta), s0, workspace_bytes=nbytes, **kw)
    else:
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s0, workspace=ws, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), sf.cpu().numpy()


def check_pair(gdn, x, chunk, nbytes, norm=None):
    Bsz, Hk, T, d = x.q.shape
    P = gdn.prefill_segments(Bsz, T, Hk, x.v.shape[1], d, nbytes, chunk=chunk)
    o_s, s_s = run(gdn, x, chunk, nbytes, True, norm)
    o_r, s_r = run(gdn, x, chunk, nbytes, False, norm)
    assert np.array_equal(o_s, o_r), f"o differs (P = {P})"
    assert np.array_equal(s_s, s_r), f"final state differs (P = {P})"
    return P, o_s, s_s


def test_two_calls_in_a_row(gdn, oracle_lib):
    # the first call fills much of the scratch (16 segments of 4 pairs), the second uses less of it
    cases = [(inputs.generate(1, 1000, 2, 4, 128, "bf16", seed=91, init_state="normal"), 64),
             (inputs.generate(1, 300, 1, 2, 128, "bf16", seed=92, init_state="normal"), 32)]
    used = []
    for x, chunk in cases:
        B, Hk, T, d = x.q.shape
        nbytes = gdn.prefill_workspace_bytes(B, T, Hk, x.v.shape[1], d, chunk=chunk)
        assert 0 < nbytes <= gdn.STATIC_SCRATCH_BYTES
        P, o, sf = check_pair(gdn, x, chunk, nbytes)
        assert P > 1
        used.append(nbytes)
        o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
        eo, es = rel_err(o, o_ref), rel_err(sf, s_ref)
        print(f"P {P}: rel err o {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16
    assert used[1] < used[0]


def test_long_prefill_preferred_workspace(gdn, oracle_lib):
    """T = 32768, 32 value heads, at the preferred segment count (the launch the bench times)."""
    wl = inputs.WORKLOADS["long_prefill_32k"]
    x = inputs.generate_workload(wl)
    B, Hk, T, d = x.q.shape
    nbytes = gdn.prefill_workspace_bytes(B, T, Hk, x.v.shape[1], d, chunk=wl.chunk)
    assert nbytes <= gdn.STATIC_SCRATCH_BYTES
    P, o, _ = check_pair(gdn, x, wl.chunk, nbytes)
    assert P > 1
    pairs = np.array([0, 31])
    o_ref, _ = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, pairs=pairs)
    err = rel_err(o.reshape(B * x.v.shape[1], T, d)[pairs], o_ref)
    print(f"long_32k P {P}: rel err o (2 heads) {err:.3e}", flush=True)
    assert err <= TOL_BF16


def test_fused_norm_and_no_workspace(gdn):
    import torch
    x = inputs.generate(2, 500, 2, 4, 128, "bf16", seed=93, init_state="normal")
    nrm = inputs.generate_norm(x.v.shape, "bf16", seed=94)
    gate = torch.from_numpy(np.ascontiguousarray(nrm.gate_bits).view(np.int16)).view(torch.bfloat16).cuda()
    norm = (dev(nrm.weight), gate)
    nbytes = gdn.prefill_workspace_bytes(2, 500, 2, 4, 128, chunk=64)
    assert check_pair(gdn, x, 64, nbytes, norm)[0] > 1
    assert check_pair(gdn, x, 64, 0)[0] == 1
