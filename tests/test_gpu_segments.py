"""GPU parity of the segmented bfloat16 prefill (head_dim 128, chunk 16, 32 and 64) against the
float64 oracle, over the segment counts the workspace size selects: one segment (no
workspace), two, several, and one per chunk; ragged tails, both head maps, in-place and
float16 storage (needs an MI355X).

The cases run from the simplest up, so that the first failure names the smallest case."""
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


def _ws_bytes(B, Hv, P):
    return 3 * B * Hv * P * 128 * 128 * 4 if P > 1 else 0


def run(gdn, x, chunk, P, head_map=0, init=True, **kw):
    """gdn_prefill with a workspace sized for P segments; checks that P is what the call uses."""
    import torch
    B, Hk, T, d = x.q.shape
    Hv = x.v.shape[1]
    nbytes = _ws_bytes(B, Hv, P)
    used = gdn.prefill_segments(B, T, Hk, Hv, d, nbytes, chunk=chunk)
    assert used == P, (used, P)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    q, k, v = qkv_dev(x)
    s0 = dev(x.s0) if (init and x.s0 is not None) else None
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s0, chunk=chunk, head_map=head_map, scale=x.scale,
                        workspace=ws, **kw)
    torch.cuda.synchronize()
    return o, sf


def check(oracle_lib, x, o, sf, head_map=0, init=True, tol=TOL_BF16, label=""):
    s0 = x.s0 if init else None
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, s0, scale=x.scale, head_map=head_map)
    o = o.float().cpu().numpy()
    eo = rel_err(o, o_ref)
    es = rel_err(sf.float().cpu().numpy(), s_ref) if sf is not None else 0.0
    print(f"{label}: rel err o {eo:.3e} state {es:.3e}", flush=True)
    assert np.isfinite(o).all()
    assert eo <= tol, (label, eo)
    assert es <= tol, (label, es)
    return o_ref, s_ref


@pytest.mark.parametrize("T,chunk,P,init", [
    (64, 64, 1, False),     # one chunk, zero state
    (64, 64, 1, True),      # one chunk from a state
    (100, 32, 1, True),     # several chunks, ragged tail, one segment
    (100, 32, 2, True),     # two segments
    (100, 32, 4, True),     # one chunk per segment
    (200, 64, 2, True),
    (200, 64, 4, True),
    (1000, 64, 3, True),
    (1000, 32, 5, True),
    (1000, 64, 16, True),   # the preferred count for 4 value heads: one chunk per segment
    (4100, 64, 8, True),
    (40, 16, 1, True),      # chunk 16: one tile per chunk, ragged tail
    (40, 16, 3, True),      # one chunk per segment
    (300, 16, 4, True),
    (1000, 16, 16, True),
])
def test_segment_counts(gdn, oracle_lib, T, chunk, P, init):
    x = inputs.generate(1, T, 2, 4, 128, "bf16", seed=T + chunk + P, init_state="normal")
    o, sf = run(gdn, x, chunk, P, init=init)
    check(oracle_lib, x, o, sf, init=init, label=f"T{T} C{chunk} P{P} init{init}")


@pytest.mark.parametrize("T,chunk,P", [(1000, 64, 16), (4100, 64, 8), (1000, 32, 5), (1000, 16, 16)])
def test_segment_counts_slow_decay(gdn, oracle_lib, T, chunk, P):
    """Gates near one: the state that enters a segment still counts at its end, so the chain
    S_{p+1} = S_p M_p + N_p carries a full-rank share of the result through every segment."""
    x = inputs.generate(1, T, 2, 4, 128, "bf16", seed=7 * T + chunk + P, init_state="normal", decay_mult=0.002)
    seg = T / P
    assert np.exp(x.g.astype(np.float64)[..., :int(seg)].sum(axis=-1)).min() > 0.05  # a segment keeps > 5%
    o, sf = run(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, label=f"slow decay T{T} C{chunk} P{P}")


@pytest.mark.parametrize("T", [1, 15, 33])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_short_sequences(gdn, oracle_lib, T, chunk):
    """Fewer tokens than a chunk (or just over one): the whole sequence is a masked tail."""
    x = inputs.generate(2, T, 2, 4, 128, "bf16", seed=40 + T, init_state="normal")
    P = gdn.prefill_segments(2, T, 2, 4, 128, 1 << 40, chunk=chunk)
    assert P == -(-T // chunk)
    o, sf = run(gdn, x, chunk, P)
    check(oracle_lib, x, o, sf, label=f"short T{T} C{chunk}")


@pytest.mark.parametrize("Hk,Hv", [(4, 4), (2, 8)])
@pytest.mark.parametrize("head_map", [0, 1])
def test_head_maps(gdn, oracle_lib, Hk, Hv, head_map):
    x = inputs.generate(2, 700, Hk, Hv, 128, "bf16", seed=50 + Hk + Hv + head_map, init_state="normal")
    for P in (1, 3):
        o, sf = run(gdn, x, 64, P, head_map=head_map)
        check(oracle_lib, x, o, sf, head_map=head_map, label=f"Hk{Hk} Hv{Hv} map{head_map} P{P}")


def test_preferred_workspace(gdn, oracle_lib):
    """The binding's default: the workspace of the preferred segment count (B=2, Hv=32,
    T=2000, chunk 64: four segments of 8 chunks, the last ragged)."""
    x = inputs.generate(2, 2000, 16, 32, 128, "bf16", seed=12, init_state="normal")
    assert gdn.prefill_segments(2, 2000, 16, 32, 128, 1 << 40, chunk=64) == 4
    q, k, v = qkv_dev(x)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale)
    check(oracle_lib, x, o, sf, label="preferred workspace")


def test_in_place_and_no_final_state(gdn, oracle_lib):
    """With several segments: the state updated in place (the output pass must start segment 0
    from the map pass's copy), and a call that asks for no final state."""
    import torch
    x = inputs.generate(1, 900, 2, 4, 128, "bf16", seed=13, init_state="normal")
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    nbytes = _ws_bytes(1, 4, 5)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    q, k, v = qkv_dev(x)
    state = dev(x.s0)
    o, _ = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), state, chunk=64, scale=x.scale, final_state=state,
                       workspace=ws)
    torch.cuda.synchronize()
    assert rel_err(o.cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_err(state.cpu().numpy(), s_ref) <= TOL_BF16
    o2, none = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale,
                           write_final_state=False, workspace=ws)
    assert none is None
    assert rel_err(o2.cpu().numpy(), o_ref) <= TOL_BF16


def test_f16_storage(gdn, oracle_lib):
    """float16 initial/final state and float16 o with several segments; the float16-o result is
    the float32-o result rounded, bit for bit."""
    import torch
    x = inputs.generate(1, 700, 2, 4, 128, "bf16", seed=14, init_state="normal")
    s0h = x.s0.astype(np.float16)
    q, k, v = qkv_dev(x)
    for P in (1, 4):
        ws = torch.empty(max(_ws_bytes(1, 4, P), 1), dtype=torch.uint8, device="cuda")
        init = torch.from_numpy(s0h).cuda()
        o32, s32 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=32, scale=x.scale, workspace=ws)
        o16, s16 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=32, scale=x.scale, workspace=ws,
                               o_dtype=torch.float16)
        torch.cuda.synchronize()
        assert s32.dtype == torch.float16
        assert torch.equal(o16, o32.half()) and torch.equal(s16, s32)
        o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, s0h.astype(np.float64), scale=x.scale)
        assert rel_err(o32.cpu().numpy(), o_ref) <= TOL_BF16
        assert rel_err(s32.float().cpu().numpy(), s_ref) <= TOL_BF16


def test_batch_fills_gpu_without_segments(gdn, oracle_lib):
    """B * Hv = 256 (B = 8, Hv = 32): the preferred count is one segment, no workspace; checked
    on a subset of pairs."""
    x = inputs.generate(8, 300, 16, 32, 128, "bf16", seed=15, init_state="normal")
    assert gdn.prefill_workspace_bytes(8, 300, 16, 32, 128, chunk=64) == 0
    q, k, v = qkv_dev(x)
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale)
    pairs = np.arange(0, 256, 17)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, pairs=pairs)
    o_np = o.cpu().numpy().reshape(256, 300, 128)[pairs]
    s_np = sf.cpu().numpy().reshape(256, 128, 128)[pairs]
    assert rel_err(o_np, o_ref) <= TOL_BF16 and rel_err(s_np, s_ref) <= TOL_BF16


def test_segmented_repeatable(gdn):
    """Bitwise run-to-run repeatability with several segments."""
    import torch
    x = inputs.generate(1, 1500, 2, 4, 128, "bf16", seed=16, init_state="normal")
    a = run(gdn, x, 64, 6)
    b = run(gdn, x, 64, 6)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
