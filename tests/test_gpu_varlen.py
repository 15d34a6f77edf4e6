"""GPU parity of gdn_prefill_varlen (sequences packed along one token axis, no padding)
against the float64 oracle run on the same sequences padded into a batch, which the padded
no-op rule makes exact on the real tokens (the oracle pins that rule bit for bit), and
against the GPU's own padded-batch prefill (needs an MI355X)."""
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


def bf(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def pack(x, lengths):
    """The real tokens of a padded ragged batch laid end to end: q, k [Hk][T][d] (bf16 bits),
    v [Hv][T][d], g, beta [Hv][T], and cu_seqlens."""
    cat = lambda a: np.concatenate([a[i, :, :n] for i, n in enumerate(lengths)], axis=1)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return cat(x.q_bits), cat(x.k_bits), cat(x.v_bits), cat(x.g), cat(x.beta), cu


def run_varlen(gdn, x, lengths, chunk, s0=None, **kw):
    import torch
    qb, kb, vb, g, beta, cu = pack(x, lengths)
    o, sf = gdn.prefill_varlen(bf(qb), bf(kb), bf(vb), dev(g), dev(beta), torch.from_numpy(cu).cuda(), s0,
                               chunk=chunk, scale=x.scale, **kw)
    return o, sf, cu


def check_against_padded(gdn, oracle_lib, x, lengths, chunk, label, tol=TOL_BF16):
    import torch
    s0 = dev(x.s0) if x.s0 is not None else None
    o, sf, cu = run_varlen(gdn, x, lengths, chunk, s0)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale)
    got = o.cpu().numpy()
    want = np.concatenate([o_ref[i, :, :n] for i, n in enumerate(lengths)], axis=1)
    eo, es = rel_err(got, want), rel_err(sf.cpu().numpy(), s_ref)
    print(f"{label}: rel err o {eo:.3e} state {es:.3e}")
    assert eo <= tol and es <= tol, (label, eo, es)
    # the GPU's padded batch on the real tokens: another kernel (the padded prefill sums in its
    # own order), so agreement to the same tolerance rather than bit for bit
    q, k, v = qkv_dev(x)
    op, sp = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), s0, chunk=chunk, scale=x.scale)
    torch.cuda.synchronize()
    opn = op.cpu().numpy()
    padded = np.concatenate([opn[i, :, :n] for i, n in enumerate(lengths)], axis=1)
    assert rel_err(got, padded) <= tol, label
    assert rel_err(sf.cpu().numpy(), sp.cpu().numpy()) <= tol, label
    return o, sf


@pytest.mark.parametrize("chunk", [64, 32])
def test_ragged_workload_packed(gdn, oracle_lib, chunk):
    """The ragged workload's sequences (401, 257, 33, 1 tokens; S0 ~ N(0, 0.1)) packed: 692
    tokens instead of 4 x 416 padded."""
    wl = inputs.WORKLOADS["ragged_continuation"]
    x = inputs.generate_workload(wl)
    check_against_padded(gdn, oracle_lib, x, list(wl.lengths), chunk, f"ragged packed C{chunk}")


def test_many_short_sequences(gdn, oracle_lib):
    """40 sequences of 0..150 tokens (empty ones first, inside and last), Hk=2, Hv=4."""
    rng = np.random.default_rng(101)
    lengths = list(rng.integers(0, 151, size=40))
    lengths[0], lengths[17], lengths[-1] = 0, 0, 0
    lengths[5], lengths[6] = 64, 1
    x = inputs.generate(40, max(lengths), 2, 4, 128, "bf16", seed=102, init_state="normal", lengths=lengths)
    check_against_padded(gdn, oracle_lib, x, lengths, 64, "40 short sequences")


def test_single_sequence_matches_prefill(gdn):
    """One packed sequence agrees with gdn_prefill on that sequence (another kernel, so to the
    bfloat16 tolerance rather than bit for bit)."""
    import torch
    x = inputs.generate(1, 300, 2, 4, 128, "bf16", seed=103, init_state="normal")
    o, sf, _ = run_varlen(gdn, x, [300], 64, dev(x.s0))
    q, k, v = qkv_dev(x)
    o2, sf2 = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), dev(x.s0), chunk=64, scale=x.scale)
    torch.cuda.synchronize()
    assert rel_err(o.cpu().numpy(), o2[0].cpu().numpy()) <= TOL_BF16
    assert rel_err(sf.cpu().numpy(), sf2.cpu().numpy()) <= TOL_BF16


def test_varlen_f16_states_in_place(gdn):
    """float16 states updated in place equal the float32 run's final states rounded."""
    import torch
    lengths = [130, 0, 77, 200]
    x = inputs.generate(4, 200, 2, 4, 128, "bf16", seed=104, init_state="normal", lengths=lengths)
    s16 = torch.from_numpy(x.s0.astype(np.float16)).cuda()
    s32 = s16.float()  # the same initial states, before the in-place update
    o16, _, _ = run_varlen(gdn, x, lengths, 64, s16, final_state=s16)
    o32, _, _ = run_varlen(gdn, x, lengths, 64, s32, final_state=s32)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)
    assert torch.equal(s16, s32.half())


def test_all_empty(gdn):
    """T = 0: every final state is its initial state."""
    import torch
    x = inputs.generate(3, 0, 2, 4, 128, "bf16", seed=105, init_state="normal")
    e = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((4, 0, 128), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((4, 0), dtype=torch.float32, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    o, sf = gdn.prefill_varlen(e, e, ev, z, z, cu, dev(x.s0), scale=x.scale)
    torch.cuda.synchronize()
    assert o.numel() == 0 and np.array_equal(sf.cpu().numpy(), x.s0)


def test_out_of_range_bounds_are_clamped(gdn):
    """cu_seqlens past the end is clamped to T, and tokens after the last sequence are left
    alone: the first sequence's results are unchanged and the rest of o keeps its contents."""
    import torch
    lengths = [100, 60]
    x = inputs.generate(2, 100, 2, 4, 128, "bf16", seed=106, init_state="normal", lengths=lengths)
    qb, kb, vb, g, beta, cu = pack(x, lengths)
    args = (bf(qb), bf(kb), bf(vb), dev(g), dev(beta))
    o_ok, sf_ok = gdn.prefill_varlen(*args, torch.from_numpy(cu).cuda(), dev(x.s0), scale=x.scale)
    big = torch.tensor([0, 100, 10_000], dtype=torch.int32, device="cuda")  # clamped to T = 160
    o_big, sf_big = gdn.prefill_varlen(*args, big, dev(x.s0), scale=x.scale)
    assert torch.equal(o_big, o_ok) and torch.equal(sf_big, sf_ok)
    short = torch.tensor([0, 100, 120], dtype=torch.int32, device="cuda")  # tokens 120.. unused
    o_s = torch.full_like(o_ok, 7.0)
    gdn.prefill_varlen(*args, short, dev(x.s0), scale=x.scale, o=o_s)
    torch.cuda.synchronize()
    assert torch.equal(o_s[:, :100], o_ok[:, :100])
    assert torch.equal(o_s[:, 100:120], o_ok[:, 100:120])  # causal: a shorter second sequence
    assert torch.all(o_s[:, 120:] == 7.0)
