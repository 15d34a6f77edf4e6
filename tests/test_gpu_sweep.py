"""Randomised GPU parity sweep: seeded random shapes and options of gdn_prefill (batch, length,
head counts and map, chunk, initial state, state and output storage) and of the packed and
per-channel-decay entry points, each against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest

from gated_delta_rule_56_amd import inputs
from tests.gpu_util import TOL_BF16, TOL_F32, dev, qkv_dev, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_56_amd import binding
    return binding


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    Hk = int(rng.choice([1, 2, 4]))
    Hv = Hk * int(rng.choice([1, 2, 3]))
    bf16 = bool(rng.integers(0, 4))  # mostly bfloat16
    d = 128 if bf16 else int(rng.choice([16, 32, 64, 128]))
    return dict(B=int(rng.integers(1, 4)), T=int(rng.integers(0, 300)), Hk=Hk, Hv=Hv, d=d,
                dtype="bf16" if bf16 else "f32", chunk=int(rng.choice([16, 32, 64])),
                head_map=int(rng.integers(0, 2)), init=bool(rng.integers(0, 2)),
                st16=bool(rng.integers(0, 3) == 0), o16=bool(rng.integers(0, 3) == 0))


@pytest.mark.parametrize("seed", range(24))
def test_prefill_sweep(gdn, oracle_lib, seed):
    import torch
    c = _case(seed)
    if c["o16"] and (c["dtype"] != "bf16" or c["chunk"] == 16):
        c["o16"] = False  # float16 o: the bfloat16 chunk-32/64 path only
    x = inputs.generate(c["B"], c["T"], c["Hk"], c["Hv"], c["d"], c["dtype"], seed=2000 + seed,
                        init_state="normal" if c["init"] else "zero")
    q, k, v = qkv_dev(x)
    s0 = x.s0.astype(np.float16) if (c["init"] and c["st16"]) else x.s0
    init = torch.from_numpy(np.ascontiguousarray(s0)).cuda() if c["init"] else None
    o, sf = gdn.prefill(q, k, v, dev(x.g), dev(x.beta), init, chunk=c["chunk"], head_map=c["head_map"],
                        scale=x.scale, state_dtype=torch.float16 if c["st16"] else None,
                        o_dtype=torch.float16 if c["o16"] else torch.float32)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta,
                                      None if s0 is None else s0.astype(np.float64), scale=x.scale,
                                      head_map=c["head_map"])
    tol = TOL_BF16 if (c["dtype"] == "bf16" or c["st16"] or c["o16"]) else TOL_F32
    eo = rel_err(o.float().cpu().numpy(), o_ref)
    es = rel_err(sf.float().cpu().numpy(), s_ref)
    print(f"sweep {seed} {c}: o {eo:.2e} state {es:.2e}")
    assert eo <= tol and es <= tol, (c, eo, es)


@pytest.mark.parametrize("seed", range(8))
def test_varlen_sweep(gdn, oracle_lib, seed):
    import torch
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.integers(1, 9))
    lengths = [int(n) for n in rng.integers(0, 200, size=N)]
    Hk = int(rng.choice([1, 2, 4]))
    Hv = Hk * int(rng.choice([1, 2]))
    chunk = int(rng.choice([32, 64]))
    head_map = int(rng.integers(0, 2))
    x = inputs.generate(N, max(max(lengths), 1), Hk, Hv, 128, "bf16", seed=3100 + seed, init_state="normal",
                        lengths=lengths)
    cat = lambda a: np.concatenate([a[i, :, :n] for i, n in enumerate(lengths)], axis=1)
    bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    o, sf = gdn.prefill_varlen(bf(cat(x.q_bits)), bf(cat(x.k_bits)), bf(cat(x.v_bits)), dev(cat(x.g)),
                               dev(cat(x.beta)), cu, dev(x.s0), chunk=chunk, head_map=head_map, scale=x.scale)
    o_ref, s_ref = oracle_lib.prefill(x.q, x.k, x.v, x.g, x.beta, x.s0, scale=x.scale, head_map=head_map)
    want = np.concatenate([o_ref[i, :, :n] for i, n in enumerate(lengths)], axis=1)
    eo, es = rel_err(o.cpu().numpy(), want), rel_err(sf.cpu().numpy(), s_ref)
    print(f"varlen sweep {seed} lengths {lengths} Hk {Hk} Hv {Hv} C{chunk} map{head_map}: o {eo:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("seed", range(12))
def test_kda_sweep(gdn, oracle_lib, seed):
    rng = np.random.default_rng(4000 + seed)
    B, T = int(rng.integers(1, 3)), int(rng.integers(0, 120 if seed < 6 else 400))
    Hk = int(rng.choice([1, 2]))
    Hv = Hk * int(rng.choice([1, 2]))
    dtype = "bf16" if rng.integers(0, 2) else "f32"
    head_map = int(rng.integers(0, 2))
    x = inputs.generate(B, T, Hk, Hv, 128, dtype, seed=4100 + seed, init_state="normal")
    g = inputs.generate_channel_decay((B, Hv, T, 128), seed=4200 + seed, factor=float(rng.choice([0.1, 1.0, 3.0])))
    q, k, v = qkv_dev(x)
    o, sf = gdn.kda_prefill(q, k, v, dev(g), dev(x.beta), dev(x.s0), head_map=head_map, scale=x.scale)
    o_ref, s_ref = oracle_lib.kda_prefill(x.q, x.k, x.v, g, x.beta, x.s0, scale=x.scale, head_map=head_map)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(sf.cpu().numpy(), s_ref)
    print(f"kda sweep {seed} B{B} T{T} Hk{Hk} Hv{Hv} {dtype} map{head_map}: o {eo:.2e} state {es:.2e}")
    assert eo <= tol and es <= tol
