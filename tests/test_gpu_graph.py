"""HIP graph capture of the entry points: replays of a captured decode sequence and of a
captured prefill give the eager results bit for bit, on every replay (needs an MI355X)."""
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


def test_decode_graph_replay(gdn, oracle_lib):
    """16 in-place decode steps captured in one graph; three replays, each from the initial
    state and with eager work between them, equal the eager steps exactly."""
    import torch
    steps = 16
    x = inputs.generate(8, 1, 2, 4, 128, "bf16", seed=81, init_state="normal", decode_steps=steps)
    q, k, v = qkv_dev(x)
    g, beta = dev(x.g), dev(x.beta)
    s0 = dev(x.s0)
    # eager
    state_e = s0.clone()
    o_e = [gdn.decode(q[s], k[s], v[s], g[s], beta[s], state_e, scale=x.scale) for s in range(steps)]
    torch.cuda.synchronize()
    # captured
    state_g = s0.clone()
    o_g = torch.empty((steps,) + tuple(o_e[0].shape), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for s in range(steps):
                gdn.decode(q[s], k[s], v[s], g[s], beta[s], state_g, scale=x.scale, o=o_g[s])
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        state_g.copy_(s0)
        o_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(o_g[s], o_e[s]), (rep, s)
        assert torch.equal(state_g, state_e), rep
        # eager work between replays
        scratch = s0.clone()
        gdn.decode(q[0], k[0], v[0], g[0], beta[0], scratch, scale=x.scale)
        torch.cuda.synchronize()
    # and the eager steps themselves against the oracle (last step, final state)
    ref_state = np.ascontiguousarray(x.s0.astype(np.float64))
    for s in range(steps):
        o_ref = oracle_lib.decode_step(x.q[s], x.k[s], x.v[s], x.g[s], x.beta[s], ref_state, scale=x.scale)
    assert rel_err(o_e[-1].cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_err(state_e.cpu().numpy(), ref_state) <= TOL_BF16


@pytest.mark.parametrize("T", [300, 2000])
def test_prefill_graph_replay(gdn, T):
    """A captured gdn_prefill (chunk prep + state pass, caller-owned workspace) replayed three
    times equals the eager call exactly."""
    import torch
    x = inputs.generate(1, T, 2, 4, 128, "bf16", seed=82 + T, init_state="normal")
    q, k, v = qkv_dev(x)
    g, beta, s0 = dev(x.g), dev(x.beta), dev(x.s0)
    o_e, sf_e = gdn.prefill(q, k, v, g, beta, s0, chunk=64, scale=x.scale)
    torch.cuda.synchronize()
    ws = gdn.prefill_workspace_bytes(1, T, 2, 4, 128, chunk=64)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    o_g = torch.empty_like(o_e)
    sf_g = torch.empty_like(sf_e)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gdn.prefill(q, k, v, g, beta, s0, chunk=64, scale=x.scale, o=o_g, final_state=sf_g,
                        workspace=workspace)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        o_g.fill_(float("nan"))
        sf_g.fill_(float("nan"))
        workspace.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(sf_g, sf_e), rep
        gdn.prefill(q, k, v, g, beta, None, chunk=64, scale=x.scale, write_final_state=False)
        torch.cuda.synchronize()
