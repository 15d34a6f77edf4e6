"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one gdn_prefill over the long-prefill workload (B=1, Hk=16, Hv=32,
T=32768, d=128, bf16 q/k/v, chunk 64) followed by one gdn_decode step over the
batched-decode workload (B=256, Hk=16, Hv=32, d=128, 537 MB fp32 state updated
in place). Inputs are seeded synthetic data of exactly those shapes, resident in
HBM before timing starts. Prints one JSON line; ``value`` is prefill tokens/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for counter scaling)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 matrix peak
PREFILL_WL = "long_prefill_32k"
DECODE_WL = "batched_decode"


def prefill_flops_per_token_head(C: int, d: int) -> float:
    """Algorithmic FLOPs of the chunked WY form per (token, value head):
    10*C*d (five C x C x d products per chunk) + 6*d^2 (three C x d x d products
    per chunk) + 2*C^2/3 (the triangular solve)."""
    return 10.0 * C * d + 6.0 * d * d + 2.0 * C * C / 3.0


def prefill_bytes(B, T, Hk, Hv, d, qkv_bytes=2, init_state=False, o_bytes=4) -> int:
    """Minimum HBM bytes of one prefill launch: q, k, v read once, g, beta read,
    o written (fp32, or fp16 with o_bytes=2), final state written (and the initial state
    read if given)."""
    qk = 2 * B * Hk * T * d * qkv_bytes
    v = B * Hv * T * d * qkv_bytes
    gb = 2 * B * Hv * T * 4
    o = B * Hv * T * d * o_bytes
    st = B * Hv * d * d * 4 * (2 if init_state else 1)
    return qk + v + gb + o + st


def decode_bytes(B, Hk, Hv, d, qkv_bytes=2, state_bytes=4) -> int:
    """Minimum HBM bytes of one decode step: the state read and written (fp32, or fp16
    with state_bytes=2), q, k, v, g, beta read, o written."""
    return 2 * B * Hv * d * d * state_bytes + 2 * B * Hk * d * qkv_bytes + B * Hv * d * qkv_bytes + 2 * B * Hv * 4 \
        + B * Hv * d * 4


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill_long32k_decode_b256_hbm_traffic.md")
# the sources of the benchmarked prefill path: the segmented kernels and the C ABI that picks the
# segment count (the committed counter summaries are only used while these are unchanged)
PREFILL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_56_amd", "csrc", f)
                   for f in ("gdn_prefill_seg.hip", "gdn_frag.h", "gdn_device.h", "gdn_internal.h", "gdn_abi.cpp")]


MFMA_PROFILE = os.path.join(ROOT, "profiles", "prefill_long32k_mfma_counters.md")


def measured_prefill_mfma_flops():
    """MFMA FLOPs per gdn_prefill launch counted by rocprofv3 (SQ_INSTS_VALU_MFMA_MOPS_* x 512)
    from the committed summary, or None when the kernel sources have changed since."""
    try:
        text = open(MFMA_PROFILE).read()
        h = hashlib.sha256()
        for f in PREFILL_SOURCES:
            h.update(open(f, "rb").read())
    except OSError:
        return None
    m_flops = re.search(r"^counted_mfma_flops_per_launch:\s*(\d+)", text, re.M)
    m_sha = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]+)", text, re.M)
    if not (m_flops and m_sha) or h.hexdigest()[:len(m_sha.group(1))] != m_sha.group(1):
        return None
    return int(m_flops.group(1))


def measured_prefill_traffic(key="traffic_bytes_per_launch"):
    """HBM bytes per gdn_prefill launch from the committed FETCH_SIZE / WRITE_SIZE summary
    (key: the fp32-o call, or traffic_bytes_per_launch_f16_o), or None when the kernel sources
    have changed since those counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        h = hashlib.sha256()
        for f in PREFILL_SOURCES:
            h.update(open(f, "rb").read())
    except OSError:
        return None
    m_bytes = re.search(r"^" + key + r":\s*(\d+)", text, re.M)
    m_sha = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]+)", text, re.M)
    if not (m_bytes and m_sha) or h.hexdigest()[:len(m_sha.group(1))] != m_sha.group(1):
        return None
    return int(m_bytes.group(1))


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 floats = 1 GiB read + 1 GiB written
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.add(x, 0.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 3}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(every (sequence, head) chain is independent, so more GPUs would each run this same "
              "single-GPU kernel on their own share)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return

    from gated_delta_rule_56_amd import binding, inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.time()
    pw = inputs.WORKLOADS[PREFILL_WL]
    px = inputs.generate_workload(pw)
    dw = inputs.WORKLOADS[DECODE_WL]
    dx = inputs.generate_workload(dw)
    t_gen = time.time() - t_gen

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- device-resident inputs
    pq, pk, pv = bf(px.q_bits), bf(px.k_bits), bf(px.v_bits)
    pg, pb = torch.from_numpy(px.g).to(dev), torch.from_numpy(px.beta).to(dev)
    B, Hk, T, d = px.q.shape
    Hv = px.v.shape[1]
    po = torch.empty((B, Hv, T, d), dtype=torch.float32, device=dev)
    psf = torch.empty((B, Hv, d, d), dtype=torch.float32, device=dev)
    dq, dk, dv = bf(dx.q_bits), bf(dx.k_bits), bf(dx.v_bits)        # [steps][B][H][d]
    dg, db = torch.from_numpy(dx.g).to(dev), torch.from_numpy(dx.beta).to(dev)
    state = torch.from_numpy(dx.s0).to(dev)
    dB, dHk, dHv, dd = dw.batch, dw.num_k_heads, dw.num_v_heads, dw.head_dim
    do = torch.empty((dB, dHv, dd), dtype=torch.float32, device=dev)
    nsteps_dec = dw.decode_steps

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.prefill(pq, pk, pv, pg, pb, None, chunk=pw.chunk, scale=px.scale, o=po, final_state=psf)
        if ev is not None:
            ev[1].record(stream)
        s = i % nsteps_dec
        binding.decode(dq[s], dk[s], dv[s], dg[s], db[s], state, scale=dx.scale, o=do)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if not (torch.isfinite(po).all() and torch.isfinite(state).all()):
        raise RuntimeError("non-finite outputs after warm-up")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the decode sequence (every pre-generated step, state in place) captured in one HIP graph
    dstate_g = state.clone()
    do_g = torch.empty((nsteps_dec,) + tuple(do.shape), dtype=torch.float32, device=dev)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for s in range(nsteps_dec):
                binding.decode(dq[s], dk[s], dv[s], dg[s], db[s], dstate_g, scale=dx.scale, o=do_g[s])
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(1, args.steps // 10))]
    for e in gev:
        e[0].record(stream)
        graph.replay()
        e[1].record(stream)
    torch.cuda.synchronize()
    dgraph_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gev])) / nsteps_dec
    if not torch.isfinite(dstate_g).all():
        raise RuntimeError("non-finite state after the captured decode sequence")
    del graph, dstate_g, do_g

    def time_batch(fn, n):
        """Mean duration of n back-to-back launches, from one pair of HIP events on the launch
        stream around all of them (per-launch event pairs add their own overhead to kernels
        of a fraction of a millisecond)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # decode on a float16 copy of the state (float32 arithmetic, the state stored in float16)
    dstate16 = state.half()
    for s in range(max(1, args.warmup)):
        binding.decode(dq[s], dk[s], dv[s], dg[s], db[s], dstate16, scale=dx.scale, o=do)
    d16_ms = time_batch(lambda i: binding.decode(dq[i % nsteps_dec], dk[i % nsteps_dec], dv[i % nsteps_dec],
                                                 dg[i % nsteps_dec], db[i % nsteps_dec], dstate16,
                                                 scale=dx.scale, o=do), args.steps)
    d16_bytes = decode_bytes(dB, dHk, dHv, dd, state_bytes=2)
    if not torch.isfinite(dstate16).all():
        raise RuntimeError("non-finite float16 state")
    del dstate16

    # the same on a bfloat16 copy (float32 arithmetic, the state stored in bfloat16)
    dstatebf = state.to(torch.bfloat16)
    for s in range(max(1, args.warmup)):
        binding.decode(dq[s], dk[s], dv[s], dg[s], db[s], dstatebf, scale=dx.scale, o=do)
    dbf_ms = time_batch(lambda i: binding.decode(dq[i % nsteps_dec], dk[i % nsteps_dec], dv[i % nsteps_dec],
                                                 dg[i % nsteps_dec], db[i % nsteps_dec], dstatebf,
                                                 scale=dx.scale, o=do), args.steps)
    if not torch.isfinite(dstatebf.float()).all():
        raise RuntimeError("non-finite bfloat16 state")
    del dstatebf

    # one sequence (B = 1): a step moves 4.2 MB, so launch overhead decides; the decode sequence
    # back to back as eager calls, and captured in one HIP graph
    s1 = state[:1].clone()
    o1 = torch.empty((1, dHv, dd), dtype=torch.float32, device=dev)

    def one(s):
        binding.decode(dq[s][:1], dk[s][:1], dv[s][:1], dg[s][:1], db[s][:1], s1, scale=dx.scale, o=o1)

    for s in range(max(1, args.warmup)):
        one(s)
    torch.cuda.synchronize()
    b1_eager_ms = time_batch(lambda i: one(i % nsteps_dec), nsteps_dec)
    g1 = torch.cuda.CUDAGraph()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g1, stream=side):
            for s in range(nsteps_dec):
                one(s)
    stream.wait_stream(side)
    g1.replay()
    torch.cuda.synchronize()
    b1_graph_ms = time_batch(lambda i: g1.replay(), 4) / nsteps_dec
    if not torch.isfinite(s1).all():
        raise RuntimeError("non-finite state after the single-sequence decode")
    b1_bytes = decode_bytes(1, dHk, dHv, dd)
    del g1, s1, o1

    # the same prefill writing float16 o, and the epilogue on those rows (generated below)
    po16 = torch.empty(po.shape, dtype=torch.float16, device=dev)
    for _ in range(max(1, args.warmup)):
        binding.prefill(pq, pk, pv, pg, pb, None, chunk=pw.chunk, scale=px.scale, o=po16, final_state=psf)
    p16_ms = time_batch(lambda i: binding.prefill(pq, pk, pv, pg, pb, None, chunk=pw.chunk, scale=px.scale,
                                                  o=po16, final_state=psf), args.steps)
    p16_bytes = prefill_bytes(B, T, Hk, Hv, d, o_bytes=2)

    # the same prefill at the other chunk lengths (the segmented passes at C = 32 and C = 16)
    chunk_ms = {}
    for ch in (32, 16):
        binding.prefill(pq, pk, pv, pg, pb, None, chunk=ch, scale=px.scale, o=po, final_state=psf)
        chunk_ms[ch] = time_batch(lambda i: binding.prefill(pq, pk, pv, pg, pb, None, chunk=ch, scale=px.scale,
                                                            o=po, final_state=psf), max(1, args.steps // 4))

    # the per-channel-decay variant: the long prefill (the chunked form, 32-token chunks in the
    # segmented passes; and token by token, chunk 16) and the batched decode step, with one
    # log-decay per key channel (-softplus(N(0,1)) * 0.1 and * 1)
    kg = torch.from_numpy(inputs.generate_channel_decay((B, Hv, T, d), seed=pw.seed + 300, factor=0.1)).to(dev)
    kws = torch.empty(binding.prefill_workspace_bytes(B, T, Hk, Hv, d, chunk=32), dtype=torch.uint8, device=dev)
    for _ in range(max(1, args.warmup)):
        binding.kda_prefill(pq, pk, pv, kg, pb, None, chunk=32, scale=px.scale, o=po, final_state=psf, workspace=kws)
    kda_p_ms = time_batch(lambda i: binding.kda_prefill(pq, pk, pv, kg, pb, None, chunk=32, scale=px.scale, o=po,
                                                        final_state=psf, workspace=kws), args.steps)
    kda_segments = binding.prefill_segments(B, T, Hk, Hv, d, kws.numel(), chunk=32)
    binding.kda_prefill(pq, pk, pv, kg, pb, None, chunk=16, scale=px.scale, o=po, final_state=psf)
    kda_tok_ms = time_batch(lambda i: binding.kda_prefill(pq, pk, pv, kg, pb, None, chunk=16, scale=px.scale, o=po,
                                                          final_state=psf), max(1, args.steps // 10))
    kda_p_bytes = prefill_bytes(B, T, Hk, Hv, d) + B * Hv * T * d * 4  # + the per-channel decays
    del kg, kws
    kdg = torch.from_numpy(inputs.generate_channel_decay((dB, dHv, dd), seed=dw.seed + 300)).to(dev)
    kstate = state.clone()
    binding.kda_decode(dq[0], dk[0], dv[0], kdg, db[0], kstate, scale=dx.scale, o=do)
    kda_d_ms = time_batch(lambda i: binding.kda_decode(dq[i % nsteps_dec], dk[i % nsteps_dec], dv[i % nsteps_dec],
                                                       kdg, db[i % nsteps_dec], kstate, scale=dx.scale, o=do),
                          args.steps)
    kda_d_bytes = decode_bytes(dB, dHk, dHv, dd) + dB * dHv * dd * 4
    del kdg, kstate

    # the gated RMSNorm epilogue on the prefill output (1M rows of 128 floats, bf16 gate)
    nrm = inputs.generate_norm(po.shape, "bf16", seed=pw.seed + 100)
    ngate = bf(nrm.gate_bits)
    nweight = torch.from_numpy(nrm.weight).to(dev)
    for _ in range(max(1, args.warmup)):
        binding.gated_rmsnorm(po, nweight, ngate)
    norm_ms = time_batch(lambda i: binding.gated_rmsnorm(po, nweight, ngate), args.steps)
    norm_bytes = po.numel() * (4 + 4 + 2) + nweight.numel() * 4
    for _ in range(max(1, args.warmup)):
        binding.gated_rmsnorm(po16, nweight, ngate)
    norm16_ms = time_batch(lambda i: binding.gated_rmsnorm(po16, nweight, ngate), args.steps)
    norm16_bytes = po16.numel() * (2 + 2 + 2) + nweight.numel() * 4
    if not torch.isfinite(po16).all():
        raise RuntimeError("non-finite float16 outputs after the gated RMSNorm")
    del po16
    # the same norm as an argument of the calls: fused into the segmented prefill's o store and
    # into the decode update (B * Hv >= 256 pairs)
    for _ in range(max(1, args.warmup)):
        binding.prefill(pq, pk, pv, pg, pb, None, chunk=pw.chunk, scale=px.scale, o=po, final_state=psf,
                        norm_weight=nweight, norm_gate=ngate)
    pnorm_ms = time_batch(lambda i: binding.prefill(pq, pk, pv, pg, pb, None, chunk=pw.chunk, scale=px.scale, o=po,
                                                    final_state=psf, norm_weight=nweight, norm_gate=ngate), args.steps)
    dnrm = inputs.generate_norm(do.shape, "bf16", seed=dw.seed + 100)
    dgate, dweight = bf(dnrm.gate_bits), torch.from_numpy(dnrm.weight).to(dev)
    dnstate = state.clone()
    binding.decode(dq[0], dk[0], dv[0], dg[0], db[0], dnstate, scale=dx.scale, o=do, norm_weight=dweight,
                   norm_gate=dgate)
    dnorm_ms = time_batch(lambda i: binding.decode(dq[i % nsteps_dec], dk[i % nsteps_dec], dv[i % nsteps_dec],
                                                   dg[i % nsteps_dec], db[i % nsteps_dec], dnstate, scale=dx.scale,
                                                   o=do, norm_weight=dweight, norm_gate=dgate), args.steps)
    del dnstate
    if not torch.isfinite(po).all():
        raise RuntimeError("non-finite outputs after the gated RMSNorm")

    # the input prologue (conv + SiLU, q/k/v split, q/k L2 norm) on the long workload's raw
    # projections: x [1][32768][(2 Hk + Hv) d] bf16
    prng = np.random.default_rng(pw.seed + 200)
    Cx = (2 * Hk + Hv) * d
    px_bits = inputs.bf16_round(prng.standard_normal((B, T, Cx), dtype=np.float32))
    xr = bf(px_bits)
    del px_bits
    cw = torch.from_numpy((prng.standard_normal((Cx, 4)) * 0.5).astype(np.float32)).to(dev)
    cst = torch.zeros((B, 3, Cx), dtype=torch.float32, device=dev)
    for _ in range(max(1, args.warmup)):
        pro = binding.qkv_prologue(xr, cw, cst, num_k_heads=Hk, num_v_heads=Hv, head_dim=d)
    del pro
    pqkv = [torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv)]
    lib = binding.load_library()
    pshape = binding.make_shape(B, T, Hk, Hv, d, 0, binding.GDN_DTYPE_BF16, 0, 1.0)

    def prologue_call(_):
        rc = lib.gdn_qkv_prologue(ctypes.byref(pshape), xr.data_ptr(), cw.data_ptr(), cst.data_ptr(),
                                  pqkv[0].data_ptr(), pqkv[1].data_ptr(), pqkv[2].data_ptr(),
                                  ctypes.c_float(1e-6), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    pro_ms = time_batch(prologue_call, args.steps)
    pro_bytes = xr.numel() * 2 + sum(t.numel() for t in pqkv) * 2 + cw.numel() * 4 + 2 * cst.numel() * 4
    del xr, pqkv

    prefill_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    decode_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    ms_per_step = wall * 1e3 / args.steps
    p_avg, d_avg = float(prefill_ms.mean()), float(decode_ms.mean())

    tokens = B * T
    value = tokens / (p_avg * 1e-3)
    flops = prefill_flops_per_token_head(pw.chunk, d) * tokens * Hv
    p_bytes = prefill_bytes(B, T, Hk, Hv, d)
    d_bytes = decode_bytes(dB, dHk, dHv, dd)
    p_gbps = p_bytes / (p_avg * 1e-3) / 1e9
    d_gbps = d_bytes / (d_avg * 1e-3) / 1e9
    p_tflops = flops / (p_avg * 1e-3) / 1e12
    counted_flops = measured_prefill_mfma_flops()  # rocprofv3 MFMA op counters, when current
    segments = binding.prefill_segments(B, T, Hk, Hv, d, binding.prefill_workspace_bytes(B, T, Hk, Hv, d, chunk=pw.chunk),
                                        chunk=pw.chunk)
    # map pass: one 12-wave workgroup per (pair, segment) but the last, at 32-token chunks
    map_wgs = B * Hv * (segments - 1)

    result = {
        "metric": "GDN prefill tokens/s (Hv=32,d=128,T=32k) + MFMA util; decode HBM GB/s",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workloads)",
        "config": {
            "workload": f"{PREFILL_WL} prefill (B={B}, Hk={Hk}, Hv={Hv}, T={T}, d={d}, chunk={pw.chunk}) + "
                        f"{DECODE_WL} step (B={dB}, Hk={dHk}, Hv={dHv}, d={dd}, fp32 state in place)",
            "prefill": {"batch": B, "seq_len": T, "num_k_heads": Hk, "num_v_heads": Hv, "head_dim": d,
                        "chunk": pw.chunk, "qkv_dtype": "bf16", "o_dtype": "f32", "segments": segments},
            "decode": {"batch": dB, "num_k_heads": dHk, "num_v_heads": dHv, "head_dim": dd,
                       "state_bytes": dB * dHv * dd * dd * 4},
        },
        "roofline": {
            "kernel": (f"gdn_prefill call, {segments} segments: gdn_seg_pass_kernel<32, false> (map pass, "
                       f"{map_wgs} workgroups) + gdn_seg_combine_kernel + gdn_seg_pass_kernel<64, true> "
                       f"(output pass, {B * Hv * segments} workgroups)"),
            "bound": "mfma",
            "achieved": p_tflops,
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": p_tflops / MFMA_PEAK_TFLOPS,
            "traffic": measured_prefill_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flops_per_launch": flops,
            "counted_mfma_flops_per_launch": counted_flops,
            "avg_launch_ms": p_avg,
            "hbm": {
                "achieved": p_gbps,
                "peak": HBM_PEAK_GBPS,
                "unit": "GB/s",
                "frac": p_gbps / HBM_PEAK_GBPS,
                "algorithmic_bytes_per_launch": p_bytes,
            },
        },
        "decode": {
            "kernel": "gdn_decode_kernel<128, bf16>",
            "avg_launch_ms": d_avg,
            "achieved": d_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": d_gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": d_bytes,
            "sequence_updates_per_s": dB / (d_avg * 1e-3),
            "head_state_updates_per_s": dB * dHv / (d_avg * 1e-3),
            "f16_state": {
                "what": "the same step with the state stored in float16 (268 MB), float32 arithmetic",
                "kernel": "gdn_decode_kernel<128, bf16, f16 state>",
                "avg_launch_ms": d16_ms,
                "achieved": d16_bytes / (d16_ms * 1e-3) / 1e9,
                "frac": d16_bytes / (d16_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "algorithmic_bytes_per_launch": d16_bytes,
                "sequence_updates_per_s": dB / (d16_ms * 1e-3),
            },
            "bf16_state": {
                "what": "the same step with the state stored in bfloat16 (268 MB), float32 arithmetic",
                "kernel": "gdn_decode_kernel<128, bf16, bf16 state>",
                "avg_launch_ms": dbf_ms,
                "achieved": d16_bytes / (dbf_ms * 1e-3) / 1e9,
                "frac": d16_bytes / (dbf_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "algorithmic_bytes_per_launch": d16_bytes,
                "sequence_updates_per_s": dB / (dbf_ms * 1e-3),
            },
            "single_sequence": {
                "what": f"B = 1, {nsteps_dec} consecutive in-place steps, per step: eager calls back to back, "
                        "and the same steps captured in one HIP graph",
                "eager_step_us": b1_eager_ms * 1e3,
                "graph_step_us": b1_graph_ms * 1e3,
                "algorithmic_bytes_per_step": b1_bytes,
                "graph_achieved": b1_bytes / (b1_graph_ms * 1e-3) / 1e9,
            },
            "graph": {
                "what": f"{nsteps_dec} consecutive in-place steps captured in one HIP graph, per step",
                "avg_step_ms": dgraph_ms,
                "achieved": d_bytes / (dgraph_ms * 1e-3) / 1e9,
                "frac": d_bytes / (dgraph_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "sequence_updates_per_s": dB / (dgraph_ms * 1e-3),
            },
        },
        "prefill_f16_o": {
            "what": "the same prefill call writing o in float16 (half the o bytes)",
            "avg_launch_ms": p16_ms,
            "tokens_per_s": tokens / (p16_ms * 1e-3),
            "achieved": p16_bytes / (p16_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": p16_bytes / (p16_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": p16_bytes,
            "traffic": measured_prefill_traffic("traffic_bytes_per_launch_f16_o"),
        },
        "prefill_chunk_lengths": {
            "what": "the same prefill call (float32 o) at chunk 32 and chunk 16",
            "avg_launch_ms": {str(ch): ms for ch, ms in chunk_ms.items()},
            "tokens_per_s": {str(ch): tokens / (ms * 1e-3) for ch, ms in chunk_ms.items()},
        },
        "kda": {
            "what": "per-channel decay (one log-decay per key channel): long prefill, chunked form "
                    "(32-token chunks, segmented passes), and token by token; batched decode step",
            "prefill_kernel": "gdn_seg_pass_kernel<32, map / output, per-channel decay> + gdn_seg_combine_kernel",
            "prefill_segments": kda_segments,
            "prefill_token_by_token_ms": kda_tok_ms,
            "prefill_ms": kda_p_ms,
            "prefill_tokens_per_s": tokens / (kda_p_ms * 1e-3),
            "prefill_achieved": kda_p_bytes / (kda_p_ms * 1e-3) / 1e9,
            "prefill_frac": kda_p_bytes / (kda_p_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "prefill_algorithmic_bytes": kda_p_bytes,
            "prefill_traffic": measured_prefill_traffic("traffic_bytes_per_launch_kda"),
            "decode_kernel": "gdn_decode_kernel<128, bf16, f32 state, per-channel decay>",
            "decode_ms": kda_d_ms,
            "decode_achieved": kda_d_bytes / (kda_d_ms * 1e-3) / 1e9,
            "decode_frac": kda_d_bytes / (kda_d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "decode_algorithmic_bytes": kda_d_bytes,
            "unit": "GB/s",
            "peak": HBM_PEAK_GBPS,
        },
        "gated_rmsnorm": {
            "kernel": "gdn_gated_rmsnorm_kernel<128, bf16 gate> on the prefill output (separate pass)",
            "avg_launch_ms": norm_ms,
            "achieved": norm_bytes / (norm_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": norm_bytes / (norm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": norm_bytes,
            "rows": po.numel() // po.shape[-1],
            "f16_o": {
                "avg_launch_ms": norm16_ms,
                "achieved": norm16_bytes / (norm16_ms * 1e-3) / 1e9,
                "frac": norm16_bytes / (norm16_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "algorithmic_bytes_per_launch": norm16_bytes,
            },
            "fused": {
                "what": "the norm as an argument of the calls: gdn_prefill (long workload, fused into the "
                        "segmented o store) and gdn_decode (B = 256, fused into the update)",
                "prefill_ms": pnorm_ms,
                "prefill_ms_without_norm": p_avg,
                "prefill_then_separate_norm_ms": p_avg + norm_ms,
                "decode_ms": dnorm_ms,
                "decode_ms_without_norm": d_avg,
            },
        },
        "qkv_prologue": {
            "kernel": "gdn_qkv_prologue_kernel<128, bf16> (conv + SiLU, q/k/v split, q/k L2 norm)",
            "shape": f"x [{B}][{T}][{Cx}] bf16 -> q, k [{B}][{Hk}][{T}][{d}], v [{B}][{Hv}][{T}][{d}]",
            "avg_launch_ms": pro_ms,
            "achieved": pro_bytes / (pro_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": pro_bytes / (pro_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": pro_bytes,
        },
        "input_generation_s": t_gen,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(px, dx)
    print(json.dumps(result))


def cpu_baseline(px, dx):
    """The float64 oracle on the host cores over the same prefill inputs."""
    import oracle
    orc = oracle.load()
    threads = len(os.sched_getaffinity(0))
    B, Hk, T, d = px.q.shape
    Hv = px.v.shape[1]
    # sample: the whole prefill workload, every value head over all T tokens (the oracle is
    # sequential per head, parallel over the B * Hv heads)
    T_s = T
    q, k = px.q[:, :, :T_s], px.k[:, :, :T_s]
    v, g, beta = px.v[:, :, :T_s], px.g[:, :, :T_s], px.beta[:, :, :T_s]
    t = time.perf_counter()
    orc.prefill(q, k, v, g, beta, None, scale=px.scale, threads=threads)
    dt = time.perf_counter() - t
    # decode: one step of all 8192 (b, h) pairs
    st = np.ascontiguousarray(dx.s0.astype(np.float64))
    t = time.perf_counter()
    orc.decode_step(dx.q[0], dx.k[0], dx.v[0], dx.g[0], dx.beta[0], st, scale=dx.scale, threads=threads)
    ddt = time.perf_counter() - t
    return {
        "value": B * T_s / dt,
        "unit": "tokens/s",
        "cores": min(threads, B * Hv),
        "kind": "oracle",
        "sample": f"the whole prefill workload: all {B * Hv} value heads over {T_s} of {T} tokens "
                  f"({dt:.2f} s); float64 sequential recurrence, OpenMP over (b, h) pairs",
        "host_threads_available": threads,
        "decode_sequence_updates_per_s": dx.s0.shape[0] / ddt,
        "decode_sample": f"one step of all {dx.s0.shape[0] * dx.s0.shape[1]} (b, h) pairs ({ddt:.2f} s)",
    }


if __name__ == "__main__":
    main()
