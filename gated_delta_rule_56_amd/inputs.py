"""Seeded synthetic inputs for the gated delta rule scan.

This module is shared by the oracle side and the HIP side of every parity
test and by the benchmark. It holds no arithmetic of the method itself: it only
draws random numbers, shapes them the way the workloads describe, rounds
q/k/v to bfloat16 where a workload asks for it, and pads ragged batches.

Input recipe (identical for every workload unless stated):

* ``numpy.random.default_rng(seed)``; draw order q, k, v, g_raw, beta_raw, S0.
  The seeded ``default_rng`` idiom is the one the tinygrad GDN unit tests use
  (tinygrad "27b 935/47" compare page, ``test_attention.py`` /
  ``test_llm_quant_cpu.py`` gated-delta tests).
* q, k ~ N(0, 1) with shape [B][Hk][T][d], then L2-normalised per (b, head, t)
  as ``x / sqrt(sum(x*x) + 1e-6)``. That normalisation (epsilon inside the
  square root) is the newer of the two conventions on the same page
  (``_normalize_np`` in ``test_attention.py``; ``gdn_qkv`` test in
  ``test_llm_quant_cpu.py``).
* v ~ N(0, 1) with shape [B][Hv][T][d].
* g = -softplus(N(0, 1)) (optionally times a slow-decay factor), with
  softplus written as ``log1p(exp(-|x|)) + max(x, 0)`` as in
  ``_softplus_np`` of the same test file.
* beta = sigmoid(N(0, 1)).
* S0 = 0, or N(0, 0.1) (standard deviation 0.1) with shape [B][Hv][dv][dk].
* Everything is computed in float64, stored as float32, and, for bfloat16
  workloads, q/k/v are rounded to bfloat16 with round-to-nearest-even. The
  float32 arrays then hold exactly the bfloat16 values, so both sides of a
  parity test see bit-identical inputs.
* Ragged batches: each sequence b has a real length L_b; every position
  t >= L_b is a padded step with q = k = v = 0, g = 0 and beta = 0, the
  padding that the tinygrad commit log for the symbolic-length prefill
  (page "mergable fast RDNA3 Qwen 3.6") states to be an exact no-op of the
  scan.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

QK_NORM_EPS = 1e-6

HEADS_TILED = 0    # head-map codes shared by both sides of a parity test
HEADS_GROUPED = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, precision and the random recipe."""
    name: str
    batch: int
    seq_len: int            # T (padded length for ragged batches); 1 for decode
    num_k_heads: int
    num_v_heads: int
    head_dim: int
    chunk: int              # prefill chunk length C (ignored by decode)
    qkv_dtype: str          # "f32" or "bf16"
    seed: int
    decay_mult: float = 1.0
    init_state: str = "zero"  # "zero" or "normal"
    lengths: Optional[Sequence[int]] = None  # real lengths of a ragged batch
    decode_steps: int = 0   # > 0 marks a decode workload

    @property
    def is_decode(self) -> bool:
        return self.decode_steps > 0

    @property
    def real_tokens(self) -> int:
        if self.lengths is not None:
            return int(sum(self.lengths))
        return self.batch * self.seq_len


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


RAGGED_LENGTHS = (401, 257, 33, 1)

WORKLOADS = {
    # B=1, Hk=Hv=2, T=64, d=32, fp32, chunk 16, zero initial state.
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 2, 2, 32, 16, "f32", seed=1),
    # B=1, Hk=16, Hv=32, T=4096, d=128, bf16 q/k/v, chunk 64, zero state.
    "prefill_4k": Workload("prefill_4k", 1, 4096, 16, 32, 128, 64, "bf16", seed=2),
    # B=4 ragged (401/257/33/1, each padded to a multiple of 32, batch shares
    # the longest padded length), Hk=16, Hv=32, d=128, bf16, S0 ~ N(0, 0.1).
    "ragged_continuation": Workload(
        "ragged_continuation", 4, _round_up(max(RAGGED_LENGTHS), 32), 16, 32, 128, 64, "bf16",
        seed=3, init_state="normal", lengths=RAGGED_LENGTHS),
    # B=1, Hk=16, Hv=32, T=32768, d=128, bf16, chunk 64, g scaled by 0.1.
    "long_prefill_32k": Workload("long_prefill_32k", 1, 32768, 16, 32, 128, 64, "bf16",
                                 seed=4, decay_mult=0.1),
    # B=256 sequences x 1 token, Hk=16, Hv=32, d=128, fp32 state ~ N(0, 0.1),
    # bf16 q/k/v, 64 consecutive in-place steps.
    "batched_decode": Workload("batched_decode", 256, 1, 16, 32, 128, 64, "bf16",
                               seed=5, init_state="normal", decode_steps=64),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(f.shape, dtype=np.uint16)
    step = 1 << 22
    for s in range(0, f.size, step):
        u = f[s:s + step].view(np.uint32).copy()
        lsb = (u >> 16) & 1
        u += 0x7FFF  # finite inputs cannot carry out of 32 bits
        u += lsb
        u >>= 16
        out[s:s + step] = u
    return out.reshape(np.shape(x))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    """x / sqrt(sum(x*x) + eps) over the last axis, in place."""
    norm = np.sqrt(np.einsum("...d,...d->...", x, x) + QK_NORM_EPS)
    x /= norm[..., None]
    return x


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclasses.dataclass
class ScanInputs:
    """Inputs of one prefill call or of a sequence of decode calls.

    Prefill shapes: q, k [B][Hk][T][d]; v [B][Hv][T][d]; g, beta [B][Hv][T];
    s0 [B][Hv][dv][dk] or None.
    Decode shapes carry a leading step axis: q, k [S][B][Hk][d];
    v [S][B][Hv][d]; g, beta [S][B][Hv].
    q/k/v are float32 arrays holding exactly the values both sides consume;
    for bfloat16 workloads the matching bit patterns are in *_bits.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: Optional[np.ndarray]
    scale: float
    qkv_dtype: str
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    lengths: Optional[Sequence[int]] = None


def _store(x64: np.ndarray, qkv_dtype: str):
    f32 = x64.astype(np.float32)
    if qkv_dtype == "bf16":
        bits = bf16_round(f32)
        return bf16_to_f32(bits), bits
    return f32, None


def generate(batch: int, seq_len: int, num_k_heads: int, num_v_heads: int, head_dim: int,
             qkv_dtype: str, seed: int, decay_mult: float = 1.0, init_state: str = "zero",
             lengths: Optional[Sequence[int]] = None, decode_steps: int = 0) -> ScanInputs:
    """Draw one seeded input set (see the module docstring for the recipe)."""
    if qkv_dtype not in ("f32", "bf16"):
        raise ValueError(f"qkv_dtype must be 'f32' or 'bf16', got {qkv_dtype!r}")
    rng = np.random.default_rng(seed)
    d = head_dim
    if decode_steps:
        lead_k = (decode_steps, batch, num_k_heads)
        lead_v = (decode_steps, batch, num_v_heads)
    else:
        lead_k = (batch, num_k_heads, seq_len)
        lead_v = (batch, num_v_heads, seq_len)
    q = _l2_normalise(rng.standard_normal(lead_k + (d,)))
    k = _l2_normalise(rng.standard_normal(lead_k + (d,)))
    v = rng.standard_normal(lead_v + (d,))
    g = -_softplus(rng.standard_normal(lead_v)) * decay_mult
    beta = _sigmoid(rng.standard_normal(lead_v))
    if init_state == "zero":
        s0 = None
    elif init_state == "normal":
        s0 = rng.normal(0.0, 0.1, (batch, num_v_heads, d, d)).astype(np.float32)
    else:
        raise ValueError(f"init_state must be 'zero' or 'normal', got {init_state!r}")

    if lengths is not None:
        if decode_steps:
            raise ValueError("ragged lengths apply to prefill inputs only")
        if len(lengths) != batch or max(lengths) > seq_len or min(lengths) < 0:
            raise ValueError("lengths must give one real length <= seq_len per sequence")
        t = np.arange(seq_len)
        for b, length in enumerate(lengths):
            pad = t >= length
            q[b][:, pad] = 0.0
            k[b][:, pad] = 0.0
            v[b][:, pad] = 0.0
            g[b][:, pad] = 0.0
            beta[b][:, pad] = 0.0

    qf, qb = _store(q, qkv_dtype)
    kf, kb = _store(k, qkv_dtype)
    vf, vb = _store(v, qkv_dtype)
    return ScanInputs(q=qf, k=kf, v=vf, g=g.astype(np.float32), beta=beta.astype(np.float32),
                      s0=s0, scale=1.0 / math.sqrt(d), qkv_dtype=qkv_dtype,
                      q_bits=qb, k_bits=kb, v_bits=vb,
                      lengths=tuple(lengths) if lengths is not None else None)


def generate_workload(wl: Workload) -> ScanInputs:
    """Inputs of a named workload."""
    return generate(wl.batch, wl.seq_len, wl.num_k_heads, wl.num_v_heads, wl.head_dim,
                    wl.qkv_dtype, wl.seed, decay_mult=wl.decay_mult, init_state=wl.init_state,
                    lengths=wl.lengths, decode_steps=wl.decode_steps)



@dataclasses.dataclass
class NormInputs:
    """Inputs of the gated RMSNorm epilogue: gate (float32 values; bf16 bits when the workload
    is bf16) of the output's shape, and weight [dv] float32."""
    gate: np.ndarray
    gate_bits: Optional[np.ndarray]
    weight: np.ndarray


def generate_norm(out_shape: Sequence[int], qkv_dtype: str, seed: int) -> NormInputs:
    """Seeded gate ~ N(0, 1) of the output's shape, stored like q/k/v (bf16-rounded for a bf16
    workload), and a weight ~ N(0, 1) over the head dimension, rounded to float16 values (the
    pages draw their norm weights in float16)."""
    rng = np.random.default_rng(seed)
    gate = rng.standard_normal(tuple(out_shape))
    weight = rng.standard_normal(out_shape[-1]).astype(np.float16).astype(np.float32)
    gf, gb = _store(gate, qkv_dtype)
    return NormInputs(gate=gf, gate_bits=gb, weight=weight)


def generate_channel_decay(shape: Sequence[int], seed: int, factor: float = 1.0) -> np.ndarray:
    """Log-decays for the per-channel-decay variant: one value per key channel,
    g = -softplus(N(0, 1)) * factor (the scalar decay's distribution, drawn per channel),
    computed in float64 and stored as float32. shape: [B][Hv][T][dk] or [steps][B][Hv][dk]."""
    rng = np.random.default_rng(seed)
    return (-_softplus(rng.standard_normal(tuple(shape))) * factor).astype(np.float32)
