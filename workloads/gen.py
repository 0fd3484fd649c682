"""Seeded synthetic inputs for the Gated DeltaNet (GDN) state-update workloads.

Both sides -- the HIP library and the CPU oracle -- consume the bytes made
here, so they are compared on identical inputs.  This module draws random
numbers, shapes them and stores them in the input dtype; it holds no step of
the state update itself (no gates, no decay, no delta rule, no rounding of
states written by the method).

Host representation of a tensor of each storage dtype:
  * ``"f32"``  -> ``np.float32`` array
  * ``"f16"``  -> ``np.float16`` array
  * ``"bf16"`` -> ``np.uint16`` array holding the raw bfloat16 bit patterns

Distributions (the hybrid-model GDN layer workload, one per tensor):
  * q, k ~ N(0, 1), then L2-normalised over the head dimension (fp32), then
    stored in the input dtype;
  * v, a, b ~ N(0, 1);
  * A_log ~ U(0, ln 16), dt_bias ~ N(0, 1), both float32 per value head;
  * initial states ~ N(0, 0.1^2) drawn in fp32 and stored in the pool dtype.

Every tensor has its own generator ``np.random.default_rng([config, tensor,
index])`` so a single slot, step or sequence can be regenerated alone (the
oracle only needs the sampled ones at full size).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "DTYPES", "TID", "rng", "store", "to_torch", "from_torch", "head_params",
    "token_inputs", "pool_slots", "slot_permutation", "seq_lengths_cu",
    "rejected_counts", "split_lengths", "DecodeShape", "CONFIGS", "WORKLOADS", "m2_params", "m2_inputs", "M2_LAYER",
]

DTYPES = ("f32", "bf16", "f16")

# tensor ids of the per-tensor seeds
TID = dict(q=1, k=2, v=3, a=4, b=5, A_log=6, dt_bias=7, pool=8, slot_perm=9,
           rejected=10, ring=11, prefill=12, counts=13, x=14, Bm=15, Cm=16, dt=17, Dskip=18)


def rng(config_id: int, tensor: str, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(config_id), TID[tensor], int(index)])


def store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 values in ``dtype`` (host representation above).

    bf16 and f16 use PyTorch's CPU casts (round to nearest even); this is a
    library routine used only to produce input bytes.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32
    import torch
    t = torch.from_numpy(x32)
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return t.to(torch.float16).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def to_torch(arr: np.ndarray, device="cpu"):
    """Host array (representation above) -> torch tensor of the same bytes."""
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def from_torch(t) -> np.ndarray:
    """Torch tensor -> host array in the representation above."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _normal(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-12)).astype(np.float32)


def head_params(config_id: int, Hv: int):
    """A_log ~ U(0, ln 16) and dt_bias ~ N(0, 1), float32 [Hv]."""
    A_log = rng(config_id, "A_log").uniform(0.0, math.log(16.0), size=Hv).astype(np.float32)
    dt_bias = _normal(rng(config_id, "dt_bias"), (Hv,))
    return A_log, dt_bias


def token_inputs(config_id: int, step: int, lead: tuple, Hk: int, Hv: int, dk: int, dv: int,
                 in_dtype: str = "bf16", a_shift: float = 0.0) -> dict:
    """Per-token inputs q, k [*lead, Hk, dk], v [*lead, Hv, dv], a, b [*lead, Hv].

    ``lead`` is (B,) for a decode step, (B, T) for a replay window, (T_total,)
    for packed prefill.  ``a_shift`` moves the mean of ``a`` (a negative shift
    gives slow decay, used by the state-carry stress cases).
    """
    lead = tuple(int(x) for x in lead)
    q = _l2n(_normal(rng(config_id, "q", step), lead + (Hk, dk)))
    k = _l2n(_normal(rng(config_id, "k", step), lead + (Hk, dk)))
    v = _normal(rng(config_id, "v", step), lead + (Hv, dv))
    a = _normal(rng(config_id, "a", step), lead + (Hv,)) + np.float32(a_shift)
    b = _normal(rng(config_id, "b", step), lead + (Hv,))
    return {name: store(x, in_dtype) for name, x in
            dict(q=q, k=k, v=v, a=a.astype(np.float32), b=b).items()}


def pool_slots(config_id: int, slots, Hv: int, dk: int, dv: int, dtype: str,
               std: float = 0.1) -> np.ndarray:
    """Initial states of the given slots, N(0, std^2), stored in ``dtype``: [len(slots), Hv, dk, dv]."""
    out = [store(_normal(rng(config_id, "pool", int(s)), (Hv, dk, dv), std), dtype) for s in slots]
    if not out:
        return store(np.zeros((0, Hv, dk, dv), np.float32), dtype)
    return np.stack(out)


def slot_permutation(config_id: int, num_slots: int) -> np.ndarray:
    return rng(config_id, "slot_perm").permutation(num_slots).astype(np.int32)


def seq_lengths_cu(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    return cu


def split_lengths(lengths, frac=0.55):
    """First call gets floor(frac * len) tokens of each sequence, the second the rest."""
    first = [int(math.floor(frac * n)) for n in lengths]
    return first, [n - f for n, f in zip(lengths, first)]


def m2_params(config_id: int, H: int):
    """Mamba2 head parameters, float32 [H]: A_log = log U(1, 16) (A in [-16, -1]); dt_bias the
    inverse softplus of a log-uniform step in [1e-3, 1e-1]; skip D ~ U(0.5, 1.5)."""
    A_log = np.log(rng(config_id, "A_log").uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt0 = np.exp(rng(config_id, "dt_bias").uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dt0)).astype(np.float32)
    Dskip = rng(config_id, "Dskip").uniform(0.5, 1.5, size=H).astype(np.float32)
    return A_log, dt_bias, Dskip


def m2_inputs(config_id: int, step: int, lead: tuple, H: int, G: int, d: int, n: int,
              in_dtype: str = "bf16", dt_shift: float = 0.0) -> dict:
    """Mamba2 per-token inputs: x [*lead, H, d] ~ N(0, 1); Bm, Cm [*lead, G, n] ~ N(0, 1/n);
    dt [*lead, H] ~ N(dt_shift, 0.5^2) (raw, before softplus with dt_bias)."""
    lead = tuple(int(v) for v in lead)
    x = _normal(rng(config_id, "x", step), lead + (H, d))
    Bm = _normal(rng(config_id, "Bm", step), lead + (G, n), n ** -0.5)
    Cm = _normal(rng(config_id, "Cm", step), lead + (G, n), n ** -0.5)
    dt = _normal(rng(config_id, "dt", step), lead + (H,), 0.5) + np.float32(dt_shift)
    return {name: store(v, in_dtype) for name, v in dict(x=x, Bm=Bm, Cm=Cm, dt=dt.astype(np.float32)).items()}


# Mamba2 layer of the ReplaySSM workload: 128 heads of headdim 64, dstate 128, 8 groups
M2_LAYER = dict(H=128, G=8, d=64, n=128)


def rejected_counts(config_id: int, step: int, B: int, max_r: int) -> np.ndarray:
    """Seeded number of rejected draft tokens per sequence, uniform in {0..max_r}."""
    return rng(config_id, "rejected", step).integers(0, max_r + 1, size=B).astype(np.int32)


@dataclass
class DecodeShape:
    B: int
    Hk: int
    Hv: int
    dk: int
    dv: int


@dataclass
class Config:
    cid: int
    name: str
    shape: DecodeShape
    in_dtype: str
    state_dtypes: tuple
    num_slots: int
    steps: int = 1
    extra: dict = field(default_factory=dict)


CONFIGS = {
    # tiny recurrence: 2 sequences, 2 heads, 16x16 state, 8 steps, fp32 everywhere
    0: Config(0, "tiny", DecodeShape(2, 2, 2, 16, 16), "f32", ("f32",), 4, steps=8,
              extra=dict(slot_map=[3, 1])),
    # single-step decode of a hybrid-model GDN layer (16 key heads, 32 value heads, 128x128)
    1: Config(1, "decode_f32", DecodeShape(256, 16, 32, 128, 128), "bf16", ("f32",), 1024, steps=64),
    # same layer with bf16 / fp16 state at B in {1, 64, 256, 512}
    2: Config(2, "decode_lowp", DecodeShape(256, 16, 32, 128, 128), "bf16", ("bf16", "f16"), 1024,
              steps=64, extra=dict(batches=[1, 64, 256, 512])),
    # chunked prefill of 4 packed sequences
    3: Config(3, "prefill", DecodeShape(4, 16, 32, 128, 128), "bf16", ("f32", "bf16"), 16,
              extra=dict(lengths=[1024, 3000, 8192, 8192], chunk=64)),
    # replay decode with a ring of 16 entries, spec window of 1 + 4 drafts
    4: Config(4, "replay", DecodeShape(512, 16, 32, 128, 128), "bf16", ("f32", "bf16"), 1024,
              extra=dict(L=16, T_spec=5)),
}
# the same workloads by name
WORKLOADS = {c.name: c for c in CONFIGS.values()}
