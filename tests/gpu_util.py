"""Helpers for the GPU parity tests (HIP library vs the CPU oracle on the same seeded bytes)."""
import sys

import numpy as np
import pytest

import gated_deltanet_state_gdn_amd as gdn
from workloads import gen

DEV = "cuda"

# tolerance per state dtype: elementwise |x - ref| <= atol + rtol |ref|
TOL = {"f32": dict(rtol=1e-4, atol=1e-4), "bf16": dict(rtol=0.0, atol=1e-2), "f16": dict(rtol=0.0, atol=1e-2)}
POISON = {"f32": np.uint32(0x7FC0DEAD), "bf16": np.uint16(0x7FDE), "f16": np.uint16(0x7E5A)}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible GPU")
    gdn.lib()  # raises if the HIP library is missing


def say(*args):
    """Name the case on stdout (flushed) before each GPU step."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev(arr):
    return gen.to_torch(arr, DEV)


def host(t):
    return gen.from_torch(t)


def widen(arr):
    import oracle
    return oracle.widen(arr)


def assert_close(got, ref, dtype, what=""):
    got = widen(got) if not (isinstance(got, np.ndarray) and got.dtype == np.float64) else got
    ref = widen(ref) if not (isinstance(ref, np.ndarray) and ref.dtype == np.float64) else ref
    tol = TOL[dtype]
    err = np.abs(got - ref)
    bound = tol["atol"] + tol["rtol"] * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside atol={tol['atol']} rtol={tol['rtol']}; "
                             f"max err {err.max():.3e}; first {idx.tolist()} got {got[bad][:5]} ref {ref[bad][:5]}")


def poisoned_pool(num_slots, Hv, dk, dv, dtype, slots, cid, std=0.1):
    """Device pool whose listed slots hold the seeded initial states and the rest a poison pattern."""
    import torch
    host_pool = np.empty((num_slots, Hv, dk, dv), {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16}[dtype])
    host_pool[...] = POISON[dtype]
    states = gen.pool_slots(cid, slots, Hv, dk, dv, dtype, std)
    view = states.view(host_pool.dtype)
    for i, s in enumerate(slots):
        host_pool[s] = view[i]
    if dtype == "f32":
        t = torch.from_numpy(host_pool.view(np.float32))
    elif dtype == "bf16":
        t = torch.from_numpy(host_pool.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(host_pool.view(np.float16))
    return t.to(DEV), states


def assert_poison_kept(pool_dev, slots, dtype):
    import torch
    if len(slots) == 0:
        return
    idx = torch.as_tensor(np.asarray(slots, np.int64), device=pool_dev.device)
    sub = host(pool_dev.index_select(0, idx))
    bits = sub.view(np.uint32 if dtype == "f32" else np.uint16)
    assert np.all(bits == POISON[dtype]), f"untouched slots {list(slots)[:4]} were modified"
