"""GPU parity of gdn_copy_state_blocks against the oracle: bit-exact on every byte.

The tensors mix the three access widths the kernel picks between (16-byte
aligned slots, 4-byte aligned ones, odd byte counts), slot sizes above and
below one 64 KiB chunk, tensors with fewer slots than some job indices, and
padded (negative) jobs.
"""
import numpy as np
import pytest

import oracle as O

from gpu_util import DEV, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bytes(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def _tensors(seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    specs = [((12, 4, 64, 64), torch.float32),   # 64 KiB slots: exactly one chunk, 16-byte path
             ((12, 2, 128, 128), torch.bfloat16),  # 64 KiB slots
             ((9, 3, 100, 101), torch.float32),   # 121200-byte slots: two chunks, 16-byte path
             ((12, 7), torch.int32),              # 28-byte slots: 4-byte path
             ((12, 37), torch.uint8),             # 37-byte slots: byte path
             ((5, 300001), torch.uint8)]          # 300001-byte slots: byte path over five chunks, 5 slots only
    out = []
    for shape, dt in specs:
        x = torch.randint(0, 255, shape, generator=g, dtype=torch.uint8) if dt == torch.uint8 else \
            torch.randn(shape, generator=g).to(dt) if dt.is_floating_point else \
            torch.randint(-2 ** 31, 2 ** 31 - 1, shape, generator=g, dtype=dt)
        out.append(x)
    return out


def test_copy_state_blocks_bit_exact():
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    host = _tensors(3)
    dev_t = [t.to(DEV) for t in host]
    # distinct destinations, no slot both a source and a destination
    src = np.int32([0, 3, 8, 10, -1, 4])
    dst = np.int32([1, 2, 11, 6, 7, 9])
    say(f"copy_state_blocks P={len(dev_t)} n={len(src)}")
    gdn.gdn_copy_state_blocks(dev_t, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    ref = O.copy_state_blocks([_bytes(t).reshape(t.shape[0], -1) for t in host], src, dst)
    for i, (t, r) in enumerate(zip(dev_t, ref)):
        got = _bytes(t).reshape(t.shape[0], -1)
        assert np.array_equal(got, r), f"tensor {i}: {np.argwhere(got != r)[:4].tolist()}"


def test_copy_state_blocks_repeated_and_empty():
    """Two calls in a row (the second with fewer jobs) and an empty call, sharing one prebuilt table."""
    import torch
    import gated_deltanet_state_gdn_amd as gdn
    host = _tensors(5)[:3]
    dev_t = [t.to(DEV) for t in host]
    ref = [_bytes(t).reshape(t.shape[0], -1) for t in host]
    table = gdn.make_state_table(dev_t, DEV)  # reused across the calls
    for src, dst in (([5, 6, 7], [0, 1, 2]), ([3], [4]), ([], [])):
        src, dst = np.int32(src), np.int32(dst)
        say(f"copy_state_blocks n={len(src)}")
        gdn.gdn_copy_state_blocks(dev_t, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), table=table)
        ref = O.copy_state_blocks(ref, src, dst)
    torch.cuda.synchronize()
    for i, (t, r) in enumerate(zip(dev_t, ref)):
        assert np.array_equal(_bytes(t).reshape(t.shape[0], -1), r), f"tensor {i}"
