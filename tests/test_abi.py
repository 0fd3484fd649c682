"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/gdn.h declares, and rejects invalid arguments synchronously on the
host (no kernel is launched in any case here: every call either fails
validation or is a B = 0 / N = 0 no-op).  Fake device pointers are plain
integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_state_gdn_amd as gdn
from gated_deltanet_state_gdn_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bd.LIB_PATH):
        from gated_deltanet_state_gdn_amd import build
        build.build()
    return gdn.lib()


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(bd.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s(gdn_\w+)$", out.stdout, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    for code in (gdn.GDN_OK, gdn.GDN_EINVAL, gdn.GDN_EUNSUPPORTED, gdn.GDN_ELAUNCH):
        s = gdn.gdn_status_string(code)
        assert s.startswith("GDN_")
    assert "unknown" in gdn.gdn_status_string(99)


def _dims(Hk=16, Hv=32, dk=128, dv=128):
    return bd.gdn_dims(Hk, Hv, dk, dv, 0.0)


def _gates(a=FAKE, b=FAKE, A=FAKE, dt=FAKE):
    return bd.gdn_gates(a, b, A, dt)


def _pool(base=FAKE, dtype=gdn.GDN_F32, n=8):
    return bd.gdn_pool(base, dtype, n)


def _decode(L, dims=None, B=4, q=FAKE, k=FAKE, v=FAKE, in_dt=gdn.GDN_BF16, gates=None, pool=None, slot_map=FAKE,
            out=FAKE, out_dt=gdn.GDN_F32):
    dims = _dims() if dims is None else dims
    gates = _gates() if gates is None else gates
    pool = _pool() if pool is None else pool
    dp = ctypes.byref(dims) if dims is not False else None
    return L.gdn_decode_step(dp, B, q, k, v, in_dt, ctypes.byref(gates), ctypes.byref(pool), slot_map, out, out_dt,
                             None)


@pytest.mark.parametrize("case,expect", [
    (dict(dims=False), gdn.GDN_EINVAL),
    (dict(dims=bd.gdn_dims(0, 32, 128, 128, 0.0)), gdn.GDN_EINVAL),
    (dict(dims=bd.gdn_dims(3, 32, 128, 128, 0.0)), gdn.GDN_EINVAL),          # Hv % Hk
    (dict(dims=bd.gdn_dims(16, 32, 96, 96, 0.0)), gdn.GDN_EUNSUPPORTED),     # head dim
    (dict(dims=bd.gdn_dims(16, 32, 128, 64, 0.0)), gdn.GDN_EUNSUPPORTED),    # dk != dv
    (dict(B=-1), gdn.GDN_EINVAL),
    (dict(q=None), gdn.GDN_EINVAL),
    (dict(out=None), gdn.GDN_EINVAL),
    (dict(q=FAKE + 1), gdn.GDN_EINVAL),                                       # misaligned bf16
    (dict(k=FAKE + 8), gdn.GDN_EINVAL),                                       # not 16-byte aligned
    (dict(out=FAKE + 2), gdn.GDN_EINVAL),                                     # misaligned f32 out
    (dict(in_dt=7), gdn.GDN_EINVAL),
    (dict(out_dt=-1), gdn.GDN_EINVAL),
    (dict(gates=bd.gdn_gates(FAKE, None, FAKE, FAKE)), gdn.GDN_EINVAL),
    (dict(pool=bd.gdn_pool(FAKE + 8, gdn.GDN_F32, 8)), gdn.GDN_EINVAL),      # pool not 16-B aligned
    (dict(pool=bd.gdn_pool(FAKE, 5, 8)), gdn.GDN_EINVAL),
    (dict(pool=bd.gdn_pool(FAKE, gdn.GDN_F32, 0)), gdn.GDN_EINVAL),
    (dict(pool=bd.gdn_pool(None, gdn.GDN_F32, 8)), gdn.GDN_EINVAL),
    (dict(slot_map=None), gdn.GDN_EINVAL),
    (dict(B=0), gdn.GDN_OK),                                                  # no-op, nothing launched
])
def test_decode_validation(L, case, expect):
    st = _decode(L, **case)
    assert st == expect, gdn.gdn_last_error()
    if expect != gdn.GDN_OK:
        assert gdn.gdn_last_error() != ""
    else:
        assert gdn.gdn_last_error() == ""


def _spec(L, B=4, T=5, dims=None, src=FAKE, dst=FAKE, pool=None):
    dims = _dims() if dims is None else dims
    pool = _pool() if pool is None else pool
    return L.gdn_spec_decode(ctypes.byref(dims), B, T, FAKE, FAKE, FAKE, gdn.GDN_BF16, ctypes.byref(_gates()),
                             ctypes.byref(pool), src, dst, FAKE, gdn.GDN_F32, None)


@pytest.mark.parametrize("case,expect", [
    (dict(T=0), gdn.GDN_EINVAL),
    (dict(B=-2), gdn.GDN_EINVAL),
    (dict(T=32), gdn.GDN_EUNSUPPORTED),                             # 48 KiB staging budget at dk = 128
    (dict(T=31, B=0), gdn.GDN_OK),                                  # fits; B = 0 keeps it a no-op
    (dict(T=64, dims=bd.gdn_dims(2, 2, 32, 32, 0.0), B=0), gdn.GDN_OK),
    (dict(src=None), gdn.GDN_EINVAL),
    (dict(dst=None), gdn.GDN_EINVAL),
    (dict(dst=FAKE + 2), gdn.GDN_EINVAL),
    (dict(pool=bd.gdn_pool(FAKE + 4, gdn.GDN_F32, 8)), gdn.GDN_EINVAL),
    (dict(dims=bd.gdn_dims(16, 32, 128, 64, 0.0)), gdn.GDN_EUNSUPPORTED),
])
def test_spec_validation(L, case, expect):
    st = _spec(L, **case)
    assert st == expect, gdn.gdn_last_error()


def _ring(L_=16, n=8, dtype=gdn.GDN_BF16, k=FAKE, count=FAKE):
    return bd.gdn_ring(k, FAKE, FAKE, FAKE, FAKE, count, n, L_, dtype)


def _replay(L, B=4, T=1, ring=None, pool=None, dims=None, in_dt=gdn.GDN_BF16, ws=FAKE, wsb=1 << 30):
    ring = _ring() if ring is None else ring
    pool = _pool() if pool is None else pool
    dims = _dims() if dims is None else dims
    return L.gdn_replay_decode(ctypes.byref(dims), B, T, FAKE, FAKE, FAKE, in_dt, ctypes.byref(_gates()),
                               ctypes.byref(pool), FAKE, ctypes.byref(ring), FAKE, gdn.GDN_F32, ws, wsb, None)


@pytest.mark.parametrize("case,expect", [
    (dict(T=0), gdn.GDN_EINVAL),
    (dict(T=17), gdn.GDN_EINVAL),                                   # T > L
    (dict(ring=_ring(L_=0)), gdn.GDN_EINVAL),
    (dict(ring=_ring(L_=65)), gdn.GDN_EUNSUPPORTED),
    (dict(ring=_ring(L_=64)), gdn.GDN_EUNSUPPORTED),                # LDS staging budget at dk = 128
    (dict(ring=_ring(L_=16), T=16), gdn.GDN_OK),                    # fits; B = 0 below keeps it a no-op
    (dict(ring=_ring(dtype=gdn.GDN_F16)), gdn.GDN_EINVAL),          # ring dtype != in_dtype
    (dict(ring=_ring(n=7)), gdn.GDN_EINVAL),                        # ring slots != pool slots
    (dict(ring=_ring(k=None)), gdn.GDN_EINVAL),
    (dict(ring=_ring(count=FAKE + 2)), gdn.GDN_EINVAL),
    (dict(ws=None), gdn.GDN_EINVAL),
    (dict(ws=FAKE + 16), gdn.GDN_EINVAL),                           # 256-byte alignment
    (dict(wsb=4 * 32 * 1 * 2 * 128 * 4 - 1), gdn.GDN_EINVAL),       # B * Hv * T * 2 * dv floats needed
])
def test_replay_validation(L, case, expect):
    if expect == gdn.GDN_OK:
        case = dict(case, B=0)
    st = _replay(L, **case)
    assert st == expect, gdn.gdn_last_error()


def test_replay_flush_and_rollback_validation(L):
    dims = _dims()
    st = L.gdn_replay_flush(ctypes.byref(dims), 4, ctypes.byref(_pool()), FAKE, ctypes.byref(_ring(n=9)), None)
    assert st == gdn.GDN_EINVAL
    st = L.gdn_replay_flush(ctypes.byref(dims), 0, ctypes.byref(_pool()), FAKE, ctypes.byref(_ring()), None)
    assert st == gdn.GDN_OK
    st = L.gdn_replay_rollback(ctypes.byref(dims), 4, FAKE, None, ctypes.byref(_ring()), None)
    assert st == gdn.GDN_EINVAL
    st = L.gdn_replay_rollback(ctypes.byref(dims), 0, FAKE, FAKE, ctypes.byref(_ring()), None)
    assert st == gdn.GDN_OK


def test_prefill_validation_and_workspace(L):
    dims = _dims()
    need = L.gdn_chunk_prefill_workspace_bytes(ctypes.byref(dims), 4, 20408, 64)
    # (N + ceil(T / 64)) chunk slots x Hv x (2 * 64 * 64 + 4 * 64) floats
    assert need == (4 + 319) * 32 * (2 * 64 * 64 + 256) * 4
    assert L.gdn_chunk_prefill_workspace_bytes(ctypes.byref(dims), 4, 20408, 48) == 0
    # chunks of 32: (N + ceil(T / 32)) chunk slots x Hv x (2 * 32 * 32 + 4 * 32) floats
    assert L.gdn_chunk_prefill_workspace_bytes(ctypes.byref(dims), 4, 20408, 32) == (4 + 638) * 32 * 2176 * 4

    def call(N=4, T=20408, chunk=64, ws=FAKE, wsb=need, cu=FAKE):
        return L.gdn_chunk_prefill(ctypes.byref(dims), N, cu, T, chunk, FAKE, FAKE, FAKE, gdn.GDN_BF16,
                                   ctypes.byref(_gates()), ctypes.byref(_pool()), FAKE, FAKE, gdn.GDN_F32, ws, wsb,
                                   None)
    assert call(chunk=48) == gdn.GDN_EUNSUPPORTED
    assert call(chunk=128) == gdn.GDN_EUNSUPPORTED
    assert call(wsb=need - 1) == gdn.GDN_EINVAL
    assert call(ws=None) == gdn.GDN_EINVAL
    assert call(ws=FAKE + 64) == gdn.GDN_EINVAL      # 256-byte alignment
    assert call(cu=None) == gdn.GDN_EINVAL
    assert call(T=-1) == gdn.GDN_EINVAL
    assert call(N=-1) == gdn.GDN_EINVAL
    assert call(N=0) == gdn.GDN_OK
    assert call(T=0, wsb=0, ws=None) == gdn.GDN_OK


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        bd.lib()


def test_state_refs_keep_every_address_bit():
    """Addresses at and above 2^63 pack as unsigned 64-bit values, bit for bit."""
    import struct
    addrs = [0, (1 << 63) - 8, 1 << 63, (1 << 64) - 8]
    raw = gdn.state_refs_bytes([(a, 2 << 20, 1024) for a in addrs])
    assert len(raw) == 24 * len(addrs) == len(addrs) * ctypes.sizeof(bd.gdn_state_ref)
    for i, a in enumerate(addrs):
        assert struct.unpack_from("<QQQ", raw, 24 * i) == (a, 2 << 20, 1024)


@pytest.mark.parametrize("case,expect", [
    (dict(P=-1), gdn.GDN_EINVAL),
    (dict(P=65536), gdn.GDN_EINVAL),
    (dict(n=-1), gdn.GDN_EINVAL),
    (dict(refs=None), gdn.GDN_EINVAL),
    (dict(refs=FAKE + 4), gdn.GDN_EINVAL),
    (dict(src=None), gdn.GDN_EINVAL),
    (dict(dst=FAKE + 1), gdn.GDN_EINVAL),
    (dict(max_bytes=0), gdn.GDN_EINVAL),
    (dict(max_bytes=(1 << 31) * 65536 + 1), gdn.GDN_EINVAL),
    (dict(n=0), gdn.GDN_OK),
    (dict(P=0), gdn.GDN_OK),
])
def test_copy_state_blocks_validation(L, case, expect):
    c = dict(refs=FAKE, P=4, max_bytes=1 << 21, src=FAKE, dst=FAKE, n=8)
    c.update(case)
    st = L.gdn_copy_state_blocks(c["refs"], c["P"], c["max_bytes"], c["src"], c["dst"], c["n"], None)
    assert st == expect, gdn.gdn_last_error()


def test_replay_dual_validation(L):
    dims = _dims()
    master, copy = _pool(), _pool(base=FAKE + 4096, dtype=gdn.GDN_BF16)
    ring = _ring()

    def dec(B=4, m=master, c=copy):
        return L.gdn_replay_decode_dual(ctypes.byref(dims), B, 1, FAKE, FAKE, FAKE, gdn.GDN_BF16,
                                        ctypes.byref(_gates()), ctypes.byref(m), ctypes.byref(c) if c else None,
                                        FAKE, ctypes.byref(ring), FAKE, gdn.GDN_F32, FAKE, 1 << 30, None)

    assert dec(c=None) == gdn.GDN_EINVAL
    assert dec(m=_pool(dtype=gdn.GDN_BF16)) == gdn.GDN_EINVAL                 # master must be f32
    assert dec(c=_pool(base=FAKE + 4096, dtype=gdn.GDN_F32)) == gdn.GDN_EINVAL  # copy must be 16-bit
    assert dec(c=_pool(base=FAKE + 4096, dtype=gdn.GDN_BF16, n=9)) == gdn.GDN_EINVAL
    assert dec(c=_pool(base=FAKE, dtype=gdn.GDN_BF16)) == gdn.GDN_EINVAL      # aliases the master
    assert dec(B=0) == gdn.GDN_OK
    st = L.gdn_replay_flush_dual(ctypes.byref(dims), 4, ctypes.byref(master), None, FAKE, ctypes.byref(ring), None)
    assert st == gdn.GDN_EINVAL


def test_replay_noalloc_validation(L):
    """The fixed-scratch replay step rejects a workspace beyond its 96 MiB before any device call
    (B = 1024 x 32 value heads x T = 5 at dv = 128 needs 162.5 MiB), and a B = 0 call is a no-op."""
    dims = _dims()
    ring, pool = _ring(), _pool()

    def call(B, T):
        return L.gdn_replay_decode_noalloc(ctypes.byref(dims), B, T, FAKE, FAKE, FAKE, gdn.GDN_BF16,
                                           ctypes.byref(_gates()), ctypes.byref(pool), FAKE, ctypes.byref(ring),
                                           FAKE, gdn.GDN_F32, None)
    assert call(1024, 5) == gdn.GDN_EUNSUPPORTED
    assert "fixed scratch" in gdn.gdn_last_error()
    assert call(0, 5) == gdn.GDN_OK
    assert call(4, 0) == gdn.GDN_EINVAL
