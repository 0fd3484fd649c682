"""ctypes binding of libgdn.so (include/gdn.h).

Argument marshalling only: shapes are read off torch tensors, pointers and
sizes are handed to the C ABI, and every step of the computation runs in the
HIP kernels behind it.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_ELAUNCH = 0, 1, 2, 3

# every symbol include/gdn.h declares
EXPORTS = (
    "gdn_decode_step", "gdn_spec_decode", "gdn_copy_state_blocks", "gdn_chunk_prefill_workspace_bytes", "gdn_chunk_prefill", "gdn_replay_workspace_bytes",
    "gdn_replay_decode", "gdn_replay_decode_noalloc",
    "gdn_replay_flush", "gdn_replay_rollback", "gdn_replay_decode_dual", "gdn_replay_flush_dual",
    "gdn_mamba2_decode_step", "gdn_mamba2_replay_decode", "gdn_mamba2_replay_flush", "gdn_mamba2_replay_rollback",
    "gdn_status_string", "gdn_last_error",
)


class gdn_state_ref(ctypes.Structure):
    _fields_ = [("base", ctypes.c_uint64), ("slot_bytes", ctypes.c_uint64), ("num_slots", ctypes.c_uint64)]


class gdn_m2_dims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("num_groups", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32)]


class gdn_m2_params(ctypes.Structure):
    _fields_ = [("dt", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("D", ctypes.c_void_p)]


class gdn_m2_ring(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("Bm", ctypes.c_void_p), ("g", ctypes.c_void_p), ("dtp", ctypes.c_void_p),
                ("start", ctypes.c_void_p), ("count", ctypes.c_void_p), ("num_slots", ctypes.c_int64),
                ("L", ctypes.c_int32), ("dtype", ctypes.c_int)]


class gdn_dims(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("scale", ctypes.c_float)]


class gdn_gates(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


class gdn_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("dtype", ctypes.c_int), ("num_slots", ctypes.c_int64)]


class gdn_ring(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("start", ctypes.c_void_p), ("count", ctypes.c_void_p), ("num_slots", ctypes.c_int64),
                ("L", ctypes.c_int32), ("dtype", ctypes.c_int)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m gated_deltanet_state_gdn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, INT = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    pd, pg, pp, pr = (ctypes.POINTER(gdn_dims), ctypes.POINTER(gdn_gates), ctypes.POINTER(gdn_pool),
                      ctypes.POINTER(gdn_ring))
    pm, pmp, pmr = ctypes.POINTER(gdn_m2_dims), ctypes.POINTER(gdn_m2_params), ctypes.POINTER(gdn_m2_ring)
    sig = {
        "gdn_decode_step": (INT, [pd, I32, P, P, P, INT, pg, pp, P, P, INT, P]),
        "gdn_spec_decode": (INT, [pd, I32, I32, P, P, P, INT, pg, pp, P, P, P, INT, P]),
        "gdn_copy_state_blocks": (INT, [P, I32, ctypes.c_uint64, P, P, I32, P]),
        "gdn_chunk_prefill_workspace_bytes": (SZ, [pd, I32, I64, I32]),
        "gdn_chunk_prefill": (INT, [pd, I32, P, I64, I32, P, P, P, INT, pg, pp, P, P, INT, P, SZ, P]),
        "gdn_replay_workspace_bytes": (SZ, [pd, I32, I32]),
        "gdn_replay_decode": (INT, [pd, I32, I32, P, P, P, INT, pg, pp, P, pr, P, INT, P, SZ, P]),
        "gdn_replay_decode_noalloc": (INT, [pd, I32, I32, P, P, P, INT, pg, pp, P, pr, P, INT, P]),
        "gdn_replay_flush": (INT, [pd, I32, pp, P, pr, P]),
        "gdn_replay_decode_dual": (INT, [pd, I32, I32, P, P, P, INT, pg, pp, pp, P, pr, P, INT, P, SZ, P]),
        "gdn_replay_flush_dual": (INT, [pd, I32, pp, pp, P, pr, P]),
        "gdn_replay_rollback": (INT, [pd, I32, P, P, pr, P]),
        "gdn_mamba2_decode_step": (INT, [pm, I32, P, P, P, INT, pmp, pp, P, P, INT, P]),
        "gdn_mamba2_replay_decode": (INT, [pm, I32, I32, P, P, P, INT, pmp, pp, P, pmr, P, INT, P]),
        "gdn_mamba2_replay_flush": (INT, [pm, I32, pp, P, pmr, P]),
        "gdn_mamba2_replay_rollback": (INT, [pm, I32, P, P, pmr, P]),
        "gdn_status_string": (ctypes.c_char_p, [INT]),
        "gdn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != GDN_OK:
        L = lib()
        raise GdnError(status, f"{L.gdn_status_string(status).decode()}: {L.gdn_last_error().decode()}")


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    torch = _torch()
    codes = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}")
    return codes[dt]


def _ptr(t) -> int:
    if not t.is_contiguous():
        raise ValueError("tensors passed to the GDN library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _keep_for_stream(tensors, stream):
    """Buffers this binding allocated on the current stream but hands to a launch on another
    stream are marked as used there, so the caching allocator does not give their memory to a
    later allocation on the current stream while the launch may still run."""
    torch = _torch()
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _dims(Hk, Hv, dk, dv, scale):
    return gdn_dims(int(Hk), int(Hv), int(dk), int(dv), float(scale) if scale else 0.0)


def _gates(a, b, A_log, dt_bias):
    return gdn_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias))


def _pool(pool):
    return gdn_pool(_ptr(pool), dtype_code(pool.dtype), int(pool.shape[0]))


@dataclass
class Ring:
    """ReplaySSM ring of inputs per slot (layout of gdn_ring; keys once per key head, one pointer pair
    per slot)."""
    k: object      # [num_slots, Hk, L, dk]
    v: object      # [num_slots, Hv, L, dv]
    g: object      # [num_slots, Hv, L] float32
    beta: object   # [num_slots, Hv, L] float32
    start: object  # [num_slots] int32
    count: object  # [num_slots] int32

    @property
    def L(self) -> int:
        return int(self.g.shape[2])

    def c_struct(self) -> gdn_ring:
        return gdn_ring(_ptr(self.k), _ptr(self.v), _ptr(self.g), _ptr(self.beta), _ptr(self.start),
                        _ptr(self.count), int(self.g.shape[0]), self.L, dtype_code(self.k.dtype))


def new_ring(num_slots, Hk, Hv, L, dk, dv, dtype, device) -> Ring:
    torch = _torch()
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
    return Ring(k=z((num_slots, Hk, L, dk), dtype), v=z((num_slots, Hv, L, dv), dtype),
                g=z((num_slots, Hv, L), torch.float32), beta=z((num_slots, Hv, L), torch.float32),
                start=z((num_slots,), torch.int32), count=z((num_slots,), torch.int32))


# ------------------------------------------------------------------ entry points
def gdn_decode_step(q, k, v, a, b, A_log, dt_bias, pool, slot_map, out=None, out_dtype=None, scale=None,
                    stream=None):
    """One decode step; q, k [B, Hk, dk]; v [B, Hv, dv]; a, b [B, Hv]; pool [slots, Hv, dk, dv]."""
    torch = _torch()
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if out is None:
        out = torch.empty((B, Hv, dv), dtype=out_dtype or torch.float32, device=q.device)
        _keep_for_stream([out], stream)
    dims = _dims(Hk, Hv, dk, dv, scale)
    _check(lib().gdn_decode_step(ctypes.byref(dims), B, _ptr(q), _ptr(k), _ptr(v), dtype_code(q.dtype),
                                 ctypes.byref(_gates(a, b, A_log, dt_bias)), ctypes.byref(_pool(pool)),
                                 _ptr(slot_map), _ptr(out), dtype_code(out.dtype), _stream(stream)))
    return out


def gdn_spec_decode(q, k, v, a, b, A_log, dt_bias, pool, src_slots, dst_slots, out=None, out_dtype=None,
                    scale=None, stream=None):
    """Speculative window keeping every state; q, k [B, T, Hk, dk]; v [B, T, Hv, dv]; a, b [B, T, Hv];
    src_slots int32 [B]; dst_slots int32 [B, T] (device)."""
    torch = _torch()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=out_dtype or torch.float32, device=q.device)
        _keep_for_stream([out], stream)
    dims = _dims(Hk, Hv, dk, dv, scale)
    _check(lib().gdn_spec_decode(ctypes.byref(dims), B, T, _ptr(q), _ptr(k), _ptr(v), dtype_code(q.dtype),
                                 ctypes.byref(_gates(a, b, A_log, dt_bias)), ctypes.byref(_pool(pool)),
                                 _ptr(src_slots), _ptr(dst_slots), _ptr(out), dtype_code(out.dtype),
                                 _stream(stream)))
    return out


def state_refs_bytes(entries) -> bytes:
    """Pack (base address, slot bytes, slot count) triples as the gdn_state_ref table: three
    little-endian unsigned 64-bit fields each, so an address at or above 2^63 keeps every bit."""
    import struct
    return b"".join(struct.pack("<QQQ", int(b), int(sb), int(n)) for b, sb, n in entries)


def make_state_table(tensors, device):
    """Device gdn_state_ref table for contiguous [num_slots, ...] device tensors:
    returns (table uint8 tensor, P, max_slot_bytes).  Reusable while the tensors live."""
    torch = _torch()
    entries = []
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("state tensors must be contiguous")
        entries.append((t.data_ptr(), t[0].numel() * t.element_size(), t.shape[0]))
    host_table = torch.frombuffer(bytearray(state_refs_bytes(entries)), dtype=torch.uint8)
    return host_table.to(device), len(entries), max((e[1] for e in entries), default=0)


def gdn_copy_state_blocks(tensors, src_slots, dst_slots, stream=None, table=None):
    """Copy slot src_slots[j] over dst_slots[j] in every tensor (each contiguous [num_slots, ...] on the
    device); src_slots, dst_slots int32 [n] (device).  `table` may be a prebuilt make_state_table()
    result for the same tensors; otherwise one is built and uploaded on the copy's stream."""
    torch = _torch()
    n = int(src_slots.shape[0])
    if len(tensors) == 0 or n == 0:
        return
    if table is None:
        if stream is None or isinstance(stream, torch.cuda.Stream):
            # upload on the stream the copy runs on, so the kernel is ordered after it
            with torch.cuda.stream(stream or torch.cuda.current_stream()):
                table = make_state_table(tensors, src_slots.device)
            if stream is not None:
                table[0].record_stream(stream)
        else:  # a raw stream handle: finish the upload before enqueueing
            table = make_state_table(tensors, src_slots.device)
            torch.cuda.current_stream().synchronize()
    dev_table, P, max_bytes = table
    _check(lib().gdn_copy_state_blocks(_ptr(dev_table), P, max_bytes, _ptr(src_slots), _ptr(dst_slots), n,
                                       _stream(stream)))


def gdn_chunk_prefill_workspace_bytes(Hk, Hv, dk, dv, N, total_tokens, chunk=64) -> int:
    dims = _dims(Hk, Hv, dk, dv, None)
    return int(lib().gdn_chunk_prefill_workspace_bytes(ctypes.byref(dims), int(N), int(total_tokens), int(chunk)))


def gdn_chunk_prefill(q, k, v, a, b, A_log, dt_bias, pool, slot_map, cu_seqlens, out=None, out_dtype=None,
                      chunk=64, workspace=None, scale=None, stream=None):
    """Packed prefill; q, k [T, Hk, dk]; v [T, Hv, dv]; a, b [T, Hv]; cu_seqlens int32 [N+1] (device)."""
    torch = _torch()
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = int(cu_seqlens.shape[0]) - 1
    if out is None:
        out = torch.empty((T, Hv, dv), dtype=out_dtype or torch.float32, device=q.device)
        _keep_for_stream([out], stream)
    need = gdn_chunk_prefill_workspace_bytes(Hk, Hv, dk, dv, N, T, chunk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _keep_for_stream([workspace], stream)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    dims = _dims(Hk, Hv, dk, dv, scale)
    _check(lib().gdn_chunk_prefill(ctypes.byref(dims), N, _ptr(cu_seqlens), T, chunk, _ptr(q), _ptr(k), _ptr(v),
                                   dtype_code(q.dtype), ctypes.byref(_gates(a, b, A_log, dt_bias)),
                                   ctypes.byref(_pool(pool)), _ptr(slot_map), _ptr(out), dtype_code(out.dtype),
                                   ws_ptr, ws_bytes, _stream(stream)))
    return out


def gdn_replay_workspace_bytes(Hk, Hv, dk, dv, B, T) -> int:
    dims = _dims(Hk, Hv, dk, dv, None)
    return int(lib().gdn_replay_workspace_bytes(ctypes.byref(dims), int(B), int(T)))


def gdn_replay_decode(q, k, v, a, b, A_log, dt_bias, ckpt, slot_map, ring: Ring, out=None, out_dtype=None,
                      workspace=None, scale=None, stream=None, read_copy=None):
    """Replay step of T tokens; q, k [B, T, Hk, dk]; v [B, T, Hv, dv]; a, b [B, T, Hv].
    With `read_copy` (a bf16/f16 pool beside the f32 `ckpt`), the dual-precision variant runs."""
    torch = _torch()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=out_dtype or torch.float32, device=q.device)
        _keep_for_stream([out], stream)
    need = gdn_replay_workspace_bytes(Hk, Hv, dk, dv, B, T)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _keep_for_stream([workspace], stream)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    dims = _dims(Hk, Hv, dk, dv, scale)
    rs = ring.c_struct()
    head = (ctypes.byref(dims), B, T, _ptr(q), _ptr(k), _ptr(v), dtype_code(q.dtype),
            ctypes.byref(_gates(a, b, A_log, dt_bias)), ctypes.byref(_pool(ckpt)))
    tail = (_ptr(slot_map), ctypes.byref(rs), _ptr(out), dtype_code(out.dtype), ws_ptr, ws_bytes, _stream(stream))
    if read_copy is None:
        _check(lib().gdn_replay_decode(*head, *tail))
    else:
        _check(lib().gdn_replay_decode_dual(*head, ctypes.byref(_pool(read_copy)), *tail))
    return out


def gdn_replay_decode_noalloc(q, k, v, a, b, A_log, dt_bias, ckpt, slot_map, ring: Ring, out, scale=None,
                              stream=None):
    """gdn_replay_decode on the library's fixed device scratch: no workspace argument, and `out`
    must be given (nothing is allocated)."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dims = _dims(Hk, Hv, dk, dv, scale)
    rs = ring.c_struct()
    _check(lib().gdn_replay_decode_noalloc(ctypes.byref(dims), B, T, _ptr(q), _ptr(k), _ptr(v), dtype_code(q.dtype),
                                           ctypes.byref(_gates(a, b, A_log, dt_bias)), ctypes.byref(_pool(ckpt)),
                                           _ptr(slot_map), ctypes.byref(rs), _ptr(out), dtype_code(out.dtype),
                                           _stream(stream)))
    return out


def gdn_replay_flush(ckpt, slot_map, ring: Ring, Hk, stream=None, read_copy=None):
    """Fold every committed ring entry of the mapped slots into their checkpoints (with `read_copy`:
    the dual-precision flush, which also refreshes the copy of every mapped slot)."""
    Hv, dk, dv = ckpt.shape[1], ckpt.shape[2], ckpt.shape[3]
    dims = _dims(Hk, Hv, dk, dv, None)
    rs = ring.c_struct()
    if read_copy is None:
        _check(lib().gdn_replay_flush(ctypes.byref(dims), int(slot_map.shape[0]), ctypes.byref(_pool(ckpt)),
                                      _ptr(slot_map), ctypes.byref(rs), _stream(stream)))
    else:
        _check(lib().gdn_replay_flush_dual(ctypes.byref(dims), int(slot_map.shape[0]), ctypes.byref(_pool(ckpt)),
                                           ctypes.byref(_pool(read_copy)), _ptr(slot_map), ctypes.byref(rs),
                                           _stream(stream)))


def gdn_replay_rollback(slot_map, num_rejected, ring: Ring, Hk, dk, stream=None):
    """count <- max(count - num_rejected[b], 0) for every value head of row b's slot."""
    Hv = int(ring.g.shape[1])
    dims = _dims(Hk, Hv, dk, dk, None)
    rs = ring.c_struct()
    _check(lib().gdn_replay_rollback(ctypes.byref(dims), int(slot_map.shape[0]), _ptr(slot_map),
                                     _ptr(num_rejected), ctypes.byref(rs), _stream(stream)))


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


# ------------------------------------------------------------------ Mamba2
@dataclass
class M2Ring:
    """Mamba2 ReplaySSM ring (layout of gdn_m2_ring); pointers are per slot."""
    x: object      # [num_slots, H, L, d]
    Bm: object     # [num_slots, G, L, n]
    g: object      # [num_slots, H, L] float32
    dtp: object    # [num_slots, H, L] float32
    start: object  # [num_slots] int32
    count: object  # [num_slots] int32

    @property
    def L(self) -> int:
        return int(self.g.shape[2])

    def c_struct(self) -> gdn_m2_ring:
        return gdn_m2_ring(_ptr(self.x), _ptr(self.Bm), _ptr(self.g), _ptr(self.dtp), _ptr(self.start),
                           _ptr(self.count), int(self.g.shape[0]), self.L, dtype_code(self.x.dtype))


def new_m2_ring(num_slots, H, G, L, d, n, dtype, device) -> M2Ring:
    torch = _torch()
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
    return M2Ring(x=z((num_slots, H, L, d), dtype), Bm=z((num_slots, G, L, n), dtype),
                  g=z((num_slots, H, L), torch.float32), dtp=z((num_slots, H, L), torch.float32),
                  start=z((num_slots,), torch.int32), count=z((num_slots,), torch.int32))


def _m2_params(dt, A_log, dt_bias, D):
    return gdn_m2_params(_ptr(dt), _ptr(A_log), _ptr(dt_bias), _ptr(D))


def gdn_mamba2_decode_step(x, Bm, Cm, dt, A_log, dt_bias, D, pool, slot_map, out=None, out_dtype=None, stream=None):
    """One Mamba2 decode step; x [B, H, d]; Bm, Cm [B, G, n]; dt [B, H]; pool [slots, H, d, n]."""
    torch = _torch()
    B, H, d = x.shape
    G, n = Bm.shape[1], Bm.shape[2]
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype or torch.float32, device=x.device)
        _keep_for_stream([out], stream)
    dims = gdn_m2_dims(H, G, d, n)
    _check(lib().gdn_mamba2_decode_step(ctypes.byref(dims), B, _ptr(x), _ptr(Bm), _ptr(Cm), dtype_code(x.dtype),
                                        ctypes.byref(_m2_params(dt, A_log, dt_bias, D)), ctypes.byref(_pool(pool)),
                                        _ptr(slot_map), _ptr(out), dtype_code(out.dtype), _stream(stream)))
    return out


def gdn_mamba2_replay_decode(x, Bm, Cm, dt, A_log, dt_bias, D, ckpt, slot_map, ring: M2Ring, out=None,
                             out_dtype=None, stream=None):
    """Mamba2 replay step of T tokens; x [B, T, H, d]; Bm, Cm [B, T, G, n]; dt [B, T, H]."""
    torch = _torch()
    B, T, H, d = x.shape
    G, n = Bm.shape[2], Bm.shape[3]
    if out is None:
        out = torch.empty((B, T, H, d), dtype=out_dtype or torch.float32, device=x.device)
        _keep_for_stream([out], stream)
    dims = gdn_m2_dims(H, G, d, n)
    rs = ring.c_struct()
    _check(lib().gdn_mamba2_replay_decode(ctypes.byref(dims), B, T, _ptr(x), _ptr(Bm), _ptr(Cm), dtype_code(x.dtype),
                                          ctypes.byref(_m2_params(dt, A_log, dt_bias, D)),
                                          ctypes.byref(_pool(ckpt)), _ptr(slot_map), ctypes.byref(rs), _ptr(out),
                                          dtype_code(out.dtype), _stream(stream)))
    return out


def gdn_mamba2_replay_flush(ckpt, slot_map, ring: M2Ring, stream=None):
    """Fold every committed entry of the mapped slots into their checkpoints."""
    H, d, n = ckpt.shape[1], ckpt.shape[2], ckpt.shape[3]
    dims = gdn_m2_dims(H, int(ring.Bm.shape[1]), d, n)
    rs = ring.c_struct()
    _check(lib().gdn_mamba2_replay_flush(ctypes.byref(dims), int(slot_map.shape[0]), ctypes.byref(_pool(ckpt)),
                                         _ptr(slot_map), ctypes.byref(rs), _stream(stream)))


def gdn_mamba2_replay_rollback(slot_map, num_rejected, ring: M2Ring, stream=None):
    """count <- max(count - num_rejected[b], 0) for row b's slot."""
    H, G = int(ring.x.shape[1]), int(ring.Bm.shape[1])
    dims = gdn_m2_dims(H, G, int(ring.x.shape[3]), int(ring.Bm.shape[3]))
    rs = ring.c_struct()
    _check(lib().gdn_mamba2_replay_rollback(ctypes.byref(dims), int(slot_map.shape[0]), _ptr(slot_map),
                                            _ptr(num_rejected), ctypes.byref(rs), _stream(stream)))
