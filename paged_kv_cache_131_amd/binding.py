"""ctypes binding of libpagedattn.so (declared in include/pagedattn.h).

Argument marshalling only: every function checks that it was given device
tensors of the right shape and dtype, derives the sizes, and calls the C
entry point of the same name on the current HIP stream. Nothing is computed
here. A missing library is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
ALGO_CODE = {"auto": 0, "vector": 1, "mfma": 2}
PA_PARTITION_AUTO = -1
PA_PARTITION_NONE = 0
WORKSPACE_COUNTER_BYTES = 32768  # PA_WORKSPACE_COUNTER_BYTES: zero between calls
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_WORKSPACE",
          -4: "PA_ERR_LAUNCH"}

# every exported symbol with its C signature (restype, argtypes)
_p, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "pa_write_kv": (_i32, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_decode": (_i32, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                         _p, _sz, _i32, _i32, _p]),
    "pa_decode_ex": (_i32, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                            _p, _sz, _i32, _i32, _i32, _p]),
    "pa_decode_noalloc": (_i32, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                 _i32, _i32, _i32, _p]),
    "pa_write_decode": (_i32, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                               _i32, _p, _sz, _i32, _i32, _p]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_launches": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_copy_blocks": (_i32, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_prefill": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                          _i32, _p]),
    "pa_swap_out": (_i32, [_p, _i32, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_swap_in": (_i32, [_p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_abi_version": (_i32, []),
}

_lib = None


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIBRARY:
        _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedAttnError(fn, status)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def pa_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """k_new/v_new [T][Hkv][d]; k_cache [NB][Hkv][B][d]; v_cache [NB][Hkv][d][B] (elements in the
    header's V order: 32-token sub-tiles for block sizes that are multiples of 32 above 32); slot_mapping [T] int32."""
    lib = load_library()
    T, Hkv, d = k_new.shape
    NB, _, B, _ = k_cache.shape
    if v_new.shape != k_new.shape or v_cache.shape != (NB, Hkv, d, B) or k_cache.shape[1:] != (Hkv, B, d):
        raise ValueError("inconsistent shapes")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    dt = k_cache.dtype
    args = [_dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt), _dev(k_cache, "k_cache", dt),
            _dev(v_cache, "v_cache", dt), _dev(slot_mapping, "slot_mapping", torch.int32)]
    _check("pa_write_kv", lib.pa_write_kv(*args, T, Hkv, d, B, NB, DTYPE_CODE[dt], _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """block_mapping [P][2] int32 (src, dst) pairs."""
    lib = load_library()
    NB, Hkv, B, d = k_cache.shape
    if v_cache.shape != (NB, Hkv, d, B):
        raise ValueError("inconsistent shapes")
    P = block_mapping.shape[0] if block_mapping.numel() else 0
    if block_mapping.numel() and tuple(block_mapping.shape) != (P, 2):
        raise ValueError("block_mapping must be [num_pairs][2]")
    dt = k_cache.dtype
    ptr = _dev(block_mapping, "block_mapping", torch.int32) if P else None
    _check("pa_copy_blocks", lib.pa_copy_blocks(_dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), ptr, P,
                                                Hkv, d, B, NB, DTYPE_CODE[dt], _stream(stream)))


def pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size=PA_PARTITION_AUTO) -> int:
    return int(load_library().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                        max_context_len, partition_size))


def pa_decode_launches(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                       partition_size=PA_PARTITION_AUTO, dtype=torch.bfloat16, algo="auto", fused=False) -> int:
    """Kernel launches pa_decode (fused=False) or pa_write_decode (fused=True) makes for these sizes on the
    current device (0 for no sequences or rejected arguments)."""
    return int(load_library().pa_decode_launches(num_seqs, num_heads, num_kv_heads, head_dim, int(max_context_len),
                                                 int(partition_size), DTYPE_CODE[dtype], ALGO_CODE[algo],
                                                 int(bool(fused))))


_workspaces = {}


def workspace_for(device, nbytes: int, stream_handle: int) -> torch.Tensor:
    """A workspace of at least nbytes on `device` for calls on the stream
    `stream_handle`, reused by later calls on that stream (they run in order,
    so they never use it at the same time). Calls on different streams get
    different workspaces. A workspace is allocated, zero-filled (its arrival
    counters start at zero), on the stream that uses it, so that when a
    larger one replaces it, the allocator reuses its memory only after the
    work already queued on that stream."""
    dev = torch.device(device)
    key = (dev, int(stream_handle))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(torch.cuda.ExternalStream(int(stream_handle), device=dev)):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
              partition_size=PA_PARTITION_AUTO, workspace=None, algo="auto", stream=None) -> None:
    """out [S][Hq][d] (f32/f16/bf16); q [S][Hq][d]; block_tables [S][max_blocks] int32; context_lens [S] int32."""
    lib = load_library()
    S, Hq, d = q.shape
    NB, Hkv, B, _ = k_cache.shape
    if out.shape != q.shape or v_cache.shape != (NB, Hkv, d, B) or k_cache.shape[3] != d:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    dt = k_cache.dtype
    ptrs = (_dev(out, "out"), _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32))
    need = int(lib.pa_decode_workspace_bytes(S, Hq, Hkv, d, int(max_context_len), int(partition_size)))
    sh = _stream(stream)
    if workspace is None and need:
        workspace = workspace_for(q.device, need, sh)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    status = lib.pa_decode_ex(
        *ptrs, S, Hq, Hkv, d, B, NB, block_tables.shape[1], int(max_context_len), float(scale), int(partition_size),
        ws_ptr, ws_bytes, DTYPE_CODE[dt], DTYPE_CODE[out.dtype], ALGO_CODE[algo], sh)
    _check("pa_decode", status)


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                      partition_size=PA_PARTITION_AUTO, stream=None) -> None:
    """pa_decode without a workspace argument: split sequences use the library's fixed per-device array
    (calls that may overlap on one device race on it)."""
    lib = load_library()
    S, Hq, d = q.shape
    NB, Hkv, B, _ = k_cache.shape
    if out.shape != q.shape or v_cache.shape != (NB, Hkv, d, B) or k_cache.shape[3] != d:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    dt = k_cache.dtype
    ptrs = (_dev(out, "out"), _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32))
    status = lib.pa_decode_noalloc(*ptrs, S, Hq, Hkv, d, B, NB, block_tables.shape[1], int(max_context_len),
                                   float(scale), int(partition_size), DTYPE_CODE[dt], DTYPE_CODE[out.dtype],
                                   _stream(stream))
    _check("pa_decode_noalloc", status)


# ---------------------------------------------------------------------------
# Host <-> device transfers of stored element arrays (numpy float32, float16,
# or uint16 raw bfloat16 bits). Pure data movement.
# ---------------------------------------------------------------------------
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(arr, etype: str, device) -> torch.Tensor:
    import numpy as np
    a = np.ascontiguousarray(arr)
    if etype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor, etype: str):
    import numpy as np
    c = t.detach().contiguous().cpu()
    if etype == "bf16":
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def int32_to_device(arr, device) -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(device)


def pa_write_decode(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                    partition_size=PA_PARTITION_AUTO, workspace=None, stream=None) -> None:
    """Store each sequence's new token (k_new/v_new [S][Hkv][d]) at position context_lens[s]-1 and decode,
    in one launch."""
    lib = load_library()
    S, Hq, d = q.shape
    NB, Hkv, B, _ = k_cache.shape
    if out.shape != q.shape or v_cache.shape != (NB, Hkv, d, B) or k_cache.shape[3] != d:
        raise ValueError("inconsistent shapes")
    if k_new.shape != (S, Hkv, d) or v_new.shape != (S, Hkv, d):
        raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    dt = k_cache.dtype
    ptrs = (_dev(out, "out"), _dev(q, "q", dt), _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
            _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32))
    need = int(lib.pa_decode_workspace_bytes(S, Hq, Hkv, d, int(max_context_len), int(partition_size)))
    sh = _stream(stream)
    if workspace is None and need:
        workspace = workspace_for(q.device, need, sh)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    status = lib.pa_write_decode(
        *ptrs, S, Hq, Hkv, d, B, NB, block_tables.shape[1], int(max_context_len), float(scale), int(partition_size),
        ws_ptr, ws_bytes, DTYPE_CODE[dt], DTYPE_CODE[out.dtype], sh)
    _check("pa_write_decode", status)


def swap_space(num_slots: int, k_cache) -> torch.Tensor:
    """Pinned host swap space for whole blocks of this pool: [slots][2][block
    elements] (K image, V image) of the pool's element type."""
    NB, Hkv, B, d = k_cache.shape
    return torch.empty((num_slots, 2, Hkv * B * d), dtype=k_cache.dtype, pin_memory=True)


def _swap_args(host, k_cache, v_cache, block_mapping):
    NB, Hkv, B, d = k_cache.shape
    if v_cache.shape != (NB, Hkv, d, B):
        raise ValueError("inconsistent shapes")
    if not isinstance(host, torch.Tensor) or host.is_cuda or not host.is_pinned() or not host.is_contiguous():
        raise TypeError("host must be a contiguous pinned CPU tensor")
    if host.dim() != 3 or host.shape[1:] != (2, Hkv * B * d) or host.dtype != k_cache.dtype:
        raise ValueError("host must be [slots][2][num_kv_heads*block_size*head_dim] of the pool's dtype")
    P = block_mapping.shape[0] if block_mapping.numel() else 0
    if block_mapping.numel() and tuple(block_mapping.shape) != (P, 2):
        raise ValueError("block_mapping must be [num_pairs][2]")
    ptr = _dev(block_mapping, "block_mapping", torch.int32) if P else None
    return host.shape[0], ptr, P, Hkv, d, B, NB


def pa_swap_out(host, k_cache, v_cache, block_mapping, stream=None) -> None:
    """block_mapping [P][2] int32 (device block, host slot): host slot <- block."""
    lib = load_library()
    slots, ptr, P, Hkv, d, B, NB = _swap_args(host, k_cache, v_cache, block_mapping)
    dt = k_cache.dtype
    _check("pa_swap_out", lib.pa_swap_out(host.data_ptr(), slots, _dev(k_cache, "k_cache", dt),
                                          _dev(v_cache, "v_cache", dt), ptr, P, Hkv, d, B, NB, DTYPE_CODE[dt],
                                          _stream(stream)))


def pa_swap_in(k_cache, v_cache, host, block_mapping, stream=None) -> None:
    """block_mapping [P][2] int32 (device block, host slot): block <- host slot."""
    lib = load_library()
    slots, ptr, P, Hkv, d, B, NB = _swap_args(host, k_cache, v_cache, block_mapping)
    dt = k_cache.dtype
    _check("pa_swap_in", lib.pa_swap_in(_dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
                                        host.data_ptr(), slots, ptr, P, Hkv, d, B, NB, DTYPE_CODE[dt],
                                        _stream(stream)))


def pa_prefill(out, q, q_start, k_cache, v_cache, block_tables, context_lens, scale, stream=None) -> None:
    """q, out [total_q][num_heads][head_dim]; q_start [num_seqs + 1] int32: sequence s owns rows
    q_start[s] .. q_start[s+1]-1, the last tokens of its context_lens[s]."""
    lib = load_library()
    TQ, Hq, d = q.shape
    NB, Hkv, B, _ = k_cache.shape
    if out.shape != q.shape or v_cache.shape != (NB, Hkv, d, B) or k_cache.shape[3] != d:
        raise ValueError("inconsistent shapes")
    S = context_lens.shape[0]
    if q_start.shape != (S + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("q_start must be [num_seqs + 1], block_tables [num_seqs][max_blocks]")
    dt = k_cache.dtype
    _check("pa_prefill", lib.pa_prefill(
        _dev(out, "out"), _dev(q, "q", dt), _dev(q_start, "q_start", torch.int32), TQ, _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, d, B, NB, block_tables.shape[1], float(scale),
        DTYPE_CODE[dt], DTYPE_CODE[out.dtype], _stream(stream)))
