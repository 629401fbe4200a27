"""Python binding of libmla_decode.so: paged absorbed-MLA decode on MI355X (gfx950).

Argument marshalling only.  Every step runs in the library's HIP kernels;
torch provides device memory and the current stream.  There is no fallback:
if the library is missing or a tensor is not on the GPU, calls raise.

Entry points (same names as the C ABI in include/mla_decode.h):
  mla_decode(q, kv_cache, block_table, seq_lens, causal_seqlens_global,
             cp_world, cp_rank, q_len, causal, scale, lse_base) -> (out, lse)
  mla_merge_lse(partials, lses, lse_base) -> (out, lse)
  cp_local_slot(positions, block_table, block_size, cp_world, cp_rank,
                num_valid=None, cp_interleave=1) -> slots
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "D_QK", "D_V", "PAD_SLOT_ID", "LSE_BASE_E", "LSE_BASE_2", "MLAError",
    "library_path", "load_library", "exported_symbols",
    "mla_decode", "mla_decode_varlen", "mla_decode_workspace_size", "mla_merge_lse", "cp_local_slot", "kv_write",
    "profile_attention_events", "mla_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "probe_mfma",
]

D_QK = 576
D_V = 512
PAD_SLOT_ID = -1
LSE_BASE_E = 0
LSE_BASE_2 = 1
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024  # MLA_NOALLOC_SCRATCH_BYTES

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmla_decode.so"
_lib = None

# (name, restype, argtypes) for every function include/mla_decode.h declares
_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = [
    ("mla_status_string", ctypes.c_char_p, [_I]),
    ("mla_decode_workspace_size", ctypes.c_size_t, [_I, _I, _I, _I]),
    ("mla_decode", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                        ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    ("mla_merge_lse", _I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    ("cp_local_slot", _I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, _P]),
    ("mla_profile_attention_events", _I, [_P, _P]),
    ("mla_probe_mfma", _I, [_I, _I, _P, _P]),
    ("mla_kv_write", _I, [_P, _P, ctypes.c_int64, _P, _I, _I, _P]),
    ("mla_decode_interleaved", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                    ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    ("mla_decode_varlen", _I, [_P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                               ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    ("mla_kv_write_fp8", _I, [_P, _P, ctypes.c_int64, ctypes.c_float, _P, _I, _I, _P]),
    ("mla_decode_fp8", _I, [_P, _P, ctypes.c_float, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                            ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    ("mla_decode_noalloc", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                ctypes.c_float, _I, _P, _P, _P]),
]

# dtypes accepted for an FP8 (E4M3) cache: torch's OCP E4M3 type or raw codes
_FP8_KV_DTYPES = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)


class MLAError(RuntimeError):
    pass


def library_path() -> str:
    return os.environ.get("MLA_DECODE_LIB", os.path.join(_PKG, _LIB_NAME))


def load_library():
    """Load the HIP library (built by decode_attention_11_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m decode_attention_11_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    return [s[0] for s in _SIGNATURES]


def _check(status: int) -> None:
    if status == 0:
        return
    msg = load_library().mla_status_string(status).decode()
    if status in (1, 2):
        raise ValueError(f"libmla_decode: {msg} (status {status})")
    raise MLAError(f"libmla_decode: {msg} (status {status})")


def _need(t: torch.Tensor, name: str, dtype, dim: Optional[int] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")


def _same_device(device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device} (every tensor of a call on one GPU)")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def profile_attention_events(start: Optional[int], stop: Optional[int]) -> None:
    """Record raw hipEvent_t handles around the attention kernel of following
    mla_decode calls of this thread (None, None to stop)."""
    _check(load_library().mla_profile_attention_events(start, stop))


def probe_mfma(workgroups: int, iters: int, out: Optional[torch.Tensor] = None,
               device: Optional[torch.device] = None) -> torch.Tensor:
    """Enqueue the library's bare bf16 MFMA loop (a measurement helper, not
    part of the decode path) on the current stream: workgroups * 4 waves *
    iters * 4 * 32768 flop.  Returns out (float32 [workgroups * 256]), which
    holds 64 * iters in every element once the launch has run."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty((workgroups * 256,), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() < workgroups * 256:
        raise ValueError("out must be a contiguous float32 tensor of workgroups * 256 values")
    _check(load_library().mla_probe_mfma(int(workgroups), int(iters), out.data_ptr(), _stream(out.device)))
    return out


def mla_decode_workspace_size(B: int, q_len: int, H: int, max_seq_len: int) -> int:
    return int(load_library().mla_decode_workspace_size(B, q_len, H, max_seq_len))


def mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
               causal_seqlens_global: Optional[torch.Tensor] = None, cp_world: int = 1, cp_rank: int = 0,
               q_len: Optional[int] = None, causal: bool = True, scale: Optional[float] = None,
               lse_base: str = "e", *, max_seq_len: Optional[int] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, return_lse: bool = True, cp_interleave: int = 1,
               kv_scale: Optional[float] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One rank's paged MLA decode.  q: [B, q_len, H, 576] (or [B*q_len, H, 576]
    with q_len given) bf16; kv_cache: [num_blocks, block_size, 576] bf16, or
    E4M3 codes (float8_e4m3fn or uint8) with kv_scale, the one dequantisation
    factor of the whole cache.  Returns out [B*q_len, H, 512] bf16 and lse
    [B*q_len, H] float32."""
    lib = load_library()
    if q.dim() == 3:
        if q_len is None:
            raise ValueError("q_len is required for a [tokens, H, 576] query")
        if q.shape[0] % q_len:
            raise ValueError("uneven query lengths are not supported: tokens must be B*q_len")
        q = q.view(q.shape[0] // q_len, q_len, q.shape[1], q.shape[2])
    _need(q, "q", torch.bfloat16, 4)
    B, Q, H, Dq = q.shape
    if q_len is not None and q_len != Q:
        raise ValueError(f"q_len={q_len} does not match q.shape[1]={Q}")
    if Dq != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    fp8 = kv_scale is not None
    if fp8:
        if kv_cache.dtype not in _FP8_KV_DTYPES:
            raise ValueError("an FP8 cache (kv_scale given) must be float8_e4m3fn or uint8 codes")
        _need(kv_cache, "kv_cache", kv_cache.dtype, 3)
    else:
        _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    if kv_cache.shape[2] != D_QK:
        raise ValueError(f"kv_cache last dim must be {D_QK}")
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have B rows")
    if causal_seqlens_global is not None:
        _need(causal_seqlens_global, "causal_seqlens_global", torch.int32, 1)
        if causal_seqlens_global.shape[0] != B:
            raise ValueError("causal_seqlens_global must have B entries")
    num_blocks, bs = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    max_blocks = int(block_table.shape[1])
    if max_seq_len is None:
        max_seq_len = max_blocks * bs  # the table's capacity bounds every local length
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    base = {"e": LSE_BASE_E, "2": LSE_BASE_2}.get(str(lse_base))
    if base is None:
        raise ValueError("lse_base must be 'e' or '2'")
    dev = q.device
    _same_device(dev, kv_cache=kv_cache, block_table=block_table, seq_lens=seq_lens,
                 causal_seqlens_global=causal_seqlens_global, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((B * Q, H, D_V), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (B * Q, H, D_V):
            raise ValueError("out must be [B*q_len, H, 512]")
    if return_lse:
        if lse is None:
            lse = torch.empty((B * Q, H), dtype=torch.float32, device=dev)
        else:
            _need(lse, "lse", torch.float32, 2)
            if tuple(lse.shape) != (B * Q, H):
                raise ValueError("lse must be [B*q_len, H]")
    ws_bytes = int(lib.mla_decode_workspace_size(B, Q, H, int(max_seq_len)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    head = (q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
            causal_seqlens_global.data_ptr() if causal_seqlens_global is not None else None,
            B, Q, H, num_blocks, bs, max_blocks, int(max_seq_len), int(cp_world), int(cp_rank))
    tail = (1 if causal else 0, float(scale), base, out.data_ptr(),
            lse.data_ptr() if (return_lse and lse is not None) else None,
            workspace.data_ptr(), int(workspace.numel()), _stream(dev))
    if fp8:
        _check(lib.mla_decode_fp8(head[0], head[1], float(kv_scale), *head[2:], int(cp_interleave), *tail))
    elif cp_interleave == 1:
        _check(lib.mla_decode(*head, *tail))
    else:
        _check(lib.mla_decode_interleaved(*head, int(cp_interleave), *tail))
    return out, (lse if return_lse else None)


def mla_decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                       causal_seqlens_global: Optional[torch.Tensor] = None, cp_world: int = 1, cp_rank: int = 0,
                       causal: bool = True, scale: Optional[float] = None, lse_base: str = "e", *,
                       out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                       max_seq_len: Optional[int] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """mla_decode that allocates nothing, for callers that cannot allocate: the split-KV
    partials live in the library's fixed per-GPU device array, and the caller passes out
    [B*q_len, H, 512] bf16 (and lse [B*q_len, H] float32, or None).  Calls on one GPU share
    that array and must not overlap.  q: [B, q_len, H, 576] bf16; other arguments as for
    mla_decode (bf16 cache, interleave 1)."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    B, Q, H, Dq = q.shape
    if Dq != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    if kv_cache.shape[2] != D_QK:
        raise ValueError(f"kv_cache last dim must be {D_QK}")
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have B rows")
    if causal_seqlens_global is not None:
        _need(causal_seqlens_global, "causal_seqlens_global", torch.int32, 1)
        if causal_seqlens_global.shape[0] != B:
            raise ValueError("causal_seqlens_global must have B entries")
    _need(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B * Q, H, D_V):
        raise ValueError("out must be [B*q_len, H, 512]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (B * Q, H):
            raise ValueError("lse must be [B*q_len, H]")
    dev = q.device
    _same_device(dev, kv_cache=kv_cache, block_table=block_table, seq_lens=seq_lens,
                 causal_seqlens_global=causal_seqlens_global, out=out, lse=lse)
    num_blocks, bs = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    max_blocks = int(block_table.shape[1])
    if max_seq_len is None:
        max_seq_len = max_blocks * bs
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    base = {"e": LSE_BASE_E, "2": LSE_BASE_2}.get(str(lse_base))
    if base is None:
        raise ValueError("lse_base must be 'e' or '2'")
    _check(lib.mla_decode_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
        causal_seqlens_global.data_ptr() if causal_seqlens_global is not None else None,
        B, Q, H, num_blocks, bs, max_blocks, int(max_seq_len), int(cp_world), int(cp_rank), 1 if causal else 0,
        float(scale), base, out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(dev)))
    return out, lse


def mla_merge_lse(partials: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], lse_base: str = "e",
                  *, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """LSE-weighted merge of partial outputs [rows, H, 512] bf16 with their lse [rows, H] f32."""
    lib = load_library()
    n = len(partials)
    if n != len(lses) or n < 1 or n > 64:
        raise ValueError("need 1..64 partials with one lse each")
    for i, (p, l) in enumerate(zip(partials, lses)):
        _need(p, f"partials[{i}]", torch.bfloat16, 3)
        _need(l, f"lses[{i}]", torch.float32, 2)
        if p.shape != partials[0].shape or tuple(l.shape) != tuple(partials[0].shape[:2]):
            raise ValueError("partials and lses must share shapes [rows, H, 512] / [rows, H]")
    rows, H, dv = partials[0].shape
    if dv != D_V:
        raise ValueError("partials must be [rows, H, 512]")
    base = {"e": LSE_BASE_E, "2": LSE_BASE_2}.get(str(lse_base))
    if base is None:
        raise ValueError("lse_base must be 'e' or '2'")
    dev = partials[0].device
    _same_device(dev, **{f"partials[{i}]": p for i, p in enumerate(partials)},
                 **{f"lses[{i}]": l for i, l in enumerate(lses)}, out=out, lse=lse)
    out = torch.empty((rows, H, D_V), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((rows, H), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (rows, H, D_V):
        raise ValueError(f"out must be [{rows}, {H}, {D_V}], got {tuple(out.shape)}")
    if tuple(lse.shape) != (rows, H):
        raise ValueError(f"lse must be [{rows}, {H}], got {tuple(lse.shape)}")
    parr = (ctypes.c_void_p * n)(*[p.data_ptr() for p in partials])
    larr = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    _check(lib.mla_merge_lse(ctypes.cast(parr, ctypes.c_void_p), ctypes.cast(larr, ctypes.c_void_p), n,
                             int(rows), int(H), base, out.data_ptr(), lse.data_ptr(), _stream(dev)))
    return out, lse


def cp_local_slot(positions: torch.Tensor, block_table: torch.Tensor, block_size: int, cp_world: int,
                  cp_rank: int, num_valid: Optional[torch.Tensor] = None, cp_interleave: int = 1,
                  *, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rank-local slots [B, n] int64 of positions [B, n] int64, PAD_SLOT_ID where not owned."""
    lib = load_library()
    _need(positions, "positions", torch.int64, 2)
    _need(block_table, "block_table", torch.int32, 2)
    B, n = positions.shape
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    if num_valid is not None:
        _need(num_valid, "num_valid", torch.int32, 1)
        if num_valid.shape[0] != B:
            raise ValueError("num_valid must have B entries")
    _same_device(positions.device, block_table=block_table, num_valid=num_valid, out=out)
    out = torch.empty((B, n), dtype=torch.int64, device=positions.device) if out is None else out
    _need(out, "out", torch.int64, 2)
    if tuple(out.shape) != (B, n):
        raise ValueError(f"out must be [{B}, {n}], got {tuple(out.shape)}")
    _check(lib.cp_local_slot(positions.data_ptr(), num_valid.data_ptr() if num_valid is not None else None,
                             int(B), int(n), block_table.data_ptr(), int(block_table.shape[1]),
                             int(block_size), int(cp_world), int(cp_rank), int(cp_interleave),
                             out.data_ptr(), _stream(positions.device)))
    return out


def kv_write(kv_new: torch.Tensor, slots: torch.Tensor, kv_cache: torch.Tensor,
             kv_scale: Optional[float] = None) -> torch.Tensor:
    """Store new KV rows [..., 576] bf16 at their slots [...] int64 in kv_cache
    [num_blocks, block_size, 576] (in place); pad and out-of-range slots
    write nothing.  A bf16 cache takes the rows as they are; an FP8 cache
    (float8_e4m3fn or uint8 codes, kv_scale given) takes the E4M3 codes of
    row / kv_scale.  Returns kv_cache."""
    lib = load_library()
    _need(kv_new, "kv_new", torch.bfloat16)
    _need(slots, "slots", torch.int64)
    fp8 = kv_scale is not None
    if fp8:
        if kv_cache.dtype not in _FP8_KV_DTYPES:
            raise ValueError("an FP8 cache (kv_scale given) must be float8_e4m3fn or uint8 codes")
        _need(kv_cache, "kv_cache", kv_cache.dtype, 3)
    else:
        _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    if kv_new.shape[-1] != D_QK or kv_cache.shape[2] != D_QK:
        raise ValueError(f"rows must be {D_QK} wide")
    n = kv_new.numel() // D_QK
    if slots.numel() != n or tuple(slots.shape) != tuple(kv_new.shape[:-1]):
        raise ValueError("slots must have one entry per row of kv_new")
    _same_device(kv_cache.device, kv_new=kv_new, slots=slots)
    if fp8:
        _check(lib.mla_kv_write_fp8(kv_new.data_ptr(), slots.data_ptr(), int(n), float(kv_scale), kv_cache.data_ptr(),
                                    int(kv_cache.shape[0]), int(kv_cache.shape[1]), _stream(kv_cache.device)))
    else:
        _check(lib.mla_kv_write(kv_new.data_ptr(), slots.data_ptr(), int(n), kv_cache.data_ptr(),
                                int(kv_cache.shape[0]), int(kv_cache.shape[1]), _stream(kv_cache.device)))
    return kv_cache


def mla_decode_varlen(q: torch.Tensor, query_start_loc: torch.Tensor, kv_cache: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor,
                      causal_seqlens_global: Optional[torch.Tensor] = None, cp_world: int = 1, cp_rank: int = 0,
                      causal: bool = True, scale: Optional[float] = None, lse_base: str = "e", *,
                      max_q_len: int, max_seq_len: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, return_lse: bool = True, cp_interleave: int = 1
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One rank's decode for requests with different query lengths: q [T, H, 576] bf16 packs the
    requests' tokens, request b owning tokens query_start_loc[b] .. query_start_loc[b+1]-1.
    Returns out [T, H, 512] bf16 and lse [T, H] float32.  max_q_len (keyword, required) is a
    host upper bound on every request's query length: it sizes the work split without reading
    query_start_loc back from the GPU, so the call never synchronises with the host."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    T, H, Dq = q.shape
    if Dq != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    B = int(query_start_loc.shape[0]) - 1
    if B < 0:
        raise ValueError("query_start_loc must have B+1 entries")
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have B rows")
    if causal_seqlens_global is not None:
        _need(causal_seqlens_global, "causal_seqlens_global", torch.int32, 1)
        if causal_seqlens_global.shape[0] != B:
            raise ValueError("causal_seqlens_global must have B entries")
    if max_q_len is None or int(max_q_len) < 1:
        raise ValueError("max_q_len (a host upper bound on the per-request query lengths) must be >= 1")
    max_q_len = int(max_q_len)
    num_blocks, bs = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    max_blocks = int(block_table.shape[1])
    if max_seq_len is None:
        max_seq_len = max_blocks * bs
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    base = {"e": LSE_BASE_E, "2": LSE_BASE_2}.get(str(lse_base))
    if base is None:
        raise ValueError("lse_base must be 'e' or '2'")
    dev = q.device
    _same_device(dev, query_start_loc=query_start_loc, kv_cache=kv_cache, block_table=block_table,
                 seq_lens=seq_lens, causal_seqlens_global=causal_seqlens_global, out=out, lse=lse,
                 workspace=workspace)
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (T, H, D_V):
            raise ValueError("out must be [T, H, 512]")
    if return_lse:
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        else:
            _need(lse, "lse", torch.float32, 2)
            if tuple(lse.shape) != (T, H):
                raise ValueError("lse must be [T, H]")
    ws_bytes = int(lib.mla_decode_workspace_size(max(B, 1), max_q_len, H, int(max_seq_len)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    _check(lib.mla_decode_varlen(
        q.data_ptr(), query_start_loc.data_ptr(), max_q_len, kv_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), causal_seqlens_global.data_ptr() if causal_seqlens_global is not None else None,
        B, H, num_blocks, bs, max_blocks, int(max_seq_len), int(cp_world), int(cp_rank), int(cp_interleave),
        1 if causal else 0, float(scale), base, out.data_ptr(),
        lse.data_ptr() if (return_lse and lse is not None) else None,
        workspace.data_ptr(), int(workspace.numel()), _stream(dev)))
    return out, (lse if return_lse else None)

