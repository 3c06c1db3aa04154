"""Python binding of libpkv: paged K/V-cache attention on MI355X (gfx950).

Argument marshalling only.  Every step runs in the HIP kernels of
``libpkv.so`` (built in-tree by ``paged_kv_cache_slots_amd.build``); if the
library is missing, loading fails loudly.  Torch supplies device memory and
the current stream; the C entry points take plain pointers and sizes.

The functions carry the C names: ``pkv_scatter_slots``, ``pkv_attn_decode``,
``pkv_attn_prefill_block_causal``, ``pkv_merge_states`` and the workspace
size queries.  Any non-OK status raises :class:`PkvError`.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_DTYPE",
                4: "PKV_ERR_UNSUPPORTED", 5: "PKV_ERR_HIP", 6: "PKV_ERR_ALIGN", 7: "PKV_ERR_SCRATCH"}
PKV_F32, PKV_BF16, PKV_FP8_E4M3FN = 0, 1, 2

EXPORTED = ["pkv_status_string", "pkv_abi_version", "pkv_scatter_slots", "pkv_attn_decode_workspace_bytes",
            "pkv_attn_decode", "pkv_attn_prefill_workspace_bytes", "pkv_attn_prefill_block_causal",
            "pkv_merge_states", "pkv_rotate_rows", "pkv_copy_slots", "pkv_causal_layout_bounds",
            "pkv_window_evicted_tokens", "pkv_causal_layout", "pkv_attn_decode_step",
            "pkv_attn_decode_shared_prefix_workspace_bytes", "pkv_attn_decode_shared_prefix", "pkv_check_slots",
            "pkv_check_tables", "pkv_attn_decode_noalloc", "pkv_attn_prefill_block_causal_ragged",
            "pkv_set_timing_events", "pkv_xcd_ids", "pkv_attn_decode_append",
            "pkv_attn_decode_shared_prefix_append"]


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


class PkvCausalBounds(ctypes.Structure):
    _fields_ = [("fixed_pages", ctypes.c_int32), ("rolling_pages", ctypes.c_int32),
                ("private_pages", ctypes.c_int32), ("table_width", ctypes.c_int32), ("list_stride", ctypes.c_int32)]


class PkvPoolStruct(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("page_stride", ctypes.c_int64),
                ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpkv.so is not built ({path}); run `python -m paged_kv_cache_slots_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    PP = ctypes.POINTER(PkvPoolStruct)
    sig = {
        "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pkv_abi_version": (I32, []),
        "pkv_scatter_slots": (ctypes.c_int, [PP, P, P, I64, I64, P, P, P, I64, P]),
        "pkv_attn_decode_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "pkv_attn_decode": (ctypes.c_int, [PP, P, ctypes.c_int, I32, I32, I32, P, I32, P, I32, F32, P,
                                           ctypes.c_int, P, P, SZ, P]),
        "pkv_attn_decode_step": (ctypes.c_int, [PP, P, ctypes.c_int, I32, I32, I32, P, I32, P, I32, F32, P,
                                                ctypes.c_int, P, P, SZ, P]),
        "pkv_attn_decode_noalloc": (ctypes.c_int, [PP, P, ctypes.c_int, I32, I32, I32, P, I32, P, I32, F32, P,
                                                   ctypes.c_int, P, P]),
        "pkv_attn_decode_append": (ctypes.c_int, [PP, P, P, I64, I64, P, ctypes.c_int, I32, I32, I32, P, I32, P,
                                                  I32, F32, P, ctypes.c_int, P, P, SZ, P]),
        "pkv_attn_decode_shared_prefix_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "pkv_attn_decode_shared_prefix": (ctypes.c_int, [PP, P, ctypes.c_int, I32, I32, I32, I32, P, I32, P, I32, P,
                                                         I32, P, I32, F32, P, ctypes.c_int, P, P, SZ, P]),
        "pkv_attn_decode_shared_prefix_append": (ctypes.c_int, [PP, P, P, I64, I64, P, ctypes.c_int, I32, I32, I32,
                                                                I32, P, I32, P, I32, P, I32, P, I32, F32, P,
                                                                ctypes.c_int, P, P, SZ, P]),
        "pkv_check_slots": (ctypes.c_int, [PP, P, I64, P, P]),
        "pkv_check_tables": (ctypes.c_int, [PP, P, I32, P, I32, P, P]),
        "pkv_attn_prefill_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "pkv_attn_prefill_block_causal": (ctypes.c_int, [PP, P, ctypes.c_int, I64, I64, I32, I32, I32, P, I32, P,
                                                         P, I32, I32, F32, P, ctypes.c_int, P, P, SZ, P]),
        "pkv_attn_prefill_block_causal_ragged": (ctypes.c_int, [PP, P, ctypes.c_int, I64, I64, I32, I32, I32, P, P,
                                                                I32, P, P, I32, I32, F32, P, ctypes.c_int, P, P, SZ,
                                                                P]),
        "pkv_merge_states": (ctypes.c_int, [P, P, I32, I64, I32, I32, P, ctypes.c_int, P, P]),
        "pkv_set_timing_events": (None, [P, P]),
        "pkv_xcd_ids": (ctypes.c_int, [P, I32, I32, P]),
        "pkv_rotate_rows": (ctypes.c_int, [P, I64, I64, I64, I32, I64, P]),
        "pkv_copy_slots": (ctypes.c_int, [PP, I32, I64, P, P, I64, P]),
        "pkv_causal_layout_bounds": (ctypes.c_int, [I32, I64, I64, P, I32, ctypes.POINTER(PkvCausalBounds)]),
        "pkv_window_evicted_tokens": (I64, [I32, I64, I64, I64]),
        "pkv_causal_layout": (ctypes.c_int, [P, I32, P, I32, I32, I64, I64, I64, I64, P, I32, P, I32, P, P, P, P,
                                             P, P, P, P, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != PKV_OK:
        text = load_library().pkv_status_string(status).decode()
        raise PkvError(fn, status, text)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PKV_F32
    if t == torch.bfloat16:
        return PKV_BF16
    if t in (torch.float8_e4m3fn, torch.uint8):
        return PKV_FP8_E4M3FN
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


@dataclass
class Pool:
    """A K/V page pool: ``k`` and ``v`` are ``[num_pages, page_size, Hkv, D]``
    views (the page dimension may be strided); fp8 pools carry float scales
    ``[num_pages, Hkv]``."""
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    def struct(self) -> PkvPoolStruct:
        k, v = self.k, self.v
        if k.shape != v.shape or k.dtype != v.dtype or k.stride() != v.stride():
            raise ValueError("K and V pools must have the same shape, dtype and strides")
        n, ps, hkv, d = k.shape
        if k.stride()[1:] != (hkv * d, d, 1):
            raise ValueError("each page must be contiguous [page_size, Hkv, D]")
        return PkvPoolStruct(k.data_ptr(), v.data_ptr(), k.stride(0), n, ps, hkv, d, _dtype_code(k.dtype),
                             _ptr(self.k_scale), _ptr(self.v_scale))


def pkv_scatter_slots(pool: Pool, src_k: torch.Tensor, src_v: torch.Tensor, slots: torch.Tensor,
                      src_idx: Optional[torch.Tensor] = None, slots2: Optional[torch.Tensor] = None,
                      n_tokens: Optional[int] = None, stream=None) -> None:
    """Write ``src_k/src_v`` token rows ([n_src, Hkv, D] views, any token and
    head stride, D contiguous) into the pool at int64 ``slots`` (and
    ``slots2``); negative slots are skipped."""
    if src_k.stride() != src_v.stride() or src_k.stride(2) != 1:
        raise ValueError("src_k and src_v must share strides with D contiguous")
    n = slots.numel() if n_tokens is None else n_tokens
    ps = pool.struct()
    _check("pkv_scatter_slots", load_library().pkv_scatter_slots(
        ctypes.byref(ps), src_k.data_ptr(), src_v.data_ptr(), src_k.stride(0), src_k.stride(1), _ptr(src_idx),
        slots.data_ptr(), _ptr(slots2), n, _stream(stream)))


def pkv_attn_decode_workspace_bytes(num_tables: int, rows_per_table: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, max_kv_len: int) -> int:
    return int(load_library().pkv_attn_decode_workspace_bytes(num_tables, rows_per_table, num_q_heads,
                                                              num_kv_heads, head_dim, max_kv_len))


def pkv_attn_decode(pool: Pool, q: torch.Tensor, block_table: torch.Tensor, kv_lens: torch.Tensor, max_kv_len: int,
                    sm_scale: float, out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Paged decode.  ``q`` is [T, n, Hq, D] contiguous; ``out`` likewise
    (fp32 or bf16); ``out_lse`` [T, n, Hq] fp32 or None."""
    if not q.is_contiguous() or not out.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("q, out and block_table must be contiguous")
    t, n, hq, _ = q.shape
    ps = pool.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_attn_decode", load_library().pkv_attn_decode(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), t, n, hq, block_table.data_ptr(),
        block_table.stride(0), kv_lens.data_ptr(), int(max_kv_len), float(sm_scale), out.data_ptr(),
        _dtype_code(out.dtype), _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def pkv_attn_decode_noalloc(pool: Pool, q: torch.Tensor, block_table: torch.Tensor, kv_lens: torch.Tensor,
                            max_kv_len: int, sm_scale: float, out: torch.Tensor,
                            out_lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Paged decode that allocates nothing: as ``pkv_attn_decode`` with the
    cross-workgroup state in the library's per-device scratch array.  Calls
    that can overlap on one GPU race on that array."""
    if not q.is_contiguous() or not out.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("q, out and block_table must be contiguous")
    t, n, hq, _ = q.shape
    ps = pool.struct()
    _check("pkv_attn_decode_noalloc", load_library().pkv_attn_decode_noalloc(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), t, n, hq, block_table.data_ptr(),
        block_table.stride(0), kv_lens.data_ptr(), int(max_kv_len), float(sm_scale), out.data_ptr(),
        _dtype_code(out.dtype), _ptr(out_lse), _stream(stream)))


def pkv_attn_decode_step(pool: Pool, q: torch.Tensor, block_table: torch.Tensor, kv_lens: torch.Tensor,
                         max_kv_len: int, sm_scale: float, out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode of a multi-token step.  ``q`` is [T, q_len, Hq, D] contiguous:
    the q_len tokens of row t are its last q_len keys, token j attending keys
    [0, kv_lens[t] - (q_len - 1 - j)).  ``out`` / ``out_lse`` as pkv_attn_decode."""
    if not q.is_contiguous() or not out.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("q, out and block_table must be contiguous")
    t, n, hq, _ = q.shape
    ps = pool.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_attn_decode_step", load_library().pkv_attn_decode_step(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), t, n, hq, block_table.data_ptr(),
        block_table.stride(0), kv_lens.data_ptr(), int(max_kv_len), float(sm_scale), out.data_ptr(),
        _dtype_code(out.dtype), _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def pkv_attn_decode_append(pool: Pool, new_k: torch.Tensor, new_v: torch.Tensor, q: torch.Tensor,
                           block_table: torch.Tensor, kv_lens: torch.Tensor, max_kv_len: int, sm_scale: float,
                           out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write a step's K/V and attend: ``new_k`` / ``new_v`` [T * q_len, Hkv, D]
    (or [T, q_len, Hkv, D]) in the pool's element type, rows of D contiguous;
    token j of row t becomes key kv_lens[t] - q_len + j, then as
    ``pkv_attn_decode_step`` with ``q`` [T, q_len, Hq, D]."""
    if not q.is_contiguous() or not out.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("q, out and block_table must be contiguous")
    t, n, hq, d = q.shape
    hkv = pool.k.shape[-2]
    nk, nv = new_k.reshape(-1, hkv, d), new_v.reshape(-1, hkv, d)
    if nk.shape[0] != t * n or nv.shape != nk.shape or nk.stride() != nv.stride() or nk.stride(2) != 1:
        raise ValueError("new_k / new_v must be [T * q_len, Hkv, D] with matching strides and contiguous rows")
    if nk.element_size() != pool.k.element_size():
        raise ValueError("new_k / new_v must have the pool's element type")
    ps = pool.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_attn_decode_append", load_library().pkv_attn_decode_append(
        ctypes.byref(ps), nk.data_ptr(), nv.data_ptr(), nk.stride(0), nk.stride(1), q.data_ptr(),
        _dtype_code(q.dtype), t, n, hq, block_table.data_ptr(), block_table.stride(0), kv_lens.data_ptr(),
        int(max_kv_len), float(sm_scale), out.data_ptr(), _dtype_code(out.dtype), _ptr(out_lse), _ptr(workspace),
        ws_bytes, _stream(stream)))


def pkv_attn_decode_shared_prefix_workspace_bytes(groups: int, samples: int, q_len: int, num_q_heads: int,
                                                  head_dim: int, max_prefix_len: int) -> int:
    return load_library().pkv_attn_decode_shared_prefix_workspace_bytes(groups, samples, q_len, num_q_heads, head_dim,
                                                                         max_prefix_len)


def pkv_attn_decode_shared_prefix(pool: Pool, q: torch.Tensor, samples: int, prefix_table: torch.Tensor,
                                  prefix_lens: torch.Tensor, max_prefix_len: int, tail_table: torch.Tensor,
                                  tail_lens: torch.Tensor, max_tail_len: int, sm_scale: float, out: torch.Tensor,
                                  workspace: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                                  stream=None) -> None:
    """One n-sample step: ``q`` [groups * samples, q_len, Hq, D] bf16; sample r
    attends its group's prefix and its own tail, the step's q_len tokens being
    the tail's last keys (causal among themselves)."""
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    if not prefix_table.is_contiguous() or not tail_table.is_contiguous():
        raise ValueError("tables must be contiguous")
    rows, q_len, hq, _ = q.shape
    if rows % samples:
        raise ValueError("q rows must be groups * samples")
    ps = pool.struct()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("pkv_attn_decode_shared_prefix", load_library().pkv_attn_decode_shared_prefix(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), rows // samples, samples, q_len, hq,
        prefix_table.data_ptr(), prefix_table.stride(0), prefix_lens.data_ptr(), int(max_prefix_len),
        tail_table.data_ptr(), tail_table.stride(0), tail_lens.data_ptr(), int(max_tail_len), float(sm_scale),
        out.data_ptr(), _dtype_code(out.dtype), _ptr(out_lse), workspace.data_ptr(), ws_bytes, _stream(stream)))


def pkv_attn_decode_shared_prefix_append(pool: Pool, new_k: torch.Tensor, new_v: torch.Tensor, q: torch.Tensor,
                                         samples: int, prefix_table: torch.Tensor, prefix_lens: torch.Tensor,
                                         max_prefix_len: int, tail_table: torch.Tensor, tail_lens: torch.Tensor,
                                         max_tail_len: int, sm_scale: float, out: torch.Tensor,
                                         workspace: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                                         stream=None) -> None:
    """Write the step's K/V into the tails and run the n-sample step:
    ``new_k`` / ``new_v`` [groups * samples * q_len, Hkv, D] (or
    [groups * samples, q_len, Hkv, D]) in the pool's element type, rows of D
    contiguous; token j of sample r becomes tail key tail_lens[r] - q_len + j,
    then as ``pkv_attn_decode_shared_prefix``."""
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    if not prefix_table.is_contiguous() or not tail_table.is_contiguous():
        raise ValueError("tables must be contiguous")
    rows, q_len, hq, d = q.shape
    if rows % samples:
        raise ValueError("q rows must be groups * samples")
    hkv = pool.k.shape[-2]
    nk, nv = new_k.reshape(-1, hkv, d), new_v.reshape(-1, hkv, d)
    if nk.shape[0] != rows * q_len or nv.shape != nk.shape or nk.stride() != nv.stride() or nk.stride(2) != 1:
        raise ValueError("new_k / new_v must be [groups * samples * q_len, Hkv, D] with matching strides and "
                         "contiguous rows")
    if nk.element_size() != pool.k.element_size():
        raise ValueError("new_k / new_v must have the pool's element type")
    ps = pool.struct()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("pkv_attn_decode_shared_prefix_append", load_library().pkv_attn_decode_shared_prefix_append(
        ctypes.byref(ps), nk.data_ptr(), nv.data_ptr(), nk.stride(0), nk.stride(1), q.data_ptr(),
        _dtype_code(q.dtype), rows // samples, samples, q_len, hq, prefix_table.data_ptr(), prefix_table.stride(0),
        prefix_lens.data_ptr(), int(max_prefix_len), tail_table.data_ptr(), tail_table.stride(0),
        tail_lens.data_ptr(), int(max_tail_len), float(sm_scale), out.data_ptr(), _dtype_code(out.dtype),
        _ptr(out_lse), workspace.data_ptr(), ws_bytes, _stream(stream)))


def pkv_attn_prefill_workspace_bytes(batch: int, s_q: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                     max_keys: int) -> int:
    return int(load_library().pkv_attn_prefill_workspace_bytes(batch, s_q, num_q_heads, num_kv_heads, head_dim,
                                                               max_keys))


def pkv_attn_prefill_block_causal(pool: Pool, q: torch.Tensor, block_table: torch.Tensor, n_ctx: torch.Tensor,
                                  seq_len: torch.Tensor, causal_block_size: int, max_keys: int, sm_scale: float,
                                  out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Block-causal prefill.  ``q`` is a [B, s_q, Hq, D] view whose rows are
    ``q_tok_stride`` apart (batch rows consecutive) and heads
    ``q_head_stride`` apart, D contiguous (a slice of a packed QKV works)."""
    b, s_q, hq, d = q.shape
    if q.stride(3) != 1 or (b > 1 and q.stride(0) != s_q * q.stride(1)):
        raise ValueError("q rows must be evenly strided across the batch with D contiguous")
    if not out.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("out and block_table must be contiguous")
    ps = pool.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_attn_prefill_block_causal", load_library().pkv_attn_prefill_block_causal(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), q.stride(1), q.stride(2), b, s_q, hq,
        block_table.data_ptr(), block_table.stride(0), n_ctx.data_ptr(), seq_len.data_ptr(),
        int(causal_block_size), int(max_keys), float(sm_scale), out.data_ptr(), _dtype_code(out.dtype),
        _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def pkv_attn_prefill_block_causal_ragged(pool: Pool, q: torch.Tensor, q_offsets: torch.Tensor,
                                         block_table: torch.Tensor, n_ctx: torch.Tensor, seq_len: torch.Tensor,
                                         causal_block_size: int, max_rows: int, max_keys: int, sm_scale: float,
                                         out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
                                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Block-causal prefill over a ragged batch.  ``q`` is a [T, Hq, D] view
    (rows ``q_tok_stride`` apart, heads ``q_head_stride`` apart, D contiguous);
    batch entry b owns rows ``q_offsets[b] .. q_offsets[b + 1] - 1`` (device
    int32 [B + 1]); ``out`` is [T, Hq, D] contiguous, ``out_lse`` [T, Hq]."""
    t, hq, d = q.shape
    if q.stride(2) != 1:
        raise ValueError("q must have D contiguous")
    if not out.is_contiguous() or not block_table.is_contiguous() or q_offsets.dtype != torch.int32:
        raise ValueError("out and block_table must be contiguous; q_offsets int32")
    b = q_offsets.numel() - 1
    ps = pool.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_attn_prefill_block_causal_ragged", load_library().pkv_attn_prefill_block_causal_ragged(
        ctypes.byref(ps), q.data_ptr(), _dtype_code(q.dtype), q.stride(0), q.stride(1), b, int(max_rows), hq,
        q_offsets.data_ptr(), block_table.data_ptr(), block_table.stride(0), n_ctx.data_ptr(), seq_len.data_ptr(),
        int(causal_block_size), int(max_keys), float(sm_scale), out.data_ptr(), _dtype_code(out.dtype),
        _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def pkv_set_timing_events(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]) -> None:
    """While set, a call's main kernel (not its merge kernel) is launched with
    ``start`` / ``stop``, which then hold that kernel's own start and end
    times; None, None turns it off.  The events must have been created (e.g.
    recorded once) before the call."""
    lib = load_library()
    lib.pkv_set_timing_events(None if start is None else start.cuda_event, None if stop is None else stop.cuda_event)


def pkv_merge_states(o_parts: torch.Tensor, lse_parts: torch.Tensor, out: torch.Tensor,
                     out_lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Merge ``o_parts`` [N, R, Hq, D] / ``lse_parts`` [N, R, Hq] (fp32,
    contiguous) into ``out`` [R, Hq, D] (fp32 or bf16) and ``out_lse``."""
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous() and out.is_contiguous()):
        raise ValueError("merge inputs and output must be contiguous")
    n, r, hq, d = o_parts.shape
    _check("pkv_merge_states", load_library().pkv_merge_states(
        o_parts.data_ptr(), lse_parts.data_ptr(), n, r, hq, d, out.data_ptr(), _dtype_code(out.dtype),
        _ptr(out_lse), _stream(stream)))


def pkv_rotate_rows(rows: torch.Tensor, shift: int, stream=None) -> None:
    """Rotate every row of ``rows`` in place: element c takes the old element
    (c + shift) mod cols.  ``rows`` is 1-D (one row) or 2-D with contiguous
    elements inside a row (any row stride); element size 1, 2, 4, 8 or 16."""
    t = rows if rows.dim() == 2 else rows.view(1, -1)
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("rows must be 1-D or 2-D with contiguous elements within a row")
    n_rows, cols = t.shape
    row_stride = t.stride(0) if n_rows > 1 else cols
    _check("pkv_rotate_rows", load_library().pkv_rotate_rows(
        t.data_ptr() if t.numel() else None, n_rows, cols, row_stride, t.element_size(), int(shift),
        _stream(stream)))


def pkv_copy_slots(pool: Pool, src_slots: torch.Tensor, dst_slots: torch.Tensor, num_layers: int = 1,
                   layer_stride: int = 0, stream=None) -> None:
    """Copy whole key rows (every kv head, K and V) from int64 slots
    ``src_slots`` to ``dst_slots`` in each of ``num_layers`` layers of the
    pool (layer l starts ``layer_stride`` elements after layer l-1); entries
    with a negative slot are skipped."""
    if src_slots.numel() != dst_slots.numel():
        raise ValueError("src_slots and dst_slots must have the same length")
    ps = pool.struct()
    _check("pkv_copy_slots", load_library().pkv_copy_slots(
        ctypes.byref(ps), num_layers, layer_stride, src_slots.data_ptr(), dst_slots.data_ptr(), src_slots.numel(),
        _stream(stream)))


def _host_block_sizes(block_sizes):
    sizes = [int(v) for v in block_sizes]
    return (ctypes.c_int32 * max(1, len(sizes)))(*sizes), len(sizes)


def pkv_causal_layout_bounds(page_size: int, pin_tokens: int, window_tokens: int, block_sizes) -> dict:
    """Table, private-page and list sizes an exact-window geometry needs."""
    arr, n = _host_block_sizes(block_sizes)
    out = PkvCausalBounds()
    _check("pkv_causal_layout_bounds", load_library().pkv_causal_layout_bounds(
        page_size, pin_tokens, window_tokens, arr, n, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in PkvCausalBounds._fields_}


def pkv_window_evicted_tokens(page_size: int, pin_tokens: int, window_tokens: int, committed: int) -> int:
    """Rolling tokens (whole pages) that no block after ``committed`` can see."""
    v = load_library().pkv_window_evicted_tokens(page_size, pin_tokens, window_tokens, committed)
    if v < 0:
        raise ValueError("bad geometry")
    return v


class CausalLayout:
    """Device tensors of one exact-window geometry, written in place by
    ``pkv_causal_layout`` (fixed addresses across commits)."""

    def __init__(self, page_size: int, pin_tokens: int, window_tokens: int, block_sizes, device="cuda"):
        self.page_size, self.pin_tokens, self.window_tokens = page_size, pin_tokens, window_tokens
        self.block_sizes = [int(v) for v in block_sizes]
        self.bounds = pkv_causal_layout_bounds(page_size, pin_tokens, window_tokens, self.block_sizes)
        nb, total = len(self.block_sizes), sum(self.block_sizes)
        i32, i64 = dict(dtype=torch.int32, device=device), dict(dtype=torch.int64, device=device)
        self.block_tables = torch.empty((nb, self.bounds["table_width"]), **i32)
        self.n_ctx = torch.empty(nb, **i32)
        self.seq_len = torch.empty(nb, **i32)
        self.stage_slots = torch.empty(total, **i64)
        self.stage_slots2 = torch.empty(total, **i64)
        ls = nb * self.bounds["list_stride"]
        self.commit_src, self.commit_dst = torch.empty(ls, **i64), torch.empty(ls, **i64)
        self.current_src, self.current_dst = torch.empty(ls, **i64), torch.empty(ls, **i64)


def pkv_causal_layout(layout: CausalLayout, table: torch.Tensor, private_pages: torch.Tensor, committed: int,
                      evicted: int, stream=None) -> None:
    """Rewrite ``layout``'s tensors from the int32 page table of the sequence
    and the int32 [num_blocks, P] private pages of its causal blocks."""
    if table.dtype != torch.int32 or private_pages.dtype != torch.int32 or private_pages.dim() != 2:
        raise ValueError("table and private_pages must be int32; private_pages [num_blocks, P]")
    if not table.is_contiguous() or private_pages.stride(1) != 1:
        raise ValueError("table and private_pages rows must be contiguous")
    arr, n = _host_block_sizes(layout.block_sizes)
    L = layout
    _check("pkv_causal_layout", load_library().pkv_causal_layout(
        table.data_ptr(), table.numel(), private_pages.data_ptr(), private_pages.stride(0), L.page_size,
        L.pin_tokens, L.window_tokens, committed, evicted, arr, n, L.block_tables.data_ptr(),
        L.block_tables.shape[1], L.n_ctx.data_ptr(), L.seq_len.data_ptr(), L.stage_slots.data_ptr(),
        L.stage_slots2.data_ptr(), L.commit_src.data_ptr(), L.commit_dst.data_ptr(), L.current_src.data_ptr(),
        L.current_dst.data_ptr(), L.bounds["list_stride"], _stream(stream)))


def pkv_check_slots(pool: Pool, slots: torch.Tensor, stream=None) -> torch.Tensor:
    """Device int32 tensor [1]: how many int64 ``slots`` point past the pool
    (negative sentinels are valid).  Asynchronous; read it after a sync."""
    bad = torch.empty(1, dtype=torch.int32, device=slots.device)
    ps = pool.struct()
    _check("pkv_check_slots", load_library().pkv_check_slots(ctypes.byref(ps), slots.data_ptr(), slots.numel(),
                                                             bad.data_ptr(), _stream(stream)))
    return bad


def pkv_xcd_ids(num_workgroups: int, threads: int = 64, device: str = "cuda:0", stream=None) -> torch.Tensor:
    """Device int32 tensor [num_workgroups]: the XCC_ID hardware register
    (the XCD in its low 4 bits) each workgroup of a launch of that shape ran
    on.  Asynchronous; read it after a sync."""
    out = torch.empty(max(0, int(num_workgroups)), dtype=torch.int32, device=device)
    _check("pkv_xcd_ids", load_library().pkv_xcd_ids(out.data_ptr() if out.numel() else None, int(num_workgroups),
                                                     int(threads), _stream(stream)))
    return out


def pkv_check_tables(pool: Pool, block_table: torch.Tensor, kv_lens: torch.Tensor, stream=None) -> torch.Tensor:
    """Device int32 tensor [1]: how many table rows have a length or a used
    page id that would read outside the pool."""
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [rows, width] with contiguous rows")
    bad = torch.empty(1, dtype=torch.int32, device=block_table.device)
    ps = pool.struct()
    _check("pkv_check_tables", load_library().pkv_check_tables(
        ctypes.byref(ps), block_table.data_ptr(), block_table.stride(0), kv_lens.data_ptr(), block_table.shape[0],
        bad.data_ptr(), _stream(stream)))
    return bad
