"""Python binding of the SparseSpec attention C ABI (include/sspec.h).

Argument marshalling only: every step of the path runs in the HIP kernels
of libsspec.so.  torch supplies device memory and the stream.  There is no
fallback: if the library is missing this module raises at import time.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSPEC_LIB selects another build of the same library (e.g. a task-trace build)
LIB_PATH = os.environ.get("SSPEC_LIB") or os.path.join(_HERE, "libsspec.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python -m sparse_self_speculative_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

SSPEC_OK = 0
SSPEC_ERR_INVALID_ARG = 1
SSPEC_ERR_UNSUPPORTED = 2
SSPEC_ERR_WORKSPACE = 3
SSPEC_ERR_HIP = 4

DEV_ERR = {
    "CTX_RANGE": 0x1, "PAGE_RANGE": 0x2, "SEL_RANGE": 0x4, "VERIFY_SHORT": 0x8,
    "TOO_MANY_VERIFY": 0x10, "WAIT_TIMEOUT": 0x20, "SEQ_RANGE": 0x40, "LAYOUT": 0x80,
}

EXPORTED = [
    "sspec_last_error", "sspec_workspace_init", "sspec_read_device_error",
    "sspec_verify_workspace_size", "sspec_verify_attn",
    "sspec_pillar_topk_workspace_size", "sspec_pillar_topk", "sspec_pillar_topk_noalloc",
    "sspec_draft_workspace_size", "sspec_sparse_draft_attn",
    "sspec_unified_workspace_size", "sspec_unified_attn", "sspec_unified_attn_naive",
    "sspec_kv_append", "sspec_kv_rollback",
]


class _PagedKV(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("bt_stride", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32)]


_c = ctypes
_P = _c.c_void_p
_i32 = _c.c_int32
_i64 = _c.c_int64
_sz = _c.c_size_t

_lib.sspec_last_error.restype = _c.c_char_p
_lib.sspec_last_error.argtypes = []
_lib.sspec_workspace_init.argtypes = [_P, _sz, _P]
_lib.sspec_read_device_error.argtypes = [_P, _c.c_int, _P, _c.POINTER(_c.c_uint32)]
_lib.sspec_verify_workspace_size.restype = _sz
_lib.sspec_verify_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.sspec_verify_attn.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _i32, _i32, _i32, _i32,
                                   _c.c_float, _P, _P, _P, _i64, _P, _sz, _P]
_lib.sspec_pillar_topk_workspace_size.restype = _sz
_lib.sspec_pillar_topk_workspace_size.argtypes = [_i32, _i32, _i32]
_lib.sspec_pillar_topk.argtypes = [_P, _P, _i64, _P, _P, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _c.c_double, _P, _i32, _P, _P, _P, _sz, _P]
_lib.sspec_pillar_topk_noalloc.argtypes = [_P, _P, _i64, _P, _P, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _c.c_double, _P, _i32, _P, _P, _P]
_lib.sspec_draft_workspace_size.restype = _sz
_lib.sspec_draft_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
_lib.sspec_sparse_draft_attn.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _P, _i32, _P, _P,
                                         _i32, _i32, _i32, _c.c_float, _P, _P, _P, _sz, _P]
_lib.sspec_unified_workspace_size.restype = _sz
_lib.sspec_unified_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.sspec_unified_attn.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _c.c_double, _c.c_float, _P, _i32, _P, _P, _P,
                                    _P, _P, _sz, _P]
_lib.sspec_unified_attn_naive.argtypes = _lib.sspec_unified_attn.argtypes


_lib.sspec_kv_append.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _P, _i32, _i32, _i32, _P, _P]
_lib.sspec_kv_rollback.argtypes = [_P, _i32, _P, _i32, _i32, _P, _P, _P]


class SspecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sspec error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != SSPEC_OK:
        raise SspecError(rc, _lib.sspec_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class PagedKV:
    """A layer's paged KV cache: bf16 pools [num_pages][Hkv][16][128] and an
    int32 block table [num_seqs][bt_stride], all on the device."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor

    def _struct(self) -> _PagedKV:
        kp, bt = self.k_pages, self.block_table
        return _PagedKV(kp.data_ptr(), self.v_pages.data_ptr(), bt.data_ptr(), kp.shape[0],
                        kp.shape[1], kp.shape[3], kp.shape[2], bt.shape[1], bt.shape[0])


def workspace(nbytes: int, device="cuda", stream=None) -> torch.Tensor:
    """Allocate and clear a workspace of nbytes (uint8, device)."""
    ws = torch.empty(max(int(nbytes), 4096), dtype=torch.uint8, device=device)
    _check(_lib.sspec_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))
    return ws


def read_device_error(ws: torch.Tensor, clear: bool = True, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(_lib.sspec_read_device_error(_ptr(ws), int(clear), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def verify_workspace_size(n, max_ctx, num_q_heads, num_kv_heads, k) -> int:
    return int(_lib.sspec_verify_workspace_size(n, max_ctx, num_q_heads, num_kv_heads, k))


def pillar_topk_workspace_size(n, max_ctx, num_kv_heads) -> int:
    return int(_lib.sspec_pillar_topk_workspace_size(n, max_ctx, num_kv_heads))


def draft_workspace_size(n, max_ctx, num_q_heads, num_kv_heads) -> int:
    return int(_lib.sspec_draft_workspace_size(n, max_ctx, num_q_heads, num_kv_heads))


def unified_workspace_size(num_seqs, max_verify, max_ctx, num_q_heads, num_kv_heads, k) -> int:
    return int(_lib.sspec_unified_workspace_size(num_seqs, max_verify, max_ctx, num_q_heads,
                                                 num_kv_heads, k))


def dump_pitch(num_q_heads, num_kv_heads, k) -> int:
    """Rows per page block of the logit dump: round_up(G*(k+1), 4)."""
    m = (num_q_heads // num_kv_heads) * (k + 1)
    return (m + 3) // 4 * 4


def verify_attn(kv: PagedKV, q, seq_ids, ctx_lens, n, max_ctx, num_q_heads, k, sm_scale,
                out, lse, logits, logit_stride, ws, stream=None):
    s = kv._struct()
    _check(_lib.sspec_verify_attn(ctypes.byref(s), _ptr(q), _ptr(seq_ids), _ptr(ctx_lens), n,
                                  max_ctx, num_q_heads, k, sm_scale, _ptr(out), _ptr(lse),
                                  _ptr(logits), logit_stride, _ptr(ws), ws.numel(),
                                  _stream(stream)))


def pillar_topk(logits, lse, logit_stride, seq_ids, ctx_lens, n, num_seqs, max_ctx,
                num_q_heads, num_kv_heads, k, s, sel_idx, sel_stride, sel_count, sel_len,
                ws, stream=None):
    _check(_lib.sspec_pillar_topk(_ptr(logits), _ptr(lse), logit_stride, _ptr(seq_ids),
                                  _ptr(ctx_lens), n, num_seqs, max_ctx, num_q_heads,
                                  num_kv_heads, k, s, _ptr(sel_idx), sel_stride,
                                  _ptr(sel_count), _ptr(sel_len), _ptr(ws), ws.numel(),
                                  _stream(stream)))


def pillar_topk_noalloc(logits, lse, logit_stride, seq_ids, ctx_lens, n, num_seqs, max_ctx,
                        num_q_heads, num_kv_heads, k, s, sel_idx, sel_stride, sel_count, sel_len,
                        stream=None):
    """sspec_pillar_topk on the library's static scratch (no workspace)."""
    _check(_lib.sspec_pillar_topk_noalloc(_ptr(logits), _ptr(lse), logit_stride, _ptr(seq_ids),
                                          _ptr(ctx_lens), n, num_seqs, max_ctx, num_q_heads,
                                          num_kv_heads, k, s, _ptr(sel_idx), sel_stride,
                                          _ptr(sel_count), _ptr(sel_len), _stream(stream)))


def sparse_draft_attn(kv: PagedKV, q, seq_ids, ctx_lens, sel_idx, sel_stride, sel_count,
                      sel_len, n, max_ctx, num_q_heads, sm_scale, out, lse, ws, stream=None):
    st = kv._struct()
    _check(_lib.sspec_sparse_draft_attn(ctypes.byref(st), _ptr(q), _ptr(seq_ids),
                                        _ptr(ctx_lens), _ptr(sel_idx), sel_stride,
                                        _ptr(sel_count), _ptr(sel_len), n, max_ctx,
                                        num_q_heads, sm_scale, _ptr(out), _ptr(lse), _ptr(ws),
                                        ws.numel(), _stream(stream)))


def unified_attn(kv: PagedKV, q, ctx_lens, bucket_ids, verify_bucket, num_seqs, max_verify,
                 max_ctx, num_q_heads, k, s, sm_scale, sel_idx, sel_stride, sel_count,
                 sel_len, out, lse, ws, stream=None):
    st = kv._struct()
    _check(_lib.sspec_unified_attn(ctypes.byref(st), _ptr(q), _ptr(ctx_lens),
                                   _ptr(bucket_ids), verify_bucket, num_seqs, max_verify,
                                   max_ctx, num_q_heads, k, s, sm_scale, _ptr(sel_idx),
                                   sel_stride, _ptr(sel_count), _ptr(sel_len), _ptr(out),
                                   _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def unified_attn_naive(kv: PagedKV, q, ctx_lens, bucket_ids, verify_bucket, num_seqs, max_verify,
                       max_ctx, num_q_heads, k, s, sm_scale, sel_idx, sel_stride, sel_count,
                       sel_len, out, lse, ws, stream=None):
    """sspec_unified_attn_naive: the same launch with one tile shape for every item."""
    st = kv._struct()
    _check(_lib.sspec_unified_attn_naive(ctypes.byref(st), _ptr(q), _ptr(ctx_lens),
                                         _ptr(bucket_ids), verify_bucket, num_seqs, max_verify,
                                         max_ctx, num_q_heads, k, s, sm_scale, _ptr(sel_idx),
                                         sel_stride, _ptr(sel_count), _ptr(sel_len), _ptr(out),
                                         _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def kv_append(kv: PagedKV, k_new, v_new, ctx_lens, bucket_ids, verify_bucket, num_seqs, k,
              err=None, stream=None):
    """Write the iteration's new K/V rows into kv's pools (see sspec_kv_append)."""
    st = kv._struct()
    _check(_lib.sspec_kv_append(ctypes.byref(st), _ptr(k_new), _ptr(v_new), _ptr(ctx_lens),
                                _ptr(bucket_ids), verify_bucket, num_seqs, k, _ptr(err),
                                _stream(stream)))


def kv_rollback(bucket_ids, verify_bucket, accepted, num_seqs, k, ctx_lens, sel_len, stream=None):
    """Cut verifying requests back to their accepted tokens (see sspec_kv_rollback)."""
    _check(_lib.sspec_kv_rollback(_ptr(bucket_ids), verify_bucket, _ptr(accepted), num_seqs, k,
                                  _ptr(ctx_lens), _ptr(sel_len), _stream(stream)))
