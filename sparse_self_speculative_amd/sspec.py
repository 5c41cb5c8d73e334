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
    "sspec_kv_pack_pages", "sspec_kv_unpack_pages",
    "sspec_offload_page_bytes", "sspec_offload_host_bytes", "sspec_offload_create", "sspec_offload_destroy",
    "sspec_offload_evict", "sspec_offload_restore", "sspec_offload_pump", "sspec_offload_poll",
    "sspec_offload_pending", "sspec_offload_trace",
    "sspec_unified_attn_slots", "sspec_kv_append_slots",
    "sspec_sched_create", "sspec_sched_destroy", "sspec_sched_admit", "sspec_sched_next",
    "sspec_sched_resolve", "sspec_sched_query", "sspec_accept_stub",
]
OFFLOAD_EVICT, OFFLOAD_RESTORE, OFFLOAD_DRY = 1, 2, 1


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
_lib.sspec_unified_attn_slots.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _P, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _c.c_double, _c.c_float, _P, _i32, _P, _P, _P,
                                          _P, _P, _sz, _P]
_lib.sspec_kv_append_slots.argtypes = [_c.POINTER(_PagedKV), _P, _P, _P, _P, _P, _i32, _i32, _i32, _P, _P]
_lib.sspec_sched_create.argtypes = [_i32, _i32, _i32, _c.POINTER(_P)]
_lib.sspec_sched_destroy.argtypes = [_P]
_lib.sspec_sched_admit.argtypes = [_P, _i32, _i32, _i32, _c.POINTER(_i32), _c.POINTER(_i32)]
_lib.sspec_sched_next.argtypes = [_P, _P, _P, _P, _c.POINTER(_i32), _c.POINTER(_i32), _c.POINTER(_i32),
                                  _c.POINTER(_i64), _P, _P]
_lib.sspec_sched_resolve.argtypes = [_P, _i64, _P, _P, _i32, _c.POINTER(_i32)]
_lib.sspec_sched_query.argtypes = [_P, _i32, _c.POINTER(_i32), _c.POINTER(_i32), _c.POINTER(_i32),
                                   _c.POINTER(_i32)]
_lib.sspec_accept_stub.argtypes = [_P, _P, _P, _i32, _i32, _i32, _i64, _c.c_double, _c.c_uint64, _i32, _P, _P]
_lib.sspec_kv_pack_pages.argtypes = [_c.POINTER(_PagedKV), _P, _i32, _P, _P, _P]
_lib.sspec_kv_unpack_pages.argtypes = [_c.POINTER(_PagedKV), _P, _i32, _P, _P, _P]
_lib.sspec_offload_page_bytes.restype = _sz
_lib.sspec_offload_page_bytes.argtypes = [_i32]
_lib.sspec_offload_host_bytes.restype = _sz
_lib.sspec_offload_host_bytes.argtypes = [_i32, _i32, _i32, _i64]
_lib.sspec_offload_create.argtypes = [_c.POINTER(_PagedKV), _i32, _i32, _P, _sz, _P, _sz, _P, _i32,
                                      _c.POINTER(_P)]
_lib.sspec_offload_destroy.argtypes = [_P]
_lib.sspec_offload_evict.argtypes = [_P, _i32, _c.POINTER(_i32), _i32]
_lib.sspec_offload_restore.argtypes = [_P, _i32, _c.POINTER(_i32), _i32]
_lib.sspec_offload_pump.argtypes = [_P, _P, _i32]
_lib.sspec_offload_poll.argtypes = [_P, _c.POINTER(_i32), _c.POINTER(_i32), _i32, _c.POINTER(_i32)]
_lib.sspec_offload_pending.argtypes = [_P, _c.POINTER(_i32), _c.POINTER(_i32), _c.POINTER(_i64)]
_lib.sspec_offload_trace.argtypes = [_P, _c.POINTER(_i32), _i32, _c.POINTER(_i32)]


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


def kv_pack_pages(kv: PagedKV, pages, dst, err=None, stream=None):
    """Gather whole pages (K and V blocks) into dst (see sspec_kv_pack_pages)."""
    st = kv._struct()
    _check(_lib.sspec_kv_pack_pages(ctypes.byref(st), _ptr(pages), int(pages.numel()), _ptr(dst), _ptr(err),
                                    _stream(stream)))


def kv_unpack_pages(kv: PagedKV, pages, src, err=None, stream=None):
    """Scatter a packed buffer back into pages (see sspec_kv_unpack_pages)."""
    st = kv._struct()
    _check(_lib.sspec_kv_unpack_pages(ctypes.byref(st), _ptr(pages), int(pages.numel()), _ptr(src), _ptr(err),
                                      _stream(stream)))


def offload_page_bytes(num_kv_heads) -> int:
    return int(_lib.sspec_offload_page_bytes(num_kv_heads))


def offload_host_bytes(num_kv_heads, chunk_pages, slots, host_pages) -> int:
    return int(_lib.sspec_offload_host_bytes(num_kv_heads, chunk_pages, slots, host_pages))


class Offload:
    """The KV offload engine (sspec_offload_*): FIFO evict / restore jobs of
    requests' pages, moved in chunks on a side stream.  The caller's buffers
    (staging on the device, a pinned host arena) are kept referenced here."""

    def __init__(self, kv, chunk_pages, slots, staging=None, host=None, side_stream=None, dry=False,
                 num_pages=None, num_kv_heads=None, host_pages=None):
        if dry:
            st = _PagedKV(None, None, None, num_pages, num_kv_heads, 128, 16, 1, 1)
            hb = offload_host_bytes(num_kv_heads, chunk_pages, slots, host_pages)
            args = (None, 0, None, hb, None, OFFLOAD_DRY)
        else:
            st = kv._struct()
            args = (_ptr(staging), staging.numel() * staging.element_size(), _ptr(host),
                    host.numel() * host.element_size(), ctypes.c_void_p(side_stream.cuda_stream), 0)
        self._keep = (kv, staging, host, side_stream)
        self._h = _P()
        _check(_lib.sspec_offload_create(ctypes.byref(st), chunk_pages, slots, *args, ctypes.byref(self._h)))

    def close(self):
        if self._h:
            h, self._h = self._h, _P()
            _check(_lib.sspec_offload_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(pages):
        a = (_i32 * len(pages))(*[int(x) for x in pages])
        return a, len(pages)

    def evict(self, req, pages):
        a, n = self._ids(pages)
        _check(_lib.sspec_offload_evict(self._h, req, a, n))

    def restore(self, req, pages):
        a, n = self._ids(pages)
        _check(_lib.sspec_offload_restore(self._h, req, a, n))

    def pump(self, max_chunks, after_event=None):
        ev = None if after_event is None else _P(after_event.cuda_event)
        _check(_lib.sspec_offload_pump(self._h, ev, max_chunks))

    def poll(self, cap=1024):
        reqs, kinds, n = (_i32 * cap)(), (_i32 * cap)(), _i32(0)
        _check(_lib.sspec_offload_poll(self._h, reqs, kinds, cap, ctypes.byref(n)))
        return [(reqs[i], kinds[i]) for i in range(n.value)]

    def pending(self):
        j, c, f = _i32(0), _i32(0), _i64(0)
        _check(_lib.sspec_offload_pending(self._h, ctypes.byref(j), ctypes.byref(c), ctypes.byref(f)))
        return j.value, c.value, f.value

    def trace(self):
        n = _i32(0)
        _check(_lib.sspec_offload_trace(self._h, None, 0, ctypes.byref(n)))
        buf = (_i32 * (4 * max(n.value, 1)))()
        _check(_lib.sspec_offload_trace(self._h, buf, n.value, ctypes.byref(n)))
        return [tuple(buf[4 * i: 4 * i + 4]) for i in range(n.value)]


def unified_attn_slots(kv: PagedKV, q, seq_ids, ctx_lens, bucket_ids, verify_bucket, num_items, max_verify,
                       max_ctx, num_q_heads, k, s, sm_scale, sel_idx, sel_stride, sel_count, sel_len, out, lse,
                       ws, stream=None):
    """sspec_unified_attn_slots: the unified launch with items naming request slots."""
    st = kv._struct()
    _check(_lib.sspec_unified_attn_slots(ctypes.byref(st), _ptr(q), _ptr(seq_ids), _ptr(ctx_lens),
                                         _ptr(bucket_ids), verify_bucket, num_items, max_verify, max_ctx,
                                         num_q_heads, k, s, sm_scale, _ptr(sel_idx), sel_stride, _ptr(sel_count),
                                         _ptr(sel_len), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream(stream)))


def kv_append_slots(kv: PagedKV, k_new, v_new, seq_ids, ctx_lens, bucket_ids, verify_bucket, num_items, k,
                    err=None, stream=None):
    st = kv._struct()
    _check(_lib.sspec_kv_append_slots(ctypes.byref(st), _ptr(k_new), _ptr(v_new), _ptr(seq_ids), _ptr(ctx_lens),
                                      _ptr(bucket_ids), verify_bucket, num_items, k, _ptr(err), _stream(stream)))


def accept_stub(req_ids, seq_ids, bucket_ids, verify_bucket, n_items, k, it, rate, seed, num_slots,
                accepted_by_slot, stream=None):
    _check(_lib.sspec_accept_stub(_ptr(req_ids), _ptr(seq_ids), _ptr(bucket_ids), verify_bucket, n_items, k, it,
                                  rate, seed, num_slots, _ptr(accepted_by_slot), _stream(stream)))


class Scheduler:
    """The unified batch scheduler with delayed verification (sspec_sched_*).
    Outputs land in caller-given int32 arrays (numpy or pinned torch CPU
    tensors): per item req_ids / seq_ids / bucket_ids, per slot ctx_lens /
    sel_len."""

    def __init__(self, k, max_slots, delayed=True):
        self.k, self.max_slots = k, max_slots
        self._h = _P()
        _check(_lib.sspec_sched_create(k, max_slots, int(bool(delayed)), ctypes.byref(self._h)))

    def close(self):
        if self._h:
            h, self._h = self._h, _P()
            _lib.sspec_sched_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, req_id, prompt_len, max_new):
        slot, bucket = _i32(0), _i32(0)
        _check(_lib.sspec_sched_admit(self._h, req_id, prompt_len, max_new, ctypes.byref(slot), ctypes.byref(bucket)))
        return slot.value, bucket.value

    @staticmethod
    def _addr(a):
        if a is None:
            return None
        if isinstance(a, torch.Tensor):
            assert a.dtype == torch.int32 and a.is_contiguous()
            return _P(a.data_ptr())
        import numpy as _np
        assert a.dtype == _np.int32 and a.flags["C_CONTIGUOUS"]
        return _P(a.ctypes.data)

    def next(self, req_ids, seq_ids, bucket_ids, ctx_lens, sel_len):
        """Form the next iteration: returns (iter, verify_bucket, n_items, n_verify)."""
        n, nv, vb, it = _i32(0), _i32(0), _i32(0), _i64(0)
        _check(_lib.sspec_sched_next(self._h, self._addr(req_ids), self._addr(seq_ids), self._addr(bucket_ids),
                                     ctypes.byref(n), ctypes.byref(nv), ctypes.byref(vb), ctypes.byref(it),
                                     self._addr(ctx_lens), self._addr(sel_len)))
        return it.value, vb.value, n.value, nv.value

    def resolve(self, it, accepted_by_slot, cap=1024):
        fin, n = (_i32 * cap)(), _i32(0)
        _check(_lib.sspec_sched_resolve(self._h, it, self._addr(accepted_by_slot), fin, cap, ctypes.byref(n)))
        return [fin[i] for i in range(min(n.value, cap))]

    def query(self, slot):
        rid, ctx, out, b = _i32(0), _i32(0), _i32(0), _i32(0)
        _check(_lib.sspec_sched_query(self._h, slot, ctypes.byref(rid), ctypes.byref(ctx), ctypes.byref(out),
                                      ctypes.byref(b)))
        return rid.value, ctx.value, out.value, b.value
