"""Host-side argument validation of the C ABI (include/sspec.h), without a GPU.

Every entry point validates its arguments before any HIP call, so these
cases run on a machine with no GPU: each bad argument must return its
status code and a message naming the problem, and the valid baseline must
pass validation and stop at the first HIP call (SSPEC_ERR_HIP, since there
is no device).  Pointers are fake, suitably aligned addresses: nothing is
ever dereferenced on the host.

Used by tests/test_abi.py in-process, and as a script
(python tests/abi_validation.py <library>) in a subprocess that loads an
AddressSanitizer / UndefinedBehaviorSanitizer build of the host code.
Pure ctypes: no torch, so the sanitizer runtime sees only this library.
"""

from __future__ import annotations

import ctypes as C
import math
import sys

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4

P, I32, I64, SZ, F32, F64 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float, C.c_double


class PagedKV(C.Structure):
    _fields_ = [("k_pages", P), ("v_pages", P), ("block_table", P), ("num_pages", I32),
                ("num_kv_heads", I32), ("head_dim", I32), ("page_size", I32),
                ("bt_stride", I32), ("num_seqs", I32)]


def bind(path):
    lib = C.CDLL(path)
    lib.sspec_last_error.restype = C.c_char_p
    lib.sspec_workspace_init.argtypes = [P, SZ, P]
    lib.sspec_read_device_error.argtypes = [P, C.c_int, P, C.POINTER(C.c_uint32)]
    lib.sspec_verify_attn.argtypes = [C.POINTER(PagedKV), P, P, P, I32, I32, I32, I32, F32, P, P, P,
                                      I64, P, SZ, P]
    lib.sspec_pillar_topk.argtypes = [P, P, I64, P, P, I32, I32, I32, I32, I32, I32, F64, P, I32, P,
                                      P, P, SZ, P]
    lib.sspec_sparse_draft_attn.argtypes = [C.POINTER(PagedKV), P, P, P, P, I32, P, P, I32, I32, I32,
                                            F32, P, P, P, SZ, P]
    lib.sspec_unified_attn.argtypes = [C.POINTER(PagedKV), P, P, P, I32, I32, I32, I32, I32, I32, F64,
                                       F32, P, I32, P, P, P, P, P, SZ, P]
    lib.sspec_unified_attn_naive.argtypes = lib.sspec_unified_attn.argtypes
    lib.sspec_kv_append.argtypes = [C.POINTER(PagedKV), P, P, P, P, I32, I32, I32, P, P]
    lib.sspec_kv_rollback.argtypes = [P, I32, P, I32, I32, P, P, P]
    lib.sspec_sched_create.argtypes = [I32, I32, I32, C.POINTER(P)]
    lib.sspec_sched_destroy.argtypes = [P]
    lib.sspec_sched_admit.argtypes = [P, I32, I32, I32, C.POINTER(I32), C.POINTER(I32)]
    lib.sspec_sched_next.argtypes = [P, P, P, P, C.POINTER(I32), C.POINTER(I32), C.POINTER(I32), C.POINTER(I64), P, P]
    lib.sspec_sched_resolve.argtypes = [P, I64, P, P, I32, C.POINTER(I32)]
    lib.sspec_offload_host_bytes.restype = SZ
    lib.sspec_offload_host_bytes.argtypes = [I32, I32, I32, I64]
    lib.sspec_offload_create.argtypes = [C.POINTER(PagedKV), I32, I32, P, SZ, P, SZ, P, I32, C.POINTER(P)]
    lib.sspec_offload_destroy.argtypes = [P]
    lib.sspec_offload_evict.argtypes = [P, I32, C.POINTER(I32), I32]
    lib.sspec_offload_restore.argtypes = [P, I32, C.POINTER(I32), I32]
    lib.sspec_offload_pump.argtypes = [P, P, I32]
    lib.sspec_offload_poll.argtypes = [P, C.POINTER(I32), C.POINTER(I32), I32, C.POINTER(I32)]
    for name, n in (("sspec_verify_workspace_size", 5), ("sspec_pillar_topk_workspace_size", 3),
                    ("sspec_draft_workspace_size", 4), ("sspec_unified_workspace_size", 6)):
        f = getattr(lib, name)
        f.restype = SZ
        f.argtypes = [I32] * n
    return lib


# fake device addresses: distinct, 256-byte aligned, never dereferenced
_A = iter(range(0x7f0000000000, 0x7f0000000000 + (1 << 30), 1 << 20))
ADDR = {n: next(_A) for n in ("k", "v", "bt", "q", "seq", "ctx", "out", "lse", "logits", "sel",
                              "cnt", "sl", "bk", "ws")}
WS_BYTES = 1 << 40   # "large enough" for every valid baseline


def kv(**kw):
    f = dict(k_pages=ADDR["k"], v_pages=ADDR["v"], block_table=ADDR["bt"], num_pages=1000,
             num_kv_heads=8, head_dim=128, page_size=16, bt_stride=300, num_seqs=64)
    f.update(kw)
    return PagedKV(**f)


# ------------------------------------------------------ baseline argument sets
def verify_args(**kw):
    a = dict(kv=kv(), q=ADDR["q"], seq=ADDR["seq"], ctx=ADDR["ctx"], n=4, max_ctx=4096, hq=32, k=8,
             scale=1 / math.sqrt(128), out=ADDR["out"], lse=ADDR["lse"], logits=ADDR["logits"],
             lstride=4096, ws=ADDR["ws"], ws_bytes=WS_BYTES)
    a.update(kw)
    return a


def call_verify(lib, a):
    k = a["kv"]
    return lib.sspec_verify_attn(None if k is None else C.byref(k), a["q"], a["seq"], a["ctx"], a["n"],
                                 a["max_ctx"], a["hq"], a["k"], a["scale"], a["out"], a["lse"],
                                 a["logits"], a["lstride"], a["ws"], a["ws_bytes"], None)


def topk_args(**kw):
    a = dict(logits=ADDR["logits"], lse=ADDR["lse"], lstride=4096, seq=ADDR["seq"], ctx=ADDR["ctx"],
             n=4, num_seqs=64, max_ctx=4096, hq=32, hkv=8, k=8, s=0.05, sel=ADDR["sel"],
             sel_stride=205, cnt=ADDR["cnt"], sl=ADDR["sl"], ws=ADDR["ws"], ws_bytes=WS_BYTES)
    a.update(kw)
    return a


def call_topk(lib, a):
    return lib.sspec_pillar_topk(a["logits"], a["lse"], a["lstride"], a["seq"], a["ctx"], a["n"],
                                 a["num_seqs"], a["max_ctx"], a["hq"], a["hkv"], a["k"], a["s"],
                                 a["sel"], a["sel_stride"], a["cnt"], a["sl"], a["ws"], a["ws_bytes"],
                                 None)


def draft_args(**kw):
    a = dict(kv=kv(), q=ADDR["q"], seq=ADDR["seq"], ctx=ADDR["ctx"], sel=ADDR["sel"], sel_stride=205,
             cnt=ADDR["cnt"], sl=ADDR["sl"], n=4, max_ctx=4096, hq=32, scale=1 / math.sqrt(128),
             out=ADDR["out"], lse=ADDR["lse"], ws=ADDR["ws"], ws_bytes=WS_BYTES)
    a.update(kw)
    return a


def call_draft(lib, a):
    k = a["kv"]
    return lib.sspec_sparse_draft_attn(None if k is None else C.byref(k), a["q"], a["seq"], a["ctx"],
                                       a["sel"], a["sel_stride"], a["cnt"], a["sl"], a["n"],
                                       a["max_ctx"], a["hq"], a["scale"], a["out"], a["lse"], a["ws"],
                                       a["ws_bytes"], None)


def unified_args(**kw):
    a = dict(kv=kv(), q=ADDR["q"], ctx=ADDR["ctx"], bk=ADDR["bk"], vb=0, num_seqs=64, max_verify=8,
             max_ctx=4096, hq=32, k=8, s=0.05, scale=1 / math.sqrt(128), sel=ADDR["sel"],
             sel_stride=205, cnt=ADDR["cnt"], sl=ADDR["sl"], out=ADDR["out"], lse=ADDR["lse"],
             ws=ADDR["ws"], ws_bytes=WS_BYTES)
    a.update(kw)
    return a


def call_unified(lib, a):
    k = a["kv"]
    return lib.sspec_unified_attn(None if k is None else C.byref(k), a["q"], a["ctx"], a["bk"], a["vb"],
                                  a["num_seqs"], a["max_verify"], a["max_ctx"], a["hq"], a["k"], a["s"],
                                  a["scale"], a["sel"], a["sel_stride"], a["cnt"], a["sl"], a["out"],
                                  a["lse"], a["ws"], a["ws_bytes"], None)


def call_naive(lib, a):
    k = a["kv"]
    return lib.sspec_unified_attn_naive(None if k is None else C.byref(k), a["q"], a["ctx"], a["bk"], a["vb"],
                                        a["num_seqs"], a["max_verify"], a["max_ctx"], a["hq"], a["k"], a["s"],
                                        a["scale"], a["sel"], a["sel_stride"], a["cnt"], a["sl"], a["out"],
                                        a["lse"], a["ws"], a["ws_bytes"], None)


def append_args(**kw):
    a = dict(kv=kv(), k_new=ADDR["q"], v_new=ADDR["out"], ctx=ADDR["ctx"], bk=ADDR["bk"], vb=0, num_seqs=64, k=8,
             err=None)
    a.update(kw)
    return a


def call_append(lib, a):
    k = a["kv"]
    return lib.sspec_kv_append(None if k is None else C.byref(k), a["k_new"], a["v_new"], a["ctx"], a["bk"], a["vb"],
                               a["num_seqs"], a["k"], a["err"], None)


def rollback_args(**kw):
    a = dict(bk=ADDR["bk"], vb=0, acc=ADDR["cnt"], num_seqs=64, k=8, ctx=ADDR["ctx"], sl=ADDR["sl"])
    a.update(kw)
    return a


def call_rollback(lib, a):
    return lib.sspec_kv_rollback(a["bk"], a["vb"], a["acc"], a["num_seqs"], a["k"], a["ctx"], a["sl"], None)


ENTRY = {"verify": (verify_args, call_verify), "topk": (topk_args, call_topk),
         "draft": (draft_args, call_draft), "unified": (unified_args, call_unified),
         "naive": (unified_args, call_naive),
         "append": (append_args, call_append), "rollback": (rollback_args, call_rollback)}

_KV_CASES = [  # (kv overrides, status, message fragment)
    (dict(k_pages=None), INVALID, "NULL"),
    (dict(block_table=None), INVALID, "NULL"),
    (dict(head_dim=64), UNSUPPORTED, "head_dim"),
    (dict(page_size=32), UNSUPPORTED, "page_size"),
    (dict(num_pages=0), INVALID, "sizes"),
    (dict(k_pages=ADDR["k"] + 8), INVALID, "aligned"),
    (dict(num_kv_heads=0), INVALID, ">= 1"),
    (dict(num_pages=1 << 28, num_kv_heads=8), UNSUPPORTED, "32 bits"),
]

_HEAD_CASES = [  # (hq, k, status, fragment) with num_kv_heads = 8
    (32, 17, UNSUPPORTED, "k must be"),
    (32, -1, UNSUPPORTED, "k must be"),
    (72, 8, UNSUPPORTED, "group size"),       # G = 9
    (36, 8, UNSUPPORTED, "multiple"),         # 36 / 8 not whole
    (64, 16, UNSUPPORTED, "G*(k+1)"),         # G = 8, 8 * 17 = 136 > 128
]


def cases():
    """(name, entry, argument overrides, expected status, message fragment)."""
    out = []
    for e in ("verify", "topk", "draft", "unified", "naive"):
        out.append((f"{e}: valid baseline reaches the device", e, {}, HIP, "hip"))
        out.append((f"{e}: max_ctx 0", e, dict(max_ctx=0), UNSUPPORTED, "max_ctx"))
        out.append((f"{e}: max_ctx 2^20+1", e, dict(max_ctx=(1 << 20) + 1), UNSUPPORTED, "max_ctx"))
        out.append((f"{e}: NULL workspace", e, dict(ws=None), WORKSPACE, "NULL"))
        out.append((f"{e}: misaligned workspace", e, dict(ws=ADDR["ws"] + 64), WORKSPACE, "aligned"))
        out.append((f"{e}: workspace too small", e, dict(ws_bytes=4096), WORKSPACE, "too small"))
        if e != "topk":
            out.append((f"{e}: kv NULL", e, dict(kv=None), INVALID, "NULL"))
            for ov, st, frag in _KV_CASES:
                out.append((f"{e}: kv {ov}", e, dict(kv=kv(**ov)), st, frag))
            out.append((f"{e}: sm_scale inf", e, dict(scale=float("inf")), INVALID, "sm_scale"))
            out.append((f"{e}: q NULL", e, dict(q=None), INVALID, "NULL"))
            out.append((f"{e}: out NULL", e, dict(out=None), INVALID, "NULL"))
            out.append((f"{e}: q misaligned", e, dict(q=ADDR["q"] + 2), INVALID, "aligned"))
        if e in ("verify", "unified", "naive"):
            for hq, k, st, frag in _HEAD_CASES:
                out.append((f"{e}: hq={hq} k={k}", e, dict(hq=hq, k=k), st, frag))
        if e == "topk":
            for hq, k, st, frag in _HEAD_CASES:
                out.append((f"{e}: hq={hq} k={k}", e, dict(hq=hq, k=k), st, frag))
            out.append((f"{e}: logits NULL", e, dict(logits=None), INVALID, "NULL"))
            out.append((f"{e}: num_seqs 0", e, dict(num_seqs=0), INVALID, "num_seqs"))
        if e in ("topk", "unified", "naive"):
            for s in (0.0, -0.1, 1.5, float("nan")):
                out.append((f"{e}: s={s}", e, dict(s=s), INVALID, "s must be"))
            out.append((f"{e}: sel_stride < ceil(s*max_ctx)", e, dict(sel_stride=204), INVALID, "sel_stride"))
        if e in ("verify", "topk"):
            out.append((f"{e}: logit_stride not a multiple of 16", e, dict(lstride=4100), INVALID, "logit_stride"))
            out.append((f"{e}: logit_stride < max_ctx", e, dict(lstride=4080), INVALID, "logit_stride"))
            out.append((f"{e}: n < 0", e, dict(n=-1), INVALID, ">= 0" if e == "verify" else "sizes"))
            out.append((f"{e}: n = 0 is a no-op", e, dict(n=0), OK, ""))
        if e == "verify":
            out.append((f"{e}: logits misaligned", e, dict(logits=ADDR["logits"] + 4), INVALID, "aligned"))
            out.append((f"{e}: lse NULL", e, dict(lse=None), INVALID, "NULL"))
        if e == "draft":
            out.append((f"{e}: n = 0 is a no-op", e, dict(n=0), OK, ""))
            out.append((f"{e}: sel_stride < 0", e, dict(sel_stride=-1), INVALID, "sizes"))
            out.append((f"{e}: sel_count NULL", e, dict(cnt=None), INVALID, "NULL"))
            out.append((f"{e}: lse NULL is allowed", e, dict(lse=None), HIP, "hip"))
        if e == "naive":
            # one tile shape for every item: only where the verify keeps its
            # query tiles in registers (G*(k+1) <= 48)
            out.append((f"{e}: G*(k+1) = 68", e, dict(hq=32, k=16), UNSUPPORTED, "naive"))
            out.append((f"{e}: G*(k+1) = 48 reaches the device", e, dict(hq=48, k=7), HIP, "hip"))
        if e in ("unified", "naive"):
            out.append((f"{e}: num_seqs 513", e, dict(num_seqs=513, kv=kv(num_seqs=600)), UNSUPPORTED, "num_seqs"))
            out.append((f"{e}: num_seqs 0", e, dict(num_seqs=0), UNSUPPORTED, "num_seqs"))
            out.append((f"{e}: num_seqs > kv rows", e, dict(num_seqs=65), INVALID, "kv->num_seqs"))
            out.append((f"{e}: max_verify < 0", e, dict(max_verify=-1), INVALID, "max_verify"))
            out.append((f"{e}: bucket_ids NULL", e, dict(bk=None), INVALID, "NULL"))
            out.append((f"{e}: lse NULL", e, dict(lse=None), INVALID, "NULL"))
    out += [
        ("append: valid baseline reaches the device", "append", {}, HIP, "hip"),
        ("append: kv NULL", "append", dict(kv=None), INVALID, "NULL"),
        ("append: head_dim 64", "append", dict(kv=kv(head_dim=64)), UNSUPPORTED, "head_dim"),
        ("append: page_size 32", "append", dict(kv=kv(page_size=32)), UNSUPPORTED, "page_size"),
        ("append: k 17", "append", dict(k=17), UNSUPPORTED, "k must be"),
        ("append: num_seqs > kv rows", "append", dict(num_seqs=65), INVALID, "num_seqs"),
        ("append: num_seqs < 0", "append", dict(num_seqs=-1), INVALID, "num_seqs"),
        ("append: num_seqs 0 is a no-op", "append", dict(num_seqs=0), OK, ""),
        ("append: k_new NULL", "append", dict(k_new=None), INVALID, "NULL"),
        ("append: v_new misaligned", "append", dict(v_new=ADDR["out"] + 8), INVALID, "aligned"),
        ("append: err may be given", "append", dict(err=ADDR["ws"]), HIP, "hip"),
        ("rollback: valid baseline reaches the device", "rollback", {}, HIP, "hip"),
        ("rollback: k -1", "rollback", dict(k=-1), UNSUPPORTED, "k must be"),
        ("rollback: accepted NULL", "rollback", dict(acc=None), INVALID, "NULL"),
        ("rollback: num_seqs < 0", "rollback", dict(num_seqs=-1), INVALID, "num_seqs"),
        ("rollback: num_seqs 0 is a no-op", "rollback", dict(num_seqs=0), OK, ""),
    ]
    return out


def run_cases(lib):
    """Run every case; return a list of failure descriptions (empty: all pass)."""
    fails = []
    for name, e, ov, want, frag in cases():
        mk, call = ENTRY[e]
        rc = call(lib, mk(**ov))
        msg = lib.sspec_last_error().decode()
        if rc != want or (want not in (OK, HIP) and frag.lower() not in msg.lower()):
            fails.append(f"{name}: got {rc} '{msg}', want {want} containing '{frag}'")
    # the other entry points of the ABI
    rc = lib.sspec_workspace_init(None, 1 << 20, None)
    if rc != WORKSPACE:
        fails.append(f"workspace_init(NULL): got {rc}")
    rc = lib.sspec_workspace_init(ADDR["ws"] + 16, 1 << 20, None)
    if rc != WORKSPACE or "aligned" not in lib.sspec_last_error().decode():
        fails.append(f"workspace_init(misaligned): got {rc}")
    rc = lib.sspec_workspace_init(ADDR["ws"], 512, None)
    if rc != WORKSPACE or "header" not in lib.sspec_last_error().decode():
        fails.append(f"workspace_init(too small): got {rc}")
    rc = lib.sspec_read_device_error(None, 0, None, None)
    if rc != INVALID:
        fails.append(f"read_device_error(NULL): got {rc}")
    fails += run_runtime_cases(lib)
    # workspace sizing: invalid shapes give 0, valid ones a positive size
    if not (lib.sspec_verify_workspace_size(4, 4096, 32, 8, 8) > 0
            and lib.sspec_verify_workspace_size(4, 0, 32, 8, 8) == 0
            and lib.sspec_unified_workspace_size(513, 8, 4096, 32, 8, 8) == 0
            and lib.sspec_draft_workspace_size(4, 4096, 4, 8) == 0):
        fails.append("workspace sizing")
    return fails


def run_runtime_cases(lib):
    """The host-only runtime (scheduler, offload planner) through a short
    session each, plus their argument checks: exercised under the sanitizers
    too."""
    fails = []
    h = P()
    if lib.sspec_sched_create(17, 4, 1, C.byref(h)) != UNSUPPORTED:
        fails.append("sched_create(k=17)")
    if lib.sspec_sched_create(3, 0, 1, C.byref(h)) != INVALID:
        fails.append("sched_create(max_slots=0)")
    if lib.sspec_sched_create(3, 6, 1, C.byref(h)) != OK:
        return fails + ["sched_create"]
    slot, b = I32(), I32()
    for r in range(5):
        if lib.sspec_sched_admit(h, r, 100 + r, 3, C.byref(slot), C.byref(b)) != OK or slot.value != r:
            fails.append(f"sched_admit {r}")
    arr = [(I32 * 6)() for _ in range(5)]
    acc = (I32 * 6)(*([1] * 6))
    fin = (I32 * 6)()
    n, nv, vb, it, nf = I32(), I32(), I32(), I64(), I32()
    for t in range(12):
        if lib.sspec_sched_next(h, arr[0], arr[1], arr[2], C.byref(n), C.byref(nv), C.byref(vb), C.byref(it),
                                arr[3], arr[4]) != OK:
            fails.append(f"sched_next t={t}: {lib.sspec_last_error().decode()}")
            break
        if t >= 1 and lib.sspec_sched_resolve(h, t - 1, acc, fin, 6, C.byref(nf)) != OK:
            fails.append(f"sched_resolve t={t}")
    if lib.sspec_sched_resolve(h, 3, acc, fin, 6, C.byref(nf)) != INVALID:
        fails.append("sched_resolve out of order")
    lib.sspec_sched_destroy(h)
    # the offload planner (planning-only mode: no device)
    e = P()
    hb = lib.sspec_offload_host_bytes(8, 4, 2, 64)
    k = kv(num_pages=200)
    if lib.sspec_offload_create(C.byref(k), 0, 2, None, 0, None, hb, None, 1, C.byref(e)) != INVALID:
        fails.append("offload_create(chunk 0)")
    if lib.sspec_offload_create(C.byref(k), 4, 2, None, 0, None, hb, None, 4, C.byref(e)) != INVALID:
        fails.append("offload_create(bad flags)")
    if lib.sspec_offload_create(C.byref(k), 4, 2, None, 0, None, hb, None, 0, C.byref(e)) != WORKSPACE:
        fails.append("offload_create(no staging)")
    if lib.sspec_offload_create(C.byref(k), 4, 2, None, 0, None, hb, None, 1, C.byref(e)) != OK:
        return fails + ["offload_create(dry)"]
    pages = (I32 * 40)(*range(40))
    for r in range(3):
        if lib.sspec_offload_evict(e, r, pages, 13 + r) != OK:
            fails.append(f"offload_evict {r}")
    if lib.sspec_offload_evict(e, 9, pages, 40) != WORKSPACE:
        fails.append("offload_evict(arena full)")
    if lib.sspec_offload_restore(e, 1, pages, 14) != OK:
        fails.append("offload_restore")
    reqs, kinds, nd = (I32 * 8)(), (I32 * 8)(), I32()
    got = []
    for _ in range(40):
        lib.sspec_offload_pump(e, None, 3)
        lib.sspec_offload_poll(e, reqs, kinds, 8, C.byref(nd))
        got += [(reqs[i], kinds[i]) for i in range(nd.value)]
    if got != [(0, 1), (1, 1), (2, 1), (1, 2)]:
        fails.append(f"offload order {got}")
    lib.sspec_offload_destroy(e)
    return fails


if __name__ == "__main__":
    f = run_cases(bind(sys.argv[1]))
    for x in f:
        print("FAIL", x)
    print(f"{len(cases())} cases, {len(f)} failures")
    sys.exit(1 if f else 0)
