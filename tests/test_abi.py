"""The C ABI without a GPU: the built library loads and exports every function
that include/sspec.h declares, the Python binding covers the same set, and
the host-side workspace sizing follows the header's rules (sizes grow with
the problem, invalid arguments give 0).  No kernel is launched."""
import ctypes
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sspec.h")
LIB = os.path.join(ROOT, "sparse_self_speculative_amd", "libsspec.so")
I32 = ctypes.c_int32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)   # comments mention names too
    return sorted(set(re.findall(r"\b(?:const\s+char\s*\*|int|size_t)\s+(sspec_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):   # nothing built yet: build it (hipcc cross-compiles without a GPU)
        import sys
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def sized(lib, name, nargs):
    f = getattr(lib, name)
    f.restype = ctypes.c_size_t
    f.argtypes = [I32] * nargs
    return f


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("sspec_verify_attn", "sspec_pillar_topk", "sspec_sparse_draft_attn", "sspec_unified_attn",
              "sspec_verify_workspace_size", "sspec_pillar_topk_workspace_size", "sspec_draft_workspace_size",
              "sspec_unified_workspace_size", "sspec_workspace_init", "sspec_read_device_error",
              "sspec_last_error"):
        assert n in names, n


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in sspec.h but not exported: {missing}"


def test_binding_covers_the_header():
    from sparse_self_speculative_amd import sspec as S
    assert sorted(S.EXPORTED) == declared_functions()
    for py in ("verify_attn", "pillar_topk", "sparse_draft_attn", "unified_attn", "verify_workspace_size",
               "pillar_topk_workspace_size", "draft_workspace_size", "unified_workspace_size", "workspace",
               "read_device_error"):
        assert callable(getattr(S, py)), py


def test_last_error_is_a_string(lib):
    f = lib.sspec_last_error
    f.restype = ctypes.c_char_p
    assert isinstance(f(), bytes)


def test_workspace_sizes(lib):
    uni = sized(lib, "sspec_unified_workspace_size", 6)   # num_seqs, max_verify, max_ctx, hq, hkv, k
    base = uni(128, 16, 32776, 32, 8, 8)
    assert base > 0
    assert uni(128, 16, 65536, 32, 8, 8) > base           # longer contexts
    assert uni(256, 32, 32776, 32, 8, 8) > base           # more requests
    assert uni(128, 16, 32776, 32, 8, 16) > base          # more verify queries
    for bad in ((0, 16, 32776, 32, 8, 8), (128, -1, 32776, 32, 8, 8), (128, 16, 0, 32, 8, 8),
                (128, 16, 32776, 4, 8, 8), (128, 16, 32776, 32, 0, 8), (128, 16, 32776, 32, 8, -1)):
        assert uni(*bad) == 0, bad

    ver = sized(lib, "sspec_verify_workspace_size", 5)    # n, max_ctx, hq, hkv, k
    assert ver(16, 4096, 32, 8, 8) > ver(8, 4096, 32, 8, 8) > 0
    assert ver(-1, 4096, 32, 8, 8) == 0 and ver(8, 0, 32, 8, 8) == 0 and ver(8, 4096, 32, 8, -1) == 0

    top = sized(lib, "sspec_pillar_topk_workspace_size", 3)   # n, max_ctx, hkv
    assert top(16, 4096, 8) > top(8, 4096, 8) > 0
    assert top(8, 0, 8) == 0 and top(8, 4096, 0) == 0

    dra = sized(lib, "sspec_draft_workspace_size", 4)   # n, max_ctx, hq, hkv
    assert dra(16, 4096, 32, 8) >= dra(8, 4096, 32, 8) > 0
    assert dra(8, 4096, 4, 8) == 0 and dra(-1, 4096, 32, 8) == 0


# ------------------------------------------------------ host-side validation
import subprocess

BUILD = os.path.join(ROOT, "sparse_self_speculative_amd", "_build")
CSRC = os.path.join(ROOT, "sparse_self_speculative_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]


def _kernel_objects():
    """The objects of the regular build other than the host code of sspec.hip."""
    objs = [os.path.join(BUILD, f"kernels_g{g}.o") for g in range(1, 9)] + \
        [os.path.join(BUILD, x) for x in ("kvcache.o", "offload.o", "sched.o")]
    return objs if all(os.path.exists(o) for o in objs) else None


def test_host_validation_rejects_bad_arguments(lib):
    """Every bad argument of every entry point returns its status and a
    message before any HIP call; the valid baselines stop at the first HIP
    call (no GPU here)."""
    from tests import abi_validation as V
    fails = V.run_cases(V.bind(LIB))
    assert not fails, "\n".join(fails)


def test_host_validation_under_sanitizers(lib, tmp_path):
    """The same cases against a build whose host code is compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual),
    loaded in a subprocess with the sanitizer runtime preloaded."""
    objs = _kernel_objects()
    rt = "/opt/rocm/llvm/lib/clang"
    rts = [os.path.join(rt, v, "lib", "linux", "libclang_rt.asan-x86_64.so") for v in sorted(os.listdir(rt))] \
        if os.path.isdir(rt) else []
    rts = [r for r in rts if os.path.exists(r)]
    if not objs or not rts or not os.path.exists(CLANGXX):
        pytest.skip("kernel objects or the sanitizer runtime are missing")
    so = str(tmp_path / "libsspec_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    hosts = []
    for src in ("sspec.hip", "kvcache.hip", "offload.hip", "sched.hip"):   # the units that hold host code
        hosts.append(str(tmp_path / (src + ".san.o")))
        subprocess.run([HIPCC, *FLAGS, "-O1", "-g", *san, "-c", os.path.join(CSRC, src), "-o", hosts[-1]],
                       check=True, capture_output=True)
    kernels = [o for o in objs if not o.endswith(("kvcache.o", "offload.o", "sched.o"))]
    subprocess.run([CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", "-o", so,
                    *hosts, *kernels, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rts[-1], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_validation.py"), so],
                         env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-4000:]


def test_mixed_build_is_rejected(lib, tmp_path):
    """A library linked from objects compiled with different build macros
    (here the G = 3 group with another score-chunk size) refuses every launch
    with SSPEC_ERR_UNSUPPORTED before touching the device."""
    objs = _kernel_objects()
    host = os.path.join(BUILD, "host.o")
    if not objs or not os.path.exists(host):
        pytest.skip("kernel objects are missing")
    odd = str(tmp_path / "kernels_g3_odd.o")
    # only the configuration string matters: the G = 3 row is left empty
    subprocess.run([HIPCC, *FLAGS, "-O1", "-DSSPEC_G=3", "-DSSPEC_ONLY_G=1", "-DSSPEC_SCORE_CHUNK=1024", "-c",
                    os.path.join(CSRC, "kernels.hip"), "-o", odd], check=True, capture_output=True)
    so = str(tmp_path / "libsspec_mixed.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so, host,
                    *[o if not o.endswith("kernels_g3.o") else odd for o in objs]],
                   check=True, capture_output=True)
    from tests import abi_validation as V
    mixed = V.bind(so)
    rc = V.call_verify(mixed, V.verify_args())
    msg = mixed.sspec_last_error().decode()
    assert rc == V.UNSUPPORTED and "mixed build" in msg and "score_chunk=1024" in msg, (rc, msg)
    rc = V.call_unified(mixed, V.unified_args())
    assert rc == V.UNSUPPORTED and "mixed build" in mixed.sspec_last_error().decode()


def _device_disassembly(obj: str, tmp: str) -> list[str]:
    """Instructions of the gfx950 code object inside one of the library's
    compiled objects (llvm-objdump of code built from these sources)."""
    llvm = "/opt/rocm/llvm/bin"
    fat, co = os.path.join(tmp, "k.fatbin"), os.path.join(tmp, "k.co")
    subprocess.run([f"{llvm}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", obj], check=True, capture_output=True)
    subprocess.run([f"{llvm}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True, capture_output=True)
    out = subprocess.run([f"{llvm}/llvm-objdump", "-d", "--no-show-raw-insn", co], check=True, capture_output=True,
                         text=True).stdout
    return [ln.split("//")[0].strip() for ln in out.splitlines() if ln.startswith("\t")]


def test_m0_is_written_only_by_the_lds_dma_sequences(tmp_path):
    """The LDS-DMA helpers set M0 in inline asm.  The compiler does not honour
    M0 as a clobber, so the kernels are only correct while the compiler keeps
    no value of its own in M0.  Check it on the built code: every instruction
    that names m0 is an `s_mov_b32 m0, sN` of the helpers, followed by its
    wait state and an LDS-DMA load."""
    objs = [os.path.join(BUILD, f"kernels_g{g}.o") for g in range(1, 9)]
    objs = [o for o in objs if os.path.exists(o)]
    if not objs or not os.path.exists("/opt/rocm/llvm/bin/llvm-objdump"):
        pytest.skip("kernel objects or the LLVM tools are missing")
    from concurrent.futures import ThreadPoolExecutor

    def check(ix_obj):
        ix, obj = ix_obj
        d = tmp_path / f"o{ix}"
        d.mkdir()
        ins = _device_disassembly(obj, str(d))
        bad, n = [], 0
        for i, s in enumerate(ins):
            if "m0" not in s.replace(",", " ").split():
                continue
            n += 1
            ok = (s.startswith("s_mov_b32 m0, s") and i + 2 < len(ins) and ins[i + 1].startswith("s_nop")
                  and ins[i + 2].startswith("global_load_lds_dwordx4"))
            if not ok:
                bad.append(f"{os.path.basename(obj)}: {s} | {' | '.join(ins[i + 1: i + 3])}")
        return n, bad

    with ThreadPoolExecutor(max_workers=min(8, len(objs))) as ex:
        res = list(ex.map(check, enumerate(objs)))
    assert sum(n for n, _ in res) > 0, "no LDS-DMA sequences found"
    bad = [b for _, bs in res for b in bs]
    assert not bad, "\n".join(bad[:20])
