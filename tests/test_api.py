"""CPU tests of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before any HIP call (no GPU needed:
a rejected call enqueues nothing, so fake device addresses are safe here)."""

import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

import exact_io_aware_28_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH),
                                reason="library not built")

# fake, 16-byte aligned device addresses: never dereferenced on these paths
P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_bias", "fa_bwd_dropout",
                                    "fa_bwd_f16", "fa_bwd_workspace_size",
                                    "fa_decode", "fa_decode_noalloc",
                                    "fa_decode_noalloc_max_splits", "fa_decode_num_splits",
                                    "fa_decode_workspace_size", "fa_fwd", "fa_fwd_bias",
                                    "fa_fwd_dropout", "fa_fwd_f16", "fa_fwd_f32",
                                    "fa_fwd_fp8", "fa_quantize_fp8", "fa_status_string"]


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH],
                             capture_output=True, text=True).stdout
        exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
        assert set(declared_functions()) <= exported


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_is_self_contained(lang, tmp_path):
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "fa_mi355x.h"\n'
                   'int (*f)(const void*, const void*, const void*, void*, float*, int,'
                   ' int, int, int, int, int, float, int, int, const int32_t*, void*)'
                   ' = fa_fwd;\nint main(void){return f == 0;}\n')
    r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", "-I",
                        os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _fwd(fn=None, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, Hq=4, Hkv=2, Nq=64,
         Nk=64, d=128, scale=0.125, causal=0, window=0, cu=None):
    fn = fn or fa.lib().fa_fwd
    return fn(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window, cu, None)


BAD_FWD = [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(0x10008)), fa.FA_ERR_INVALID_ARG),   # misaligned
    (dict(lse=ctypes.c_void_p(0x10002)), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-5), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(window=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(cu=P[5], Nq=64, Nk=128), fa.FA_ERR_UNSUPPORTED),
    (dict(cu=ctypes.c_void_p(0x10001)), fa.FA_ERR_INVALID_ARG),
    # 64 rows of one head would span 4 GiB: beyond the 32-bit tile descriptors
    (dict(Hq=262144, Hkv=1), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=262144 * 2, Hkv=2, d=64), fa.FA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("bad,code", BAD_FWD)
@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f16", "fa_fwd_f32"])
def test_forward_rejects(entry, bad, code):
    assert _fwd(getattr(fa.lib(), entry), **bad) == code


def _bwd(ws=P[9], ws_bytes=None, entry="fa_bwd", **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7],
             dv=P[8], B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, scale=0.125, causal=0,
             window=0, cu=None)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(a["B"] * a["Nq"], a["Hq"], a["d"])
    return getattr(fa.lib(), entry)(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                    a["dq"], a["dk"], a["dv"], ws, ws_bytes, a["B"], a["Hq"],
                                    a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                    a["causal"], a["window"], a["cu"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),
    (dict(dq=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=None), fa.FA_ERR_INVALID_ARG),
    (dict(do=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=ctypes.c_void_p(0x20004)), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(window=-3), fa.FA_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("entry", ["fa_bwd", "fa_bwd_f16"])
def test_backward_rejects(entry, bad, code):
    assert _bwd(entry=entry, **bad) == code


def test_workspace_is_linear_in_rows():
    s1 = fa.fa_bwd_workspace_size(16384, 16, 128)
    s2 = fa.fa_bwd_workspace_size(32768, 16, 128)
    assert s1 >= 16384 * 16 * 4 and s2 <= 2 * s1 + 256
    assert fa.fa_bwd_workspace_size(0, 16, 128) == 0
    assert fa.fa_bwd_workspace_size(10, -1, 128) == 0


def _dec(ws=P[9], ws_bytes=None, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, Hq=8, Hkv=2, Nq=1, Nk=4096,
             d=128, scale=0.125, causal=1, window=0, lens=None, splits=4)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_decode_workspace_size(a["B"], a["Hq"], a["Nq"], a["d"],
                                               max(a["splits"], 1))
    return fa.lib().fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                              a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                              a["window"], a["lens"], a["splits"], ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=64), fa.FA_ERR_INVALID_ARG),
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=1025), fa.FA_ERR_INVALID_ARG),
    (dict(lens=ctypes.c_void_p(0x10002)), fa.FA_ERR_INVALID_ARG),  # misaligned
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=ctypes.c_void_p(0x20004)), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(window=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
])
def test_decode_rejects(bad, code):
    assert _dec(**bad) == code


def _dec_noalloc(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, Hq=8, Hkv=2, Nq=1, Nk=4096,
             d=128, scale=0.125, causal=1, window=0, lens=None, splits=4)
    a.update(kw)
    return fa.lib().fa_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                      a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                      a["causal"], a["window"], a["lens"], a["splits"], None)


@pytest.mark.parametrize("bad,code", [
    # partials of 8 splits x 64 x 16 x 64 rows x 128 floats: 256 MiB > 32 MiB
    (dict(B=64, Hq=64, Hkv=8, Nq=16, splits=8), fa.FA_ERR_TOO_LARGE),
    # even one split (32 MiB of partial outputs plus their LSEs) does not fit
    (dict(B=64, Hq=64, Hkv=8, Nq=16, splits=0), fa.FA_ERR_TOO_LARGE),
    (dict(splits=1025), fa.FA_ERR_INVALID_ARG),
    (dict(splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(lens=ctypes.c_void_p(0x10002)), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
])
def test_decode_noalloc_rejects_before_any_hip_call(bad, code):
    assert _dec_noalloc(**bad) == code


def test_decode_noalloc_max_splits():
    cap = fa.DECODE_NOALLOC_SCRATCH_BYTES
    # 16 sequences x 32 heads x 128 floats per split, plus 16 x 32 LSEs
    assert fa.fa_decode_noalloc_max_splits(16, 32, 1, 128) == cap // (16 * 32 * 129 * 4)
    for args in [(16, 32, 1, 128), (3, 8, 4, 64), (64, 32, 8, 128)]:
        s = fa.fa_decode_noalloc_max_splits(*args)
        assert fa.fa_decode_workspace_size(*args, s) <= cap
        assert s == 1024 or fa.fa_decode_workspace_size(*args, s + 1) > cap
    assert fa.fa_decode_noalloc_max_splits(64, 64, 16, 128) == 0
    assert fa.fa_decode_noalloc_max_splits(0, 64, 16, 128) == 0
    assert "FA_ERR_TOO_LARGE" in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)


def test_decode_workspace_and_default_splits():
    # partial outputs (d floats) and partial LSEs (1 float) per split and row
    s1 = fa.fa_decode_workspace_size(16, 32, 1, 128, 8)
    assert 8 * 16 * 32 * 129 * 4 <= s1 <= 8 * 16 * 32 * 129 * 4 + 512
    assert fa.fa_decode_workspace_size(16, 32, 1, 128, 0) == 0
    assert fa.fa_decode_workspace_size(0, 32, 1, 128, 4) == 0
    # enough work-groups to fill the chip, at least ~256 keys per split
    assert fa.fa_decode_num_splits(16, 32, 8, 1, 8192) == 12
    assert fa.fa_decode_num_splits(1, 32, 8, 1, 512) == 2
    assert fa.fa_decode_num_splits(64, 32, 8, 1, 65536) == 3
    assert fa.fa_decode_num_splits(1, 1, 1, 1, 100) == 1
    assert 1 <= fa.fa_decode_num_splits(1, 8, 1, 1, 1 << 24) <= 128
    assert fa.fa_decode_num_splits(1, 6, 4, 1, 100) == 0  # Hq % Hkv != 0


def _fwd_bias(bias=P[6], sb=0, sh=0, sq=64, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, Hq=4, Hkv=2, Nq=64, Nk=64,
             d=128, scale=0.125, causal=0, window=0)
    a.update(kw)
    return fa.lib().fa_fwd_bias(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                a["window"], bias, sb, sh, sq, None)


def _bwd_bias(bias=P[10], sb=0, sh=0, sq=64, ws_bytes=None, **kw):
    a = dict(B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, scale=0.125, causal=0, window=0)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(a["B"] * a["Nq"], a["Hq"], a["d"])
    return fa.lib().fa_bwd_bias(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9],
                                ws_bytes, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                a["scale"], a["causal"], a["window"], bias, sb, sh, sq, None)


BAD_BIAS = [
    (dict(bias=None), fa.FA_ERR_INVALID_ARG),
    (dict(bias=ctypes.c_void_p(0x70002)), fa.FA_ERR_INVALID_ARG),  # not 4-byte aligned
    (dict(sb=-4), fa.FA_ERR_INVALID_ARG),
    (dict(sh=-1), fa.FA_ERR_INVALID_ARG),
    (dict(sq=-64), fa.FA_ERR_INVALID_ARG),
    # 32 rows of one head must span less than 2^32 bytes: (31 sq + Nk) * 4
    (dict(sq=(1 << 30) // 31), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=5), fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("bad,code", BAD_BIAS)
def test_bias_entry_points_reject(bad, code):
    assert _fwd_bias(**bad) == code
    assert _bwd_bias(**{k: v for k, v in bad.items()}) == code


def test_bias_backward_checks_workspace():
    assert _bwd_bias(ws_bytes=8) == fa.FA_ERR_INVALID_ARG


def _fwd_drop(p=0.1, **kw):
    a = dict(B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, scale=0.125, causal=0, window=0, cu=None)
    a.update(kw)
    return fa.lib().fa_fwd_dropout(P[0], P[1], P[2], P[3], P[4], a["B"], a["Hq"], a["Hkv"],
                                   a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                   a["window"], a["cu"], p, 1234, None)


def _bwd_drop(p=0.1, ws_bytes=None, **kw):
    a = dict(B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=128, scale=0.125, causal=0, window=0, cu=None)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(a["B"] * a["Nq"], a["Hq"], a["d"])
    return fa.lib().fa_bwd_dropout(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8],
                                   P[9], ws_bytes, a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                   a["Nk"], a["d"], a["scale"], a["causal"], a["window"],
                                   a["cu"], p, 1234, None)


BAD_DROPOUT = [
    (dict(p=1.0), fa.FA_ERR_INVALID_ARG),
    (dict(p=1.5), fa.FA_ERR_INVALID_ARG),
    (dict(p=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(p=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(window=-1), fa.FA_ERR_INVALID_ARG),
    (dict(cu=ctypes.c_void_p(0x70002)), fa.FA_ERR_INVALID_ARG),  # misaligned cu_seqlens
]


@pytest.mark.parametrize("bad,code", BAD_DROPOUT)
def test_dropout_entry_points_reject(bad, code):
    assert _fwd_drop(**bad) == code
    assert _bwd_drop(**bad) == code


def test_dropout_backward_checks_workspace():
    assert _bwd_drop(ws_bytes=8) == fa.FA_ERR_INVALID_ARG


def test_status_strings():
    for st in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        assert fa.fa_status_string(st).startswith("FA_")
    assert "unknown" in fa.fa_status_string(99)


# ------------------------------------------------- host AddressSanitizer run
ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
STUB_RUN = os.environ.get("FA_API_STUB_LAUNCHERS") == "1"


@pytest.mark.skipif(not STUB_RUN, reason="only against the stub-launcher build (no GPU work)")
def test_valid_calls_reach_the_launcher():
    """With stub launchers every well-formed call passes its checks, fills its
    parameter block and returns the launcher's failure as FA_ERR_HIP: the
    whole host path of each entry point runs under the sanitizer."""
    L = fa.lib()
    for call in (lambda: _fwd(), lambda: _bwd(), lambda: _bwd(entry="fa_bwd_f16"),
                 lambda: _dec(), lambda: _fwd_bias(), lambda: _bwd_bias()):
        assert call() == fa.FA_ERR_HIP
    assert L.fa_quantize_fp8(P[0], P[1], P[2], 2, 100, 3, 128, 1, P[3], None) == fa.FA_ERR_HIP
    assert L.fa_fwd_fp8(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 1, 4, 2, 100, 100, 128,
                        0.1, 1, 0, None) == fa.FA_ERR_HIP


def _host_build(tmp_path, srcs, out):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-g",
           "-O1", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "exact_io_aware_28_amd", "csrc"), *srcs, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def _run_sanitized(script, lib):
    env = dict(os.environ, LD_PRELOAD=ASAN_RT, FA_API_STUB_LAUNCHERS="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86")
    return subprocess.run([sys.executable, "-c", script, str(lib)], capture_output=True,
                          text=True, env=env, cwd=ROOT, timeout=600)


@pytest.mark.skipif(STUB_RUN or not os.path.exists(ASAN_RT), reason="needs the ASan runtime")
def test_api_checks_under_address_sanitizer(tmp_path):
    """The C ABI layer (csrc/fa_api.hip) built with host AddressSanitizer and
    stub launchers; this file's checks run against it in a child process."""
    lib = _host_build(tmp_path, [os.path.join(ROOT, "exact_io_aware_28_amd", "csrc",
                                              "fa_api.hip"),
                                 os.path.join(ROOT, "tests", "host", "api_stub_launchers.cpp")],
                      tmp_path / "libfa_api_asan.so")
    script = ("import sys, pytest\n"
              "import exact_io_aware_28_amd as fa\n"
              "fa.LIB_PATH = sys.argv[1]\n"
              "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_api.py',\n"
              "                      '-k', 'not sanitizer']))\n")
    r = _run_sanitized(script, lib)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    summary = r.stdout.strip().splitlines()[-1]
    assert " passed" in summary and "skipped" not in summary, summary


@pytest.mark.skipif(STUB_RUN or not os.path.exists(ASAN_RT), reason="needs the ASan runtime")
def test_sanitizer_harness_reports_a_heap_overflow(tmp_path):
    """The same build and preload catch a real error: a host function that
    reads one element past a heap buffer (test code, not the library)."""
    src = tmp_path / "overflow.hip"
    src.write_text('#include <cstdlib>\nextern "C" int past_the_end(int n) {\n'
                   '  int* a = (int*)std::malloc(n * sizeof(int));\n'
                   '  for (int i = 0; i < n; ++i) a[i] = i;\n'
                   '  volatile int x = a[n];\n  std::free(a);\n  return x;\n}\n')
    lib = _host_build(tmp_path, [str(src)], tmp_path / "liboverflow.so")
    r = _run_sanitized("import ctypes, sys\nctypes.CDLL(sys.argv[1]).past_the_end(8)\n", lib)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
