"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle (C, gcc) is rebuilt with -fsanitize=address,undefined and a
representative set of its entry points runs in a subprocess with the
sanitizer runtime preloaded.  The HIP library's host code is rebuilt with
the sanitizers on its host compilation pass only (the device code is the
same) and driven by tests/abi_host_check.c: size and capacity queries and
argument validation, which need no GPU.  Any sanitizer report fails the
test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]

ORACLE_SCRIPT = r'''
import numpy as np
import oracle

def make(S, d, h, E, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return (f(S, d), f(E, d) / np.float32(np.sqrt(d)), 0.3 * f(E), f(E, h, d) / np.float32(np.sqrt(d)),
            0.2 * f(E, h), f(E, d, h) / np.float32(np.sqrt(h)), 0.2 * f(E, d), f(S, d))

def bf16(a):
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

for (S, d, h, E, k, cf, seed) in [(70, 16, 24, 6, 2, 0.6, 1), (45, 8, 12, 9, 3, 1.0, 2),
                                  (33, 8, 8, 4, 1, 2.0, 3), (64, 16, 16, 12, 4, 0.5, 4)]:
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, seed)
    C = oracle.capacity(S, E, k, cf)
    for act in (lambda a: a, bf16):
        xs, w1s, b1s, w2s, b2s, dys = (act(a) for a in (x, w1, b1, w2, b2, dy))
        lg = oracle.logits(xs, wg, bg)
        for rr in (False, True):
            r = oracle.route(lg, k, C, reroute=rr)
            res = oracle.layer(xs, wg, bg, w1s, b1s, w2s, b2s, k, C, lg=lg, reroute=rr)
            g = oracle.layer_backward(xs, wg, w1s, b1s, w2s, b2s, k, C, lg, dys, 0.3, 0.2,
                                      reroute=rr)
            tok = np.arange(0, S, 5)
            oracle.token_output(tok, xs, w1s, b1s, w2s, b2s, r["serve"], r["slot"], r["w"])
            oracle.backward_entries(xs, wg, w1s, b1s, w2s, b2s, k, C, lg, dys, 0.3, 0.2, tok,
                                    [(1, 0, 1, 2), (2, E - 1, 0, 1), (3, 1, 2, 0), (4, 0, 3, 0)],
                                    reroute=rr)
        oracle.router_backward(lg, r["idx"], r["w"], g["dw"], r["counts"][:k], 0.3, 0.2)
        dl = oracle.layer_dropless(xs, wg, bg, w1s, b1s, w2s, b2s, k, lg=lg)
        oracle.compact_rows(dl["idx"], E)
        oracle.layer_backward(xs, wg, w1s, b1s, w2s, b2s, k, S, lg, dys, 0.1, 0.1)
# integer logits full of ties, with re-routing at capacity 1
rng = np.random.default_rng(9)
lg = (rng.integers(-2, 3, (40, 7)) / 2).astype(np.float32)
oracle.route(lg, 3, 1, reroute=True)
print("oracle ok")
'''


def _clean(stderr: str) -> bool:
    return "ERROR: AddressSanitizer" not in stderr and "runtime error:" not in stderr


def test_oracle_under_asan_ubsan(tmp_path):
    gcc_asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.exists(gcc_asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", *SAN_FLAGS,
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", str(so), "-lm"])
    env = dict(os.environ, LD_PRELOAD=gcc_asan, ASAN_OPTIONS="detect_leaks=0",
               MOE_ORACLE_LIBRARY=str(so), OMP_NUM_THREADS="2", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", ORACLE_SCRIPT], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and _clean(r.stderr), r.stderr[-6000:]
    assert "oracle ok" in r.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    llvm = "/opt/rocm/llvm/bin"
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    hipcc = "/opt/rocm/bin/hipcc"
    if not rt or not os.path.exists(hipcc):
        pytest.skip("ROCm's clang AddressSanitizer runtime is not installed")
    from sparse_moe_layer_wg_amd import _build
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    objs = []
    for src in sorted(glob.glob(os.path.join(_build.CSRC, "*.hip"))):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.check_call([hipcc, *_build.HIPCC_FLAGS, *host_san, "-c", src, "-o", str(obj)])
        objs.append(str(obj))
    lib = tmp_path / "libmoe.so"
    subprocess.check_call([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *objs,
                           "-o", str(lib)])
    exe = tmp_path / "abi_host_check"
    subprocess.check_call([os.path.join(llvm, "clang"), "-std=c11", *SAN_FLAGS,
                           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "abi_host_check.c"), str(lib),
                           f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-lamdhip64",
                           "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and _clean(r.stderr), (r.stdout[-3000:], r.stderr[-6000:])
    assert "ok: 0 failed" in r.stdout
