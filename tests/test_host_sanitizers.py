"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the fp64 oracle (oracle/fd_oracle.c) driven by
tests/sanitize/oracle_check.c, and the library's host runtime
(decode_attention_12_amd/csrc/fd_api.cpp: planner, workspace layout, every
entry point's argument checks and launch records) driven by
tests/sanitize/api_check.cpp against host-only kernel stand-ins
(tests/sanitize/kernels_stub.cpp) that launch nothing. Both are built with
gcc / g++ (no device code is involved) and must run clean; the plans the
sanitized build makes must equal the real library's."""
import ctypes
import os
import shutil
import subprocess

import pytest

import decode_attention_12_amd as fd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = {**os.environ, "ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11", "-Wall", "-Wno-unknown-pragmas", *SAN_FLAGS, os.path.join(ROOT, "oracle", "fd_oracle.c"),
          os.path.join(SAN, "oracle_check.c"), "-lm", "-o", exe])
    assert "oracle_check: ok" in _run([exe], env=ENV)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_runtime_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_check")
    csrc = os.path.join(ROOT, "decode_attention_12_amd", "csrc")
    _run(["g++", "-std=c++17", "-Wall", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "fd_api.cpp"),
          os.path.join(SAN, "kernels_stub.cpp"), os.path.join(SAN, "api_check.cpp"),
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    out = _run([exe], env=ENV)
    assert "api_check: ok" in out
    plans = [line.split() for line in out.splitlines() if line.startswith("PLAN")]
    assert len(plans) > 100
    # Every plan of the sanitized build (stub geometry) equals the real library's.
    for t in plans:
        B, Hq, Hkv, D, L, page, kv, q_len, S = map(int, t[1:10])
        want = [int(x) for x in t[11:]]
        p = fd.make_problem(B, Hq, Hkv, D, L, kv_dtype=kv, page_size=page,
                            num_pages=(L + page - 1) // page * B if page else 0, q_len=q_len,
                            out_dtype=fd.FD_F32 if kv == fd.FD_F32 else fd.FD_BF16)
        plan = fd.fd_plan()
        st = fd.binding._lib.fd_plan_splits(ctypes.byref(p), 256, S, ctypes.byref(plan))
        got = [st] + ([plan.num_splits, plan.chunk_len, plan.path, plan.mode, plan.workers, plan.tile,
                       plan.lead_workers, plan.lead_pct, fd.fd_workspace_size(p, plan)] if st == 0 else [0] * 9)
        assert got == want, f"plan differs for {t[1:10]}: real {got}, sanitized build {want}"
