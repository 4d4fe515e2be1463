"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer:
every entry point, driven through the ctypes wrapper on small inputs, runs
without a sanitizer report (out-of-bounds access, use after free, signed
overflow, misaligned or invalid shifts...).  CPU only; the whole CPU suite can
be run against this build too:

    python -m oracle.build --sanitize
    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
        NVFP4_ORACLE_LIB=oracle/liboracle_san.so python -m pytest tests -m "not gpu"
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r'''
import numpy as np, oracle
from decode_attention_nvfp4_amd import workloads as W
rng = np.random.default_rng(1)
x = rng.standard_normal((37, 3, 128)).astype(np.float32)
x[0, 0, :16] = 0.0
x[1, 1, 16:32] *= 1e-30
st = oracle.tensor_scale(x)
c, s = oracle.quantize_rows(x, st)
xh = oracle.dequant_rows(c, s, st)
cm, sm = oracle.quantize_rows_mse(x[:5], st)
mc, ms = oracle.mx_quantize_rows(x)
oracle.mx_dequant_rows(mc, ms)
f8 = oracle.fp8_codes(x, oracle.fp8_tensor_scale(x))
oracle.fp8_dequant(f8, 0.01)
packed = (c[:, :, 0::2] | (c[:, :, 1::2] << 4)).reshape(-1, 64)
oracle.nvfp4_to_fp8_packed(packed, s.reshape(-1, 8), 3.0, 0.5)
q = rng.standard_normal((2, 6, 128)).astype(np.float32)
seqs = [(c[:0], s[:0], c[:0], s[:0]), (c, s, c, s)]
oracle.decode_batch(q, seqs, 3, st, st)
oracle.decode_batch_dense(q, [(xh[:5], xh[:5]), (xh, xh)], 3)
oracle.prefill_rows(rng.standard_normal((4, 6, 128)).astype(np.float32), np.array([0, 1, 5, 6], np.int32), 3,
                    c, s, st, c, s, st, 30, causal=True)
oracle.prefill_rows(rng.standard_normal((2, 6, 128)).astype(np.float32), np.array([0, 6], np.int32), 3,
                    c, s, st, c, s, st, 30, causal=False)
print("sanitized oracle ok")
'''


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_address_and_ub_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import build
    lib = build.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", NVFP4_ORACLE_LIB=lib, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", DRIVER], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "sanitized oracle ok" in r.stdout
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
