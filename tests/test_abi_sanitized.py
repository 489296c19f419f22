"""The CPU-side ABI tests again, against a build of the library whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged): argument validation, shard
geometry, error strings and the profiling calls must run without a sanitizer report.  Runs in a
child process with the ASan runtime preloaded; no GPU is touched."""

import os
import subprocess
import sys

from tensor_transformer_layer_mlp_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _stale():
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(B.INCLUDE, "tpshard.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


def test_abi_under_host_sanitizers():
    if _stale():
        B.build(sanitize=True)
    env = B.sanitizer_env()
    probe = ("import sys; sys.path.insert(0, %r); from tensor_transformer_layer_mlp_amd import binding as bd; "
             "bd.raw(); print([l.split()[-1] for l in open('/proc/self/maps') if 'libtpshard' in l][0])" % ROOT)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("libtpshard_san.so"), r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")], env=env, capture_output=True, text=True, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
