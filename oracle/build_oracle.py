"""Build the oracle's shared library with gcc (no HIP, no shared code)."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "minikv_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "liboracle.so")


def lib_path():
    return _LIB


def build(force=True):
    """Compile minikv_oracle.c into oracle/_build/liboracle.so.

    -ffp-contract=off and no fast-math: every fp32 operation of the codec is a
    single IEEE round-to-nearest-even operation, in source order.
    """
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB
