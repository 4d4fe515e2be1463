"""Compile the C oracle into oracle/liboracle.so (plain gcc, -O2, no fast-math).

Test infrastructure: the product library never links or loads this.

    python -m oracle.build            # oracle/liboracle.so
    python -m oracle.build --sanitize # oracle/liboracle_san.so, built with
                                      # AddressSanitizer and UndefinedBehavior-
                                      # Sanitizer (load it with NVFP4_ORACLE_LIB
                                      # and LD_PRELOAD=$(gcc -print-file-name=libasan.so))
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", *(SAN_FLAGS if sanitize else []),
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
