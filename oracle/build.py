"""Build the CPU oracle shared library (test infrastructure only).

    python -m oracle.build          # from the repository root

Compiles ``gdn_oracle.c`` with gcc into ``liboracle_gdn.so`` beside it. No
fast-math: the oracle relies on IEEE double semantics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle_gdn.so")


SAN_LIB = os.path.join(HERE, "liboracle_gdn_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build the oracle library; sanitize=True builds liboracle_gdn_san.so with
    AddressSanitizer and UndefinedBehaviorSanitizer (host code only), for a test
    run with the sanitizer runtimes preloaded."""
    out = SAN_LIB if sanitize else LIB
    flags = ["-O2"]
    if sanitize:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"]
    cmd = ["gcc"] + flags + ["-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                             "-ffp-contract=off", "-Wall", "-Wextra", "-o", out + ".tmp", SRC,
                             "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
