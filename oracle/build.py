"""Compile the C oracle (test infrastructure only) into oracle/liboracle_kda.so,
and on request a copy built with AddressSanitizer and UndefinedBehaviorSanitizer
(oracle/liboracle_kda_san.so, loaded with gcc's ASan runtime preloaded)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_kda.so")
SAN_LIB = os.path.join(HERE, "liboracle_kda_san.so")
SRC = os.path.join(HERE, "kda_oracle.c")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    opt = SAN_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
