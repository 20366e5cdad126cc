"""Build step for the oracle (test infrastructure): plain gcc, fp64, no fast-math."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


FLAGS = ["-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-Wall", "-Wextra"]
#: extra flags of the checking build: address and undefined-behaviour sanitizers
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"]


def build_oracle(verbose: bool = False, src: str | None = None, out: str | None = None,
                 sanitize: bool = False) -> str:
    """Compile the oracle (by default qi4_oracle.c -> libqi4_oracle.so here);
    sanitize adds AddressSanitizer and UndefinedBehaviorSanitizer (the library
    then needs libasan loaded first in the process)."""
    src = src or os.path.join(HERE, "qi4_oracle.c")
    out = out or os.path.join(HERE, "libqi4_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", *(SANITIZE if sanitize else ["-O2"]), *FLAGS, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
