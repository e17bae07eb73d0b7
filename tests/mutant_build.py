"""Build a copy of the oracle's C source with one planted mistake (test
infrastructure: the mutant tests show that the pins catch each mistake)."""
import functools
import os
import subprocess

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn2_oracle.c")


@functools.lru_cache(maxsize=None)
def build_mutant(name, old, new, tmpdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path_c = os.path.join(tmpdir, f"mut_{name}.c")
    path_so = os.path.join(tmpdir, f"mut_{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_POSIX_C_SOURCE=200809L",
                           "-o", path_so, path_c, "-lpthread"])
    return path_so
