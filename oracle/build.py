"""Build the CPU oracle shared library (test infrastructure only).

``python -m oracle.build`` or ``oracle.build.build()`` compiles
``kda_oracle.c`` with gcc into ``oracle/libkda_oracle.so``.  Plain -O2 with
the compiler's own vectorisation; no target-specific flags, so the library
runs on any x86-64 host.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkda_oracle.so")
SOURCES = [os.path.join(HERE, "kda_oracle.c")]
HEADERS = [os.path.join(HERE, "kda_oracle.h"), os.path.join(HERE, "kda_oracle_body.h")]


def compile_command(out=LIB, sources=None, extra=()):
    return (["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-Wall",
             "-Wextra", "-Wno-unused-parameter", "-o", out]
            + list(sources or SOURCES) + list(extra) + ["-lm"])


def build(out=LIB, sources=None, extra=()):
    """Compile the oracle; raises CalledProcessError on a compiler error."""
    tmp = out + ".tmp"
    subprocess.run(compile_command(tmp, sources, extra), check=True, cwd=HERE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
