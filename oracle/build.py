"""Build the fp64 CPU oracle (plain C, OpenMP) -- test infrastructure only.

`build()` compiles oracle/attn_oracle.c into oracle/libattn_oracle.so with gcc.
`build_mutant(n, outdir)` compiles the same source with ORACLE_MUTANT=n, a
variant with one planted mistake that the pin tests must reject.
No fast-math: the oracle keeps IEEE double semantics and source order.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "libattn_oracle.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math"]

# Planted mistakes, each a one-line change under ORACLE_MUTANT in attn_oracle.c.
MUTANTS = {
    1: "scale dropped",
    2: "GQA map h % Hkv instead of h / (Hq/Hkv)",
    3: "causal diagonal off by one",
    4: "top-left instead of bottom-right alignment",
    5: "window one key too wide",
    6: "row max left out of the LSE",
    7: "V operand indexed transposed",
    9: "weights not normalised",
    10: "per-sequence lengths ignored",
    11: "last channel of the dot product dropped",
    12: "score sign flipped",
    13: "LSE in base 2",
    14: "causal limit kept for non-causal rows",
    15: "fp16 exponent bias off by one",
    16: "backward: softmax Jacobian delta term dropped",
    17: "backward: scale missing from dK",
    18: "backward: dV from unnormalised weights",
    19: "backward: dV accumulated into kv-head h % Hkv",
}
# Mutants of the backward only; the forward pins cannot see them.
BWD_MUTANTS = (16, 17, 18, 19)


def _compile(out, defines=()):
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


SANITIZE_MAIN = os.path.join(HERE, "sanitize_main.c")


def build() -> str:
    """The oracle library, and a compile-and-link check of the sanitizer driver
    (tests/test_oracle_sanitized.py builds and runs it under ASan/UBSan)."""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-Wall", "-Wextra", "-o", os.path.join(d, "driver"),
                        SRC, SANITIZE_MAIN, "-lm"], check=True)
    return _compile(LIB)


def build_mutant(n: int, outdir: str) -> str:
    return _compile(os.path.join(outdir, f"libattn_oracle_m{n}.so"), [f"ORACLE_MUTANT={n}"])


if __name__ == "__main__":
    print(build())
