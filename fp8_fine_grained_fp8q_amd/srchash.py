"""Hash of the GEMM source's code with comments and blank lines removed, the key under
which the committed counter and traffic summaries (profiles/gemm_counters.json,
profiles/gemm_traffic.json) record the kernels they were measured on: a change to the
code invalidates them, a change to a comment does not."""
import hashlib
import os
import re

GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")


def code_hash(path: str = GEMM_SOURCE) -> str:
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # block comments
    lines = []
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()  # line comments (the source has no "//" in strings)
        if line.strip():
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]
