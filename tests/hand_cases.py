"""Loader for the hand-worked golden cases (tests/golden/hand_cases.json).

Builds the e4m3 code matrices, the scale tables and the expected bf16 bits of
each case. Shared by the oracle pins and the GPU bit-exact tests; it holds no
GEMM arithmetic (expected values are the hand-derived numbers in the file).
"""
import json
import os

import numpy as np

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def load():
    with open(_PATH) as f:
        cases = json.load(f)["cases"]
    out = []
    for c in cases:
        M, N, K = c["M"], c["N"], c["K"]
        a = np.full((M, K), c["a_fill"], dtype=np.uint8)
        for r, k, code in c["a"]:
            a[r, k] = code
        b = np.full((N, K), c["b_fill"], dtype=np.uint8)
        for r, k, code in c["b"]:
            b[r, k] = code
        sa = np.array(c["sa"], dtype=np.float32).reshape(M, K // 128)
        sb = np.array(c["sb"], dtype=np.float32).reshape(N // 128, K // 128)
        if "expect_by_block" in c:
            exp = np.zeros((M, N), dtype=np.uint16)
            for key, bits in c["expect_by_block"].items():
                m, nb = (int(x) for x in key.split(","))
                exp[m, nb * 128:(nb + 1) * 128] = bits
        else:
            exp = np.full((M, N), c["expect_default"], dtype=np.uint16)
            for m, n, bits in c["expect"]:
                exp[m, n] = bits
        allowed = exp.copy()
        for m, n, bits in c.get("gpu_allowed", []):
            allowed[m, n] = bits
        out.append(dict(name=c["name"], M=M, N=N, K=K, a=a, b=b, sa=sa, sb=sb,
                        expect=exp, gpu_exact=c["gpu_exact"], gpu_alt=allowed))
    return out
