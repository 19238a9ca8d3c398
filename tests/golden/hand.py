"""Loader for the hand-derived examples in hand_examples.json."""
import json
import os

import numpy as np

from verify_matmul_amd import synth

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_examples.json")


def cases():
    with open(_PATH) as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        M, K, N, g = c["M"], c["K"], c["N"], c["group"]
        qweight = np.array([[int(w, 16)] * N for w in c["qweight_row_words"]], dtype=np.uint32)
        assert qweight.shape == (K // 8, N)
        qzeros = None
        if c["qzeros_words"] is not None:
            qzeros = np.array([[int(w, 16)] * (N // 8) for w in c["qzeros_words"]], dtype=np.uint32)
        scales = np.array([[int(s, 16)] * N for s in c["scale_bits"]], dtype=np.uint16)
        rows = []
        for pattern in c["act_rows"]:
            rows.append([pattern[k % len(pattern)] for k in range(K)])
        act = synth.f32_to_bf16_bits(np.array(rows, dtype=np.float32))
        out.append(dict(name=c["name"], M=M, K=K, N=N, group=g, qweight=qweight, qzeros=qzeros,
                        scales=scales, act=act, y=np.array(c["y"], dtype=np.float64)))
    return out
