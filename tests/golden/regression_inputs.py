"""Formula-defined tiny inputs for the oracle regression fixture.

Shared by ``make_golden.py`` (which writes the expected values by calling
only the oracle) and by the test that re-checks them.  No randomness: every
value is a small dyadic rational, exactly representable in BF16 / E4M3FN.
"""

import numpy as np
import torch

D = 512


def _bits(x, dtype):
    t = torch.as_tensor(np.asarray(x, np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def case(dtype="bf16"):
    T, H, K = 3, 2, 136
    d = np.arange(D)
    q = np.empty((T, H, D))
    for t in range(T):
        for h in range(H):
            q[t, h] = ((d * (3 + h) + 5 * t) % 9 - 4) / 16.0
    swa = np.array([((d * 7 + 11 * r) % 13 - 6) / 8.0 for r in range(20)])
    comp = np.array([((d * 5 + 3 * r) % 11 - 5) / 4.0 for r in range(30)])
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        idx[t, :128] = (np.arange(128) * (t + 3)) % 20
        idx[t, 128:] = (np.arange(8) * 7 + t) % 30
    idx[0, [3, 130]] = -1
    idx[2, :] = -1
    idx[2, 129] = 4
    topk = np.array([136, 100, 136], np.int32)
    sinks = np.array([0.5, -0.25], np.float32)
    return dict(q_bits=_bits(q, dtype), q_dtype=dtype,
                swa_bits=_bits(swa, dtype), comp_bits=_bits(comp, dtype),
                kv_dtype=dtype, indices=idx, topk_lens=topk, sinks=sinks,
                bmm1_scale=0.0625, bmm2_scale=0.5, lse_scale=1.0)
