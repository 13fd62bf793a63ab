"""Independent brute-force references used to pin the oracle.

Written without any code from ``oracle/``: plain Python floats and
``math.exp`` over explicit loops (no max-subtraction, no numpy matmul), and
a thin wrapper over torch's CPU scaled-dot-product attention in float64.
Only for tiny inputs.
"""

import math

import numpy as np


def bits_to_float(b: int) -> float:
    """bf16 bits -> Python float via the IEEE single layout (struct)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def brute_attention(qvec, keys, values, scale):
    """sum_j e^{s_j} v_j / sum_j e^{s_j}, log sum_j e^{s_j}; pure Python."""
    s = []
    for k in keys:
        acc = 0.0
        for a, b in zip(qvec, k):
            acc += a * b
        s.append(scale * acc)
    w = [math.exp(x) for x in s]
    z = sum(w)
    out = [0.0] * len(values[0])
    for wj, v in zip(w, values):
        for d in range(len(v)):
            out[d] += wj * v[d]
    return [o / z for o in out], math.log(z)


def decode_brute(inp):
    """Decode of every request via explicit loops over the page table."""
    B, Hq, D = inp.dec_q.shape
    ratio = Hq // inp.num_kv_heads
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for r in range(B):
        row = int(inp.dec_req_rows[r])
        L = int(inp.dec_seq_lens[r])
        slots = [int(inp.page_table[row, j]) for j in range(L)]
        for h in range(Hq):
            g = h // ratio
            qv = [bits_to_float(x) for x in inp.dec_q[r, h]]
            ks = [[bits_to_float(x) for x in inp.k_pool[s, g]] for s in slots]
            vs = [[bits_to_float(x) for x in inp.v_pool[s, g]] for s in slots]
            o, l = brute_attention(qv, ks, vs, inp.sm_scale)
            out[r, h] = o
            lse[r, h] = l
    return out, lse


def sdpa_extend(q_f64, k_f64, v_f64, prefix, scale):
    """torch CPU SDPA for one request: q [E, Hq, D], k/v [P+E, Hkv, D] float64.

    GQA by repeating each kv head over its group of q heads; the causal mask
    is given explicitly (bottom-right aligned), since ``is_causal`` aligns
    top-left and the two agree only when the prefix is empty.
    """
    import torch
    E, Hq, D = q_f64.shape
    N, Hkv, _ = k_f64.shape
    ratio = Hq // Hkv
    q = torch.from_numpy(np.ascontiguousarray(q_f64.transpose(1, 0, 2)))           # [Hq, E, D]
    k = torch.from_numpy(np.ascontiguousarray(k_f64.transpose(1, 0, 2))).repeat_interleave(ratio, 0)
    v = torch.from_numpy(np.ascontiguousarray(v_f64.transpose(1, 0, 2))).repeat_interleave(ratio, 0)
    i = torch.arange(E)[:, None]
    j = torch.arange(N)[None, :]
    mask = j <= prefix + i
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], attn_mask=mask[None, None], scale=scale)[0]
    return o.permute(1, 0, 2).numpy()
