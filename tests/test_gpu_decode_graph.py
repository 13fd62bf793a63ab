"""Graph-replayed decode step (msgl_decode_graph_*): the ladder of captured
batch sizes, padding with the dummy request on the sentinel slot, replays
bit-identical to eager calls on the same padded batch, results within the
attention tolerance of the oracle, and no slot written but the live ones and
the sentinel — including after a larger batch left stale rows behind.  Both
capture forms: store_kv + decode as two calls (page-table rows that overlap,
so one request's new slot can be another's key) and the one-launch store +
decode (disjoint rows: each new slot is its own request's newest key only).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_30_amd as msgl
from workloads import random_bf16
from tests.gpu_util import up, bits, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu

S, HQ, HKV, D, MAXB, STRIDE = 65536, 32, 8, 128, 64, 4096
SCALE = 1.0 / np.sqrt(D)


def banner(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fused", [False, True])
def test_decode_graph_ladder_padding_and_replay(fused):
    banner(f"fused store {fused}")
    rng = np.random.default_rng(31 + fused)
    S_, STRIDE_ = (S, STRIDE) if not fused else (MAXB * 1024 + 1024, 1024)
    kp = random_bf16(rng, (S_, HKV, D))
    vp = random_bf16(rng, (S_, HKV, D))
    sentinel, dummy_row = S_ - 1, MAXB
    perm = rng.permutation(S_ - 1).astype(np.int32)          # the sentinel is never a request slot
    table = np.zeros((MAXB + 1, STRIDE_), np.int32)
    for r in range(MAXB):
        if fused:        # disjoint rows
            table[r] = perm[r * STRIDE_:(r + 1) * STRIDE_]
        else:            # rows overlapping by half
            table[r] = perm[r * STRIDE_ // 2: r * STRIDE_ // 2 + STRIDE_] \
                if (r + 2) * STRIDE_ // 2 <= S_ - 1 else perm[(r * 997) % (S_ - 1 - STRIDE_):][:STRIDE_]
    table[dummy_row, 0] = sentinel
    k_dev, v_dev, pt_dev = up(kp), up(vp), up(table)
    g = msgl.DecodeGraph(k_dev, v_dev, pt_dev, HQ, MAXB, STRIDE_, SCALE, dummy_row, sentinel,
                         fused_store=fused)
    assert [g.bucket(b) for b in (1, 2, 3, 4, 5, 9, 17, 63, 64)] == [1, 2, 4, 4, 8, 16, 24, 64, 64]
    with pytest.raises(msgl.MsglError):
        g.run(MAXB + 1)
    mirror_k, mirror_v = kp.copy(), vp.copy()
    mirror_k[sentinel] = 0          # create's warm-up runs fully padded batches
    mirror_v[sentinel] = 0
    lens_now = rng.integers(100, 2000 if not fused else 1000, MAXB)
    for step, bs in enumerate([64, 1, 3, 17, 24, 40, 8, 5]):
        banner(f"step {step}: batch {bs} -> bucket {g.bucket(bs)}")
        rows = rng.choice(MAXB, bs, replace=False).astype(np.int32)
        lens_now[rows] += 1
        seq = lens_now[rows].astype(np.int32)
        loc = table[rows, seq - 1].astype(np.int32)           # slot of each new token
        q = random_bf16(rng, (bs, HQ, D))
        kn, vn = random_bf16(rng, (bs, HKV, D)), random_bf16(rng, (bs, HKV, D))
        g.q[:bs].copy_(up(q)); g.k_new[:bs].copy_(up(kn)); g.v_new[:bs].copy_(up(vn))
        g.seq_lens[:bs].copy_(up(seq)); g.req_rows[:bs].copy_(up(rows)); g.out_loc[:bs].copy_(up(loc))
        out, lse = g.run(bs)
        torch.cuda.synchronize()
        o_graph, l_graph = bits(out).copy(), lse.cpu().numpy().copy()
        # the pool: live slots and (when padded) the zeroed sentinel, nothing else
        mirror_k[loc], mirror_v[loc] = kn, vn
        bucket = g.bucket(bs)
        if bucket > bs:
            mirror_k[sentinel] = 0
            mirror_v[sentinel] = 0
        check = np.unique(np.concatenate([loc, [sentinel], rng.integers(0, S_, 4000)]))
        assert np.array_equal(bits(k_dev)[check], mirror_k[check])
        assert np.array_equal(bits(v_dev)[check], mirror_v[check])
        # eager calls on the same padded batch give the same bits
        pad = bucket - bs
        pq = np.concatenate([q, np.zeros((pad, HQ, D), np.uint16)])
        pseq = np.concatenate([seq, np.ones(pad, np.int32)])
        prows = np.concatenate([rows, np.full(pad, dummy_row, np.int32)])
        eo, el = msgl.paged_decode(up(pq), k_dev, v_dev, pt_dev, up(pseq), STRIDE_, SCALE,
                                   req_rows=up(prows))
        torch.cuda.synchronize()
        assert np.array_equal(bits(eo)[:bs], o_graph)
        assert np.array_equal(el.cpu().numpy()[:bs], l_graph)
        # a second replay after eager work is identical
        out2, _ = g.run(bs)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out2), o_graph)
        sel = np.unique(np.linspace(0, bs - 1, min(bs, 6)).astype(int))
        ro, rl = oracle.paged_decode(q[sel], mirror_k, mirror_v, table, rows[sel], seq[sel], SCALE, HKV)
        t = torch.from_numpy(sel).cuda()
        assert_close(out[t], ro, f"graph step {step}")
        assert_lse_close(lse[t], rl, f"graph step {step}")
    g.close()
