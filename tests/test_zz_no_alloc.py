"""GPU test of msgl_store_kv_paged_decode_noalloc, the fused store + decode
entry point whose partial results live in the library's static device
scratch instead of a caller-provided workspace.

Each call is checked against msgl_store_kv_paged_decode (same kernels, a
torch-allocated workspace) on a separate copy of the same seeded input:
pools, outputs and lse bit-identical, and the outputs within the oracle's
tolerance on a sample of requests.  Two calls run back to back, the second
with a smaller batch (fewer requests, fewer heads, shorter keys), so the
second reads nothing the first left in the scratch.  A batch whose partials
exceed the scratch is rejected before any launch.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_30_amd as msgl
from workloads import small_decode
from tests.gpu_util import Uploaded, up, bits, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def run_pair(inp, split):
    d_lens = up(inp.dec_seq_lens)
    runs = []
    for noalloc in (False, True):
        u = Uploaded(inp)
        loc = up(inp.out_loc.astype(np.int64))
        fn = msgl.store_kv_paged_decode_noalloc if noalloc else msgl.store_kv_paged_decode
        out, lse = fn(u.dq, u.k, u.v, u.k_new, u.v_new, loc, u.pt, d_lens, u.d_max,
                      inp.sm_scale, req_rows=u.d_rows, split_tokens=split)
        runs.append((u, out, lse))
    torch.cuda.synchronize()
    (ua, oa, la), (ub, ob, lb) = runs
    assert torch.equal(ua.k.view(torch.int16), ub.k.view(torch.int16)), "K pools differ"
    assert torch.equal(ua.v.view(torch.int16), ub.v.view(torch.int16)), "V pools differ"
    assert np.array_equal(bits(oa), bits(ob)), "outputs differ"
    assert np.array_equal(la.cpu().numpy().view(np.uint32), lb.cpu().numpy().view(np.uint32))
    L = inp.dec_seq_lens
    sel = np.array(sorted({0, len(L) - 1, int(np.argmax(L)), int(np.argmin(L)), len(L) // 2}))
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 L[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(ob[t], ro, "no-alloc decode")
    assert_lse_close(lb[t], rl, "no-alloc decode lse")


@pytest.mark.parametrize("split", [0, 256])
def test_noalloc_matches_workspace_call_twice_second_smaller(split):
    rng = np.random.default_rng(2024 + split)
    big = rng.integers(512, 4097, 64)
    banner(f"split {split}: 64 requests, Hq 32 / Hkv 8, lens up to {int(big.max())}")
    run_pair(small_decode(300 + split, 32, 8, big, num_slots=1 << 19), split)
    small = [700, 1, 129, 33, 2000]
    banner(f"split {split}: 5 requests, Hq 16 / Hkv 8, lens {small}")
    run_pair(small_decode(301 + split, 16, 8, small, num_slots=1 << 13), split)


def test_noalloc_rejects_partials_beyond_the_scratch():
    banner("oversized batch rejected before launch")
    B, hq, hkv = 40000, 64, 8
    q = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1024, hkv, 128), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, hkv, 128), dtype=torch.bfloat16, device="cuda")
    loc = torch.zeros((B,), dtype=torch.int32, device="cuda")
    pt = torch.zeros((1, 64), dtype=torch.int32, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    rows = torch.zeros((B,), dtype=torch.int32, device="cuda")
    with pytest.raises(msgl.MsglError) as e:
        msgl.store_kv_paged_decode_noalloc(q, k, k.clone(), kn, kn.clone(), loc, pt, lens, 64,
                                           0.1, req_rows=rows)
    assert "MSGL_ERR_WORKSPACE" in str(e.value) and "scratch" in str(e.value)
    torch.cuda.synchronize()
