"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

The oracle cannot redo a whole multi-GB batch in seconds, so each test runs the
full workload on the GPU and compares a sample of outputs the oracle computes
one by one: the longest and shortest requests plus a spread of others, and,
for extend, the first, last and spread query rows of every request.
store_kv is checked bit-exactly on every stored row and on a sample of the
untouched ones.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_30_amd as msgl
from workloads import make_config
from tests.gpu_util import Uploaded, bits, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"[gpu-config] {msg}", flush=True)
    sys.stdout.flush()


def check_store(u, inp, rng):
    k_bits = bits(u.k)
    v_bits = bits(u.v)
    loc = inp.out_loc
    assert np.array_equal(k_bits[loc], inp.k_new) and np.array_equal(v_bits[loc], inp.v_new)
    others = np.setdiff1d(rng.choice(inp.num_slots, 20000, replace=False), loc)
    assert np.array_equal(k_bits[others], inp.k_pool[others])
    assert np.array_equal(v_bits[others], inp.v_pool[others])
    return k_bits, v_bits


def stored_pool(inp):
    return oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)


def decode_sample(inp, n=10):
    L = inp.dec_seq_lens
    idx = {int(np.argmax(L)), int(np.argmin(L)), 0, len(L) - 1}
    idx.update(np.linspace(0, len(L) - 1, n).astype(int).tolist())
    return np.array(sorted(idx))


def check_decode(u, inp, kp, vp, tag):
    out, lse = u.decode()
    torch.cuda.synchronize()
    sel = decode_sample(inp)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 inp.dec_seq_lens[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(out[t], ro, f"{tag} decode")
    assert_lse_close(lse[t], rl, f"{tag} decode lse")
    return out


def check_extend(u, inp, kp, vp, tag):
    out, lse = u.extend()
    torch.cuda.synchronize()
    rows = []
    for r in range(inp.num_extend):
        base, E = int(inp.ext_q_offsets[r]), int(inp.ext_extend_lens[r])
        rows += [base, base + E - 1] + (base + np.linspace(0, E - 1, 6).astype(int)).tolist()
    rows = sorted(set(rows))
    ro, rl = oracle.paged_extend(inp.ext_q, kp, vp, inp.page_table, inp.ext_req_rows,
                                 inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                                 inp.sm_scale, inp.num_kv_heads, query_subset=rows)
    t = torch.tensor(rows, device="cuda")
    assert_close(out[t], ro[rows], f"{tag} extend")
    assert_lse_close(lse[t], rl[rows], f"{tag} extend lse")
    return out


@pytest.mark.parametrize("name", ["C2", "C4"])
def test_full_decode_config(name):
    banner(f"{name}: generate + upload")
    inp = make_config(name)
    u = Uploaded(inp)
    u.store()
    torch.cuda.synchronize()
    banner(f"{name}: store_kv check")
    check_store(u, inp, np.random.default_rng(1))
    kp, vp = stored_pool(inp)
    banner(f"{name}: decode (balanced split) vs oracle sample")
    check_decode(u, inp, kp, vp, name)


def test_full_extend_config_c3():
    banner("C3: generate + upload")
    inp = make_config("C3")
    u = Uploaded(inp)
    u.store()
    torch.cuda.synchronize()
    check_store(u, inp, np.random.default_rng(3))
    kp, vp = stored_pool(inp)
    banner("C3: extend vs oracle sample")
    planned = check_extend(u, inp, kp, vp, "C3")
    banner("C3: natural work order must be bit-identical to the planned one")
    natural, _ = u.extend(plan=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(planned), bits(natural))


def test_full_mixed_batch_c5_page16_and_page1():
    banner("C5b: generate + upload")
    inp = make_config("C5b")
    u = Uploaded(inp)
    u.store()
    torch.cuda.synchronize()
    check_store(u, inp, np.random.default_rng(5))
    kp, vp = stored_pool(inp)
    banner("C5b: decode + extend at page_size 16 vs oracle sample")
    od16 = check_decode(u, inp, kp, vp, "C5b")
    oe16 = check_extend(u, inp, kp, vp, "C5b")
    banner("C5b: same table at page_size 1 must be bit-identical")
    od1, _ = u.decode(page_size=1)
    oe1, _ = u.extend(page_size=1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(od16), bits(od1))
    assert np.array_equal(bits(oe16), bits(oe1))


def test_full_mixed_batch_c5a():
    banner("C5a: generate + upload")
    inp = make_config("C5a")
    u = Uploaded(inp)
    u.store()
    torch.cuda.synchronize()
    check_store(u, inp, np.random.default_rng(6))
    kp, vp = stored_pool(inp)
    banner("C5a: decode + extend vs oracle sample")
    check_decode(u, inp, kp, vp, "C5a")
    check_extend(u, inp, kp, vp, "C5a")
