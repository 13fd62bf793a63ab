"""The path under HIP graph capture (as a serving loop replays its step).

Each phase (store_kv, decode with the balanced split + merge, extend with
its planner) is captured once and replayed several times, with eager work
and synchronisations between the replays; every replay must reproduce the
eager results bit for bit.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_30_amd as msgl
from workloads import small_extend
from tests.gpu_util import Uploaded, bits

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_bitwise():
    print("[gpu-graph] mixed decode + extend under graph capture", flush=True)
    inp = small_extend(97, 32, 8, [(300, 129), (0, 70), (2000, 33)],
                       decode_lens=[17, 900, 1, 2500, 64], num_slots=16384)
    u = Uploaded(inp)
    B, hq = inp.num_decode, inp.num_q_heads
    need, _ = msgl.paged_decode_workspace_size(B, hq, inp.num_kv_heads, u.d_max)
    dws = msgl.alloc_workspace(need)
    ews = msgl.alloc_workspace(msgl.paged_extend_workspace_size(
        inp.num_extend, hq, inp.num_kv_heads, u.e_max, u.e_kv))
    dout = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    dlse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    eout = torch.empty((inp.ext_tokens, hq, 128), dtype=torch.bfloat16, device="cuda")
    else_ = torch.empty((inp.ext_tokens, hq), dtype=torch.float32, device="cuda")

    def step():
        u.store()
        u.decode(out=dout, lse=dlse, workspace=dws)
        u.extend(out=eout, lse=else_, workspace=ews)

    step()
    torch.cuda.synchronize()
    ref = [bits(dout), dlse.cpu().numpy().copy(), bits(eout), else_.cpu().numpy().copy()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work in between: scribble over the outputs and workspaces
        dout.fill_(7.0)
        eout.fill_(-3.0)
        dlse.zero_()
        else_.zero_()
        if dws is not None:
            dws.fill_(0xA5)
        ews.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits(dout), dlse.cpu().numpy(), bits(eout), else_.cpu().numpy()]
        assert np.array_equal(got[0], ref[0]), f"replay {rep}: decode out"
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32)), f"replay {rep}: decode lse"
        assert np.array_equal(got[2], ref[2]), f"replay {rep}: extend out"
        assert np.array_equal(got[3].view(np.uint32), ref[3].view(np.uint32)), f"replay {rep}: extend lse"
