"""Helpers for the GPU parity tests: uploads, calls through the C ABI, checks."""

import numpy as np
import torch

import paged_kv_attention_30_amd as msgl

ATOL = 2e-2      # max abs error on bf16 attention outputs vs the fp64 oracle
RTOL_INF = 1e-2  # max abs error / max |reference| per output tensor
LSE_ATOL = 1e-3  # internal check on the log-sum-exp


def dev():
    return torch.device("cuda:0")


def up(a: np.ndarray) -> torch.Tensor:
    """numpy -> GPU tensor; uint16 arrays become bf16 with the same bits."""
    x = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        x = x.view(torch.int16).view(torch.bfloat16)
    return x.to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 GPU tensor -> uint16 numpy bits."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: torch.Tensor, ref: np.ndarray, what: str, mask=None):
    g = f64(got)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    rel = max_abs / scale if scale > 0 else max_abs
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert max_abs <= ATOL, f"{what}: max abs err {max_abs:.3e} > {ATOL}"
    assert rel <= RTOL_INF, f"{what}: max abs err / max |ref| = {rel:.3e} > {RTOL_INF}"
    return max_abs, rel


def assert_lse_close(got: torch.Tensor, ref: np.ndarray, what: str, mask=None):
    g = f64(got)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: lse infinities differ"
    if fin.any():
        d = float(np.abs(g[fin] - ref[fin]).max())
        assert d <= LSE_ATOL, f"{what}: lse max abs diff {d:.3e}"


class Uploaded:
    """One PagedInputs bundle on the GPU (pool pre-store)."""

    def __init__(self, inp):
        self.inp = inp
        self.k = up(inp.k_pool)
        self.v = up(inp.v_pool)
        self.pt = up(inp.page_table)
        self.out_loc = up(inp.out_loc)
        self.k_new = up(inp.k_new)
        self.v_new = up(inp.v_new)
        if inp.num_decode:
            self.dq = up(inp.dec_q)
            self.d_rows = up(inp.dec_req_rows)
            self.d_lens = up(inp.dec_seq_lens)
            self.d_max = int(inp.dec_seq_lens.max())
        if inp.num_extend:
            self.eq = up(inp.ext_q)
            self.e_rows = up(inp.ext_req_rows)
            self.e_pre = up(inp.ext_prefix_lens)
            self.e_ext = up(inp.ext_extend_lens)
            self.e_off = up(inp.ext_q_offsets)
            self.e_max = int(inp.ext_extend_lens.max())
            self.e_kv = int((inp.ext_prefix_lens + inp.ext_extend_lens).max())

    def store(self):
        msgl.store_kv(self.k, self.v, self.k_new, self.v_new, self.out_loc)

    def decode(self, split_tokens=0, page_size=None, **kw):
        ps = self.inp.page_size if page_size is None else page_size
        return msgl.paged_decode(self.dq, self.k, self.v, self.pt, self.d_lens, self.d_max,
                                 self.inp.sm_scale, req_rows=self.d_rows, page_size=ps,
                                 split_tokens=split_tokens, **kw)

    def extend(self, page_size=None, **kw):
        ps = self.inp.page_size if page_size is None else page_size
        return msgl.paged_extend(self.eq, self.k, self.v, self.pt, self.e_pre, self.e_ext,
                                 self.e_off, self.e_max, self.e_kv, self.inp.sm_scale,
                                 req_rows=self.e_rows, page_size=ps, **kw)
