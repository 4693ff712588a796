"""Helpers shared by the GPU tests: device upload and calls through the C ABI."""
from __future__ import annotations

import numpy as np

import sparse_dual_chunk_amd as S


def dev(arr: np.ndarray):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def workspace(cfg: S.Config):
    import torch
    return torch.empty(S.dca_workspace_size(cfg), dtype=torch.uint8, device="cuda")


def run_prefill(inp: dict, cfg: S.Config, v_idx=None, s_off=None, with_lse=False, ws=None):
    """Upload inputs, call dca_sparse_prefill, return (out bf16 bits [n_q][h_q][d], lse or None)."""
    import torch
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    out = torch.empty(q.shape, dtype=torch.int16, device="cuda")
    lse = torch.empty((cfg.h_q, cfg.n_q), dtype=torch.float32, device="cuda") if with_lse else None
    vi = dev(np.asarray(v_idx, dtype=np.int32)) if v_idx is not None else None
    so = dev(np.asarray(s_off, dtype=np.int32)) if s_off is not None else None
    ws = workspace(cfg) if ws is None else ws
    S.dca_sparse_prefill(q, k, v, inp["positions"], cfg, out, ws, v_idx=vi, s_off=so, lse_out=lse)
    torch.cuda.synchronize()
    return host_u16(out), (lse.cpu().numpy() if lse is not None else None)


def run_index(inp: dict, cfg: S.Config, ws=None, budgets=None):
    import torch
    q, k = dev(inp["q"]), dev(inp["k"])
    vi = torch.empty((cfg.h_q, max(cfg.vs_k_vertical, 1)), dtype=torch.int32, device="cuda")
    so = torch.empty((cfg.h_q, max(cfg.vs_k_slash, 1)), dtype=torch.int32, device="cuda")
    ws = workspace(cfg) if ws is None else ws
    kh = dev(np.asarray(budgets, dtype=np.int32)) if budgets is not None else None
    S.vs_index_build(q, k, inp["positions"], cfg, vi, so, ws, k_per_head=kh)
    torch.cuda.synchronize()
    return vi.cpu().numpy()[:, :cfg.vs_k_vertical], so.cpu().numpy()[:, :cfg.vs_k_slash]


def oracle_cfg(cfg: S.Config) -> dict:
    return dict(h_q=cfg.h_q, h_kv=cfg.h_kv, dca_chunk=cfg.dca_chunk, dca_local=cfg.dca_local,
                rope_base=cfg.rope_base, yarn_s=cfg.yarn_s, vs_k_vertical=cfg.vs_k_vertical,
                vs_k_slash=cfg.vs_k_slash, vs_last_q=cfg.vs_last_q)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# Output tolerance for bf16 outputs against the fp64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def check_close(got_bits: np.ndarray, ref: np.ndarray, what: str):
    got = bf16_f64(got_bits)
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"
    return mx, mean
