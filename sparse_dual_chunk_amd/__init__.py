"""Python binding of libdcasparse.so: DCA + vertical-slash sparse prefill attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of the library; torch provides device memory and the stream.  If the
library has not been built the import of :func:`lib` fails loudly; there is no
CPU fallback.

Names follow the C ABI in ``include/dcasparse.h``:

* :func:`dca_workspace_size`
* :func:`vs_index_build`
* :func:`dca_sparse_prefill`
* :func:`dca_key_cache_append`
* :func:`dca_sparse_prefill_cached`
* :func:`dca_decode_workspace_size`
* :func:`dca_decode`
* :func:`dca_paged_append`
* :func:`dca_decode_paged`
* :func:`dca_chunk_cost_default`
* :func:`dca_chunk_schedule`
* :func:`dca_prefill_sequence_workspace_size`
* :func:`dca_prefill_sequence`
* :func:`dca_strerror`

and ``include/moe.h`` (the fused MoE layer, in the same library):

* :func:`moe_workspace_size`
* :func:`moe_pack_weights`
* :func:`moe_forward`
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import sys
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdcasparse.so")

DCA_OK = 0
DCA_EINVAL = -1
DCA_EUNSUPPORTED = -2
DCA_EWORKSPACE = -3
DCA_EHIP = -4
DCA_ESCRATCH = -5
DCA_STATIC_SCRATCH_BYTES = 256 << 20
DCA_STAGE_COUNT = 4
STAGES = ("rotate", "plan", "attention", "lse_merge")


class dca_cfg(ctypes.Structure):
    """Mirror of ``struct dca_cfg`` (field order and types as in the header)."""
    _fields_ = [
        ("n_q", ctypes.c_int32),
        ("n_k", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dca_chunk", ctypes.c_int32),
        ("dca_local", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("yarn_s", ctypes.c_double),
        ("vs_last_q", ctypes.c_int32),
        ("vs_k_vertical", ctypes.c_int32),
        ("vs_k_slash", ctypes.c_int32),
        ("v_idx", ctypes.c_void_p),
        ("s_off", ctypes.c_void_p),
        ("lse_out", ctypes.c_void_p),
        ("cover_pairs", ctypes.c_void_p),
        ("precise_norm", ctypes.c_float),
        ("split_k", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
        ("slash_exact", ctypes.c_int32),
        ("vs_k_per_head", ctypes.c_void_p),
        ("attended_pairs", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class dca_key_cache(ctypes.Structure):
    """Mirror of ``struct dca_key_cache``."""
    _fields_ = [
        ("k_hi", ctypes.c_void_p),
        ("k_lo", ctypes.c_void_p),
        ("k_flags", ctypes.c_void_p),
        ("capacity", ctypes.c_int32),
    ]


class dca_paged_kv(ctypes.Structure):
    """Mirror of ``struct dca_paged_kv``."""
    _fields_ = [
        ("k_hi", ctypes.c_void_p),
        ("k_lo", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_flags", ctypes.c_void_p),
        ("n_pages", ctypes.c_int32),
        ("page_keys", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("n_table", ctypes.c_int32),
    ]


class dca_chunk_cost(ctypes.Structure):
    """Mirror of ``struct dca_chunk_cost``."""
    _fields_ = [
        ("per_call", ctypes.c_double),
        ("per_row", ctypes.c_double),
        ("per_index_key", ctypes.c_double),
        ("per_pair", ctypes.c_double),
        ("cover_cap", ctypes.c_int64),
    ]


class dca_sequence_plan(ctypes.Structure):
    """Mirror of ``struct dca_sequence_plan``."""
    _fields_ = [
        ("bounds", ctypes.c_void_p),
        ("n_chunks", ctypes.c_int32),
        ("sparse", ctypes.c_int32),
        ("index_stream", ctypes.c_void_p),
        ("chunk_events", ctypes.c_void_p),
        ("index_events", ctypes.c_void_p),
        ("cover_pairs", ctypes.c_void_p),
    ]


class moe_cfg(ctypes.Structure):
    """Mirror of ``struct moe_cfg``."""
    _fields_ = [
        ("n_tokens", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
    ]


MOE_STAGE_COUNT = 4
MOE_STAGES = ("sort", "gate_up", "down", "sum")


class DcaError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: error {code} ({dca_strerror(code)})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_dual_chunk_amd.build` "
                              "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        L.dca_workspace_size.argtypes = [ctypes.POINTER(dca_cfg), ctypes.POINTER(ctypes.c_size_t)]
        L.dca_workspace_size.restype = ctypes.c_int
        L.vs_index_build.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(dca_cfg),
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.vs_index_build.restype = ctypes.c_int
        L.dca_sparse_prefill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.POINTER(dca_cfg), ctypes.c_void_p]
        L.dca_sparse_prefill.restype = ctypes.c_int
        L.dca_sparse_prefill_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.POINTER(dca_cfg), ctypes.c_void_p]
        L.dca_sparse_prefill_noalloc.restype = ctypes.c_int
        L.dca_key_cache_append.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(dca_cfg),
                                           ctypes.POINTER(dca_key_cache)]
        L.dca_key_cache_append.restype = ctypes.c_int
        L.dca_sparse_prefill_cached.argtypes = [ctypes.c_void_p, ctypes.POINTER(dca_key_cache), ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.POINTER(dca_cfg), ctypes.c_void_p]
        L.dca_sparse_prefill_cached.restype = ctypes.c_int
        L.dca_decode_workspace_size.argtypes = [ctypes.POINTER(dca_cfg), ctypes.POINTER(ctypes.c_size_t)]
        L.dca_decode_workspace_size.restype = ctypes.c_int
        L.dca_decode.argtypes = [ctypes.c_void_p, ctypes.POINTER(dca_key_cache), ctypes.c_void_p,
                                 ctypes.POINTER(dca_cfg), ctypes.c_void_p]
        L.dca_decode.restype = ctypes.c_int
        L.dca_paged_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(dca_cfg), ctypes.POINTER(dca_paged_kv)]
        L.dca_paged_append.restype = ctypes.c_int
        L.dca_decode_paged.argtypes = [ctypes.c_void_p, ctypes.POINTER(dca_paged_kv), ctypes.POINTER(dca_cfg),
                                       ctypes.c_void_p]
        L.dca_decode_paged.restype = ctypes.c_int
        L.dca_chunk_cost_default.argtypes = [ctypes.POINTER(dca_cfg), ctypes.c_int32, ctypes.POINTER(dca_chunk_cost)]
        L.dca_chunk_cost_default.restype = ctypes.c_int
        L.dca_chunk_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(dca_chunk_cost), ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
        L.dca_chunk_schedule.restype = ctypes.c_int
        L.dca_prefill_sequence_workspace_size.argtypes = [ctypes.POINTER(dca_cfg), ctypes.POINTER(dca_sequence_plan),
                                                          ctypes.POINTER(ctypes.c_size_t)]
        L.dca_prefill_sequence_workspace_size.restype = ctypes.c_int
        L.dca_prefill_sequence.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(dca_sequence_plan), ctypes.POINTER(dca_cfg),
                                           ctypes.POINTER(dca_key_cache), ctypes.c_void_p]
        L.dca_prefill_sequence.restype = ctypes.c_int
        L.dca_paged_prefill_workspace_size.argtypes = [ctypes.POINTER(dca_cfg), ctypes.POINTER(ctypes.c_size_t)]
        L.dca_paged_prefill_workspace_size.restype = ctypes.c_int
        L.dca_sparse_prefill_paged.argtypes = [ctypes.c_void_p, ctypes.POINTER(dca_paged_kv), ctypes.c_void_p,
                                               ctypes.POINTER(dca_cfg), ctypes.c_void_p]
        L.dca_sparse_prefill_paged.restype = ctypes.c_int
        L.dca_prefill_sequence_paged_workspace_size.argtypes = [ctypes.POINTER(dca_cfg),
                                                                ctypes.POINTER(dca_sequence_plan),
                                                                ctypes.POINTER(ctypes.c_size_t)]
        L.dca_prefill_sequence_paged_workspace_size.restype = ctypes.c_int
        L.dca_prefill_sequence_paged.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.POINTER(dca_sequence_plan), ctypes.POINTER(dca_cfg),
                                                 ctypes.POINTER(dca_paged_kv), ctypes.c_void_p]
        L.dca_prefill_sequence_paged.restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [ctypes.POINTER(moe_cfg), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(moe_cfg), ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(moe_cfg), ctypes.c_void_p]
        L.moe_forward.restype = ctypes.c_int
        L.dca_strerror.argtypes = [ctypes.c_int]
        L.dca_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


@dataclasses.dataclass
class Config:
    """Python view of ``dca_cfg``; pointers are filled in by the calls."""
    n_q: int
    n_k: int
    h_q: int
    h_kv: int
    dca_chunk: int
    dca_local: int
    rope_base: float
    yarn_s: float
    head_dim: int = 128
    vs_last_q: int = 64
    vs_k_vertical: int = 0
    vs_k_slash: int = 0
    precise_norm: float = 0.0
    split_k: int = 0
    slash_exact: int = 0

    def to_c(self, **ptrs) -> dca_cfg:
        c = dca_cfg()
        for f in dataclasses.fields(self):
            setattr(c, f.name, getattr(self, f.name))
        for k, v in ptrs.items():
            setattr(c, k, v)
        return c


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _dev(t, name: str, nbytes: int = 0, dtype: Optional[str] = None) -> Optional[int]:
    """Address of a buffer that crosses the boundary.

    The library sees only the address, so a torch tensor is checked here:
    device memory, contiguous, the element type of its layout ("bf16": any
    2-byte type holding raw bfloat16 bits; else a torch dtype name such as
    "int32") and at least ``nbytes`` bytes.  A bad tensor raises ValueError
    before anything is enqueued.  Other objects exposing data_ptr() pass
    unchecked."""
    if t is None:
        return None
    torch = sys.modules.get("torch")
    if torch is not None and isinstance(t, torch.Tensor):
        if dtype == "bf16":
            if t.element_size() != 2 or (t.is_floating_point() and t.dtype != torch.bfloat16):
                raise ValueError(f"{name}: needs raw bfloat16 bits (int16, uint16 or bfloat16), got {t.dtype}")
        elif dtype is not None and t.dtype != getattr(torch, dtype):
            raise ValueError(f"{name}: needs {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: the tensor must be contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{name}: holds {have} bytes, the call's layout covers {nbytes}")
        if t.device.type != "cuda":
            raise ValueError(f"{name}: needs a device tensor, got one on {t.device}")
    return int(t.data_ptr())


def _ws(workspace) -> dict:
    """Workspace fields of a config: address and size (the library checks the size)."""
    return dict(workspace=_dev(workspace, "workspace"),
                workspace_bytes=workspace.numel() * workspace.element_size())


def _check_cache(cache: "KeyCache", cfg: "Config") -> None:
    row = cfg.h_kv * cfg.head_dim * 2
    _dev(cache.k_hi, "cache.k_hi", cache.capacity * row, "bf16")
    _dev(cache.k_lo, "cache.k_lo", cache.capacity * row, "bf16")
    _dev(cache.k_flags, "cache.k_flags", cfg.h_kv * ((cache.capacity + 31) // 32) * 4, "int32")


def _check_paged(cache: "PagedKV", cfg: "Config") -> None:
    pool = cache.n_pages * cfg.h_kv * cache.page_keys * cfg.head_dim * 2
    for nm in ("k_hi", "k_lo", "v"):
        _dev(getattr(cache, nm), "cache." + nm, pool, "bf16")
    _dev(cache.k_flags, "cache.k_flags", cache.n_pages * cfg.h_kv * (cache.page_keys // 32) * 4, "int32")
    _dev(cache.page_table, "cache.page_table", 0, "int32")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(stream)


def _positions(positions, n_q: int, stream: Optional[int]):
    """Device int32 positions of a call: a cuda int32 tensor is checked and passed as is;
    anything else is copied into a new device tensor (kept alive by the caller until the
    call has been enqueued; torch's allocator orders its reuse on the stream it was made on,
    and a call on another stream records it there)."""
    import torch
    if isinstance(positions, torch.Tensor):
        if positions.device.type == "cuda":
            return positions, _dev(positions, "positions", n_q * 4, "int32")
    elif hasattr(positions, "data_ptr"):
        return positions, _dev(positions, "positions", n_q * 4, "int32")
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(positions, dtype=np.int32))).cuda()
    if stream is not None and stream != int(torch.cuda.current_stream().cuda_stream):
        t.record_stream(torch.cuda.ExternalStream(stream))
    return t, _dev(t, "positions", n_q * 4, "int32")


def dca_strerror(code: int) -> str:
    return lib().dca_strerror(int(code)).decode()


def dca_workspace_size(cfg: Config) -> int:
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().dca_workspace_size(ctypes.byref(c), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_workspace_size")
    return int(n.value)


def vs_index_build(q, k, positions, cfg: Config, v_idx, s_off, workspace, stream=None, k_per_head=None,
                   status=None) -> None:
    """Vertical-slash index of one chunk; writes v_idx [h_q][k_v] and s_off [h_q][k_s] (int32, device).
    positions: device int32 tensor [n_q] (host arrays are uploaded); k_per_head: optional device
    int32 [h_q][2] per-head budgets (k_v, k_s); status: optional device int32 [1]."""
    st = _stream(stream)
    pos, pos_p = _positions(positions, cfg.n_q, st)
    hd2 = cfg.head_dim * 2
    c = cfg.to_c(**_ws(workspace), stream=st,
                 vs_k_per_head=_dev(k_per_head, "k_per_head", cfg.h_q * 8, "int32"),
                 status=_dev(status, "status", 4, "int32"))
    rc = lib().vs_index_build(_dev(q, "q", cfg.n_q * cfg.h_q * hd2, "bf16"),
                              _dev(k, "k", cfg.n_k * cfg.h_kv * hd2, "bf16"), pos_p, ctypes.byref(c),
                              _dev(v_idx, "v_idx", cfg.h_q * cfg.vs_k_vertical * 4, "int32"),
                              _dev(s_off, "s_off", cfg.h_q * cfg.vs_k_slash * 4, "int32"))
    if rc != DCA_OK:
        raise DcaError(rc, "vs_index_build")


def dca_sparse_prefill(q, k, v, positions, cfg: Config, out, workspace, v_idx=None, s_off=None, lse_out=None,
                       cover_pairs=None, stream=None, stage_events: Optional[Sequence[int]] = None,
                       attended_pairs=None, status=None) -> None:
    """DCA prefill attention of one chunk (dense when v_idx and s_off are None).
    positions: device int32 tensor [n_q] (host arrays are uploaded)."""
    st = _stream(stream)
    pos, pos_p = _positions(positions, cfg.n_q, st)
    ev_arr = None
    if stage_events is not None:
        ev_arr = (ctypes.c_void_p * (2 * DCA_STAGE_COUNT))(*[int(e) for e in stage_events])
    c = cfg.to_c(**_ws(workspace), stream=st,
                 v_idx=_dev(v_idx, "v_idx", cfg.h_q * cfg.vs_k_vertical * 4, "int32"),
                 s_off=_dev(s_off, "s_off", cfg.h_q * cfg.vs_k_slash * 4, "int32"),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 cover_pairs=_dev(cover_pairs, "cover_pairs", 8, "int64"),
                 attended_pairs=_dev(attended_pairs, "attended_pairs", 8, "int64"),
                 status=_dev(status, "status", 4, "int32"),
                 stage_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    qb, kb = cfg.n_q * cfg.h_q * cfg.head_dim * 2, cfg.n_k * cfg.h_kv * cfg.head_dim * 2
    rc = lib().dca_sparse_prefill(_dev(q, "q", qb, "bf16"), _dev(k, "k", kb, "bf16"), _dev(v, "v", kb, "bf16"),
                                  pos_p, ctypes.byref(c), _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_sparse_prefill")


def dca_sparse_prefill_noalloc(q, k, v, positions, cfg: Config, out, v_idx=None, s_off=None, lse_out=None,
                               cover_pairs=None, stream=None, attended_pairs=None, status=None) -> None:
    """dca_sparse_prefill with the library's static per-GPU scratch instead of a workspace
    (no allocation; calls that overlap in time on one GPU race)."""
    st = _stream(stream)
    pos, pos_p = _positions(positions, cfg.n_q, st)
    c = cfg.to_c(workspace=None, workspace_bytes=0, stream=st,
                 v_idx=_dev(v_idx, "v_idx", cfg.h_q * cfg.vs_k_vertical * 4, "int32"),
                 s_off=_dev(s_off, "s_off", cfg.h_q * cfg.vs_k_slash * 4, "int32"),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 cover_pairs=_dev(cover_pairs, "cover_pairs", 8, "int64"),
                 attended_pairs=_dev(attended_pairs, "attended_pairs", 8, "int64"),
                 status=_dev(status, "status", 4, "int32"))
    qb, kb = cfg.n_q * cfg.h_q * cfg.head_dim * 2, cfg.n_k * cfg.h_kv * cfg.head_dim * 2
    rc = lib().dca_sparse_prefill_noalloc(_dev(q, "q", qb, "bf16"), _dev(k, "k", kb, "bf16"),
                                          _dev(v, "v", kb, "bf16"), pos_p, ctypes.byref(c),
                                          _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_sparse_prefill_noalloc")


def config_for(w, chunk: int = 0, **overrides) -> Config:
    """Config of one prefill call of a workload description (see ``workloads``)."""
    p0, n_q = w.chunks[chunk]
    cfg = Config(n_q=n_q, n_k=p0 + n_q, h_q=w.h_q, h_kv=w.h_kv, dca_chunk=w.dca_chunk, dca_local=w.dca_local,
                 rope_base=w.rope_base, yarn_s=w.yarn_s, head_dim=w.head_dim, vs_last_q=w.vs_last_q,
                 vs_k_vertical=w.k_vertical, vs_k_slash=w.k_slash)
    for k2, v2 in overrides.items():
        setattr(cfg, k2, v2)
    return cfg


# ---------------------------------------------------------------- generation step (decode)
@dataclasses.dataclass
class KeyCache:
    """Device arrays of a rotated key cache (see ``struct dca_key_cache``)."""
    k_hi: object       # int16 tensor [capacity][h_kv][128]
    k_lo: object       # int16 tensor [capacity][h_kv][128]
    k_flags: object    # int32 tensor [h_kv][(capacity + 31) // 32], zero before the first append
    capacity: int

    @staticmethod
    def allocate(capacity: int, h_kv: int, head_dim: int = 128, device: str = "cuda") -> "KeyCache":
        import torch
        return KeyCache(k_hi=torch.empty((capacity, h_kv, head_dim), dtype=torch.int16, device=device),
                        k_lo=torch.empty((capacity, h_kv, head_dim), dtype=torch.int16, device=device),
                        k_flags=torch.zeros((h_kv, (capacity + 31) // 32), dtype=torch.int32, device=device),
                        capacity=capacity)

    def to_c(self) -> dca_key_cache:
        c = dca_key_cache()
        c.k_hi, c.k_lo, c.k_flags, c.capacity = _ptr(self.k_hi), _ptr(self.k_lo), _ptr(self.k_flags), self.capacity
        return c


def dca_key_cache_append(k, j0: int, cfg: Config, cache: KeyCache, stream=None) -> None:
    """Rotate keys j0 .. j0 + k.shape[0] - 1 (k: [n][h_kv][128] raw bf16 bits) into the cache."""
    c = cfg.to_c(stream=_stream(stream))
    _check_cache(cache, cfg)
    kc = cache.to_c()
    n = int(k.shape[0])
    rc = lib().dca_key_cache_append(_dev(k, "k", n * cfg.h_kv * cfg.head_dim * 2, "bf16"), int(j0), n,
                                    ctypes.byref(c), ctypes.byref(kc))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_key_cache_append")


def dca_decode_workspace_size(cfg: Config) -> int:
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().dca_decode_workspace_size(ctypes.byref(c), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_decode_workspace_size")
    return int(n.value)


def dca_decode(q, cache: KeyCache, v, cfg: Config, out, workspace, lse_out=None, stream=None,
               stage_events: Optional[Sequence[int]] = None) -> None:
    """Attention of the cfg.n_q newest tokens (q [n_q][h_q][128]) over cache keys 0 .. cfg.n_k - 1."""
    ev_arr = None
    if stage_events is not None:
        ev_arr = (ctypes.c_void_p * (2 * DCA_STAGE_COUNT))(*[int(e) for e in stage_events])
    c = cfg.to_c(**_ws(workspace), stream=_stream(stream),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 stage_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    _check_cache(cache, cfg)
    kc = cache.to_c()
    qb = cfg.n_q * cfg.h_q * cfg.head_dim * 2
    rc = lib().dca_decode(_dev(q, "q", qb, "bf16"), ctypes.byref(kc),
                          _dev(v, "v", cfg.n_k * cfg.h_kv * cfg.head_dim * 2, "bf16"), ctypes.byref(c),
                          _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_decode")


def dca_sparse_prefill_cached(q, cache: KeyCache, v, positions, cfg: Config, out, workspace, v_idx=None, s_off=None,
                              lse_out=None, cover_pairs=None, stream=None,
                              stage_events: Optional[Sequence[int]] = None, attended_pairs=None,
                              status=None) -> None:
    """dca_sparse_prefill with keys 0 .. cfg.n_k - 1 from a rotated key cache."""
    st = _stream(stream)
    pos, pos_p = _positions(positions, cfg.n_q, st)
    ev_arr = None
    if stage_events is not None:
        ev_arr = (ctypes.c_void_p * (2 * DCA_STAGE_COUNT))(*[int(e) for e in stage_events])
    c = cfg.to_c(**_ws(workspace), stream=st,
                 v_idx=_dev(v_idx, "v_idx", cfg.h_q * cfg.vs_k_vertical * 4, "int32"),
                 s_off=_dev(s_off, "s_off", cfg.h_q * cfg.vs_k_slash * 4, "int32"),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 cover_pairs=_dev(cover_pairs, "cover_pairs", 8, "int64"),
                 attended_pairs=_dev(attended_pairs, "attended_pairs", 8, "int64"),
                 status=_dev(status, "status", 4, "int32"),
                 stage_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    _check_cache(cache, cfg)
    kc = cache.to_c()
    qb = cfg.n_q * cfg.h_q * cfg.head_dim * 2
    rc = lib().dca_sparse_prefill_cached(_dev(q, "q", qb, "bf16"), ctypes.byref(kc),
                                         _dev(v, "v", cfg.n_k * cfg.h_kv * cfg.head_dim * 2, "bf16"), pos_p,
                                         ctypes.byref(c), _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_sparse_prefill_cached")


# ---------------------------------------------------------------- paged cache
@dataclasses.dataclass
class PagedKV:
    """A page pool plus one sequence's page table (see ``struct dca_paged_kv``)."""
    k_hi: object        # int16 [n_pages][h_kv][page_keys][128]
    k_lo: object
    v: object
    k_flags: object     # int32 [n_pages][h_kv][page_keys // 32], zero before the first append
    page_table: object  # int32 [n_table] (device)
    n_pages: int
    page_keys: int

    @staticmethod
    def allocate(n_pages: int, page_keys: int, h_kv: int, page_table, head_dim: int = 128,
                 device: str = "cuda") -> "PagedKV":
        import torch
        shape = (n_pages, h_kv, page_keys, head_dim)
        pt = torch.as_tensor(np.asarray(page_table, dtype=np.int32)).to(device)
        return PagedKV(k_hi=torch.empty(shape, dtype=torch.int16, device=device),
                       k_lo=torch.empty(shape, dtype=torch.int16, device=device),
                       v=torch.empty(shape, dtype=torch.int16, device=device),
                       k_flags=torch.zeros((n_pages, h_kv, page_keys // 32), dtype=torch.int32, device=device),
                       page_table=pt, n_pages=n_pages, page_keys=page_keys)

    def to_c(self) -> dca_paged_kv:
        c = dca_paged_kv()
        c.k_hi, c.k_lo, c.v, c.k_flags = _ptr(self.k_hi), _ptr(self.k_lo), _ptr(self.v), _ptr(self.k_flags)
        c.n_pages, c.page_keys = self.n_pages, self.page_keys
        c.page_table = _ptr(self.page_table)
        c.n_table = int(self.page_table.numel())
        return c


def dca_paged_append(k, v, j0: int, cfg: Config, cache: PagedKV, stream=None) -> None:
    """Rotate keys j0 .. j0 + k.shape[0] - 1 into their pages and copy their values."""
    c = cfg.to_c(stream=_stream(stream))
    _check_paged(cache, cfg)
    kc = cache.to_c()
    n = int(k.shape[0])
    kb = n * cfg.h_kv * cfg.head_dim * 2
    rc = lib().dca_paged_append(_dev(k, "k", kb, "bf16"), _dev(v, "v", kb, "bf16"), int(j0), n, ctypes.byref(c),
                                ctypes.byref(kc))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_paged_append")


def dca_decode_paged(q, cache: PagedKV, cfg: Config, out, workspace, lse_out=None, stream=None,
                     stage_events: Optional[Sequence[int]] = None) -> None:
    """dca_decode over a paged cache."""
    ev_arr = None
    if stage_events is not None:
        ev_arr = (ctypes.c_void_p * (2 * DCA_STAGE_COUNT))(*[int(e) for e in stage_events])
    c = cfg.to_c(**_ws(workspace), stream=_stream(stream),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 stage_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    _check_paged(cache, cfg)
    kc = cache.to_c()
    qb = cfg.n_q * cfg.h_q * cfg.head_dim * 2
    rc = lib().dca_decode_paged(_dev(q, "q", qb, "bf16"), ctypes.byref(kc), ctypes.byref(c),
                                _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_decode_paged")


def dca_paged_prefill_workspace_size(cfg: Config) -> int:
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().dca_paged_prefill_workspace_size(ctypes.byref(c), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_paged_prefill_workspace_size")
    return int(n.value)


def dca_sparse_prefill_paged(q, cache: PagedKV, positions, cfg: Config, out, workspace, v_idx=None, s_off=None,
                             lse_out=None, cover_pairs=None, stream=None, attended_pairs=None, status=None) -> None:
    """dca_sparse_prefill with keys and values 0 .. cfg.n_k - 1 of a sequence in a paged pool."""
    st = _stream(stream)
    pos, pos_p = _positions(positions, cfg.n_q, st)
    c = cfg.to_c(**_ws(workspace), stream=st,
                 v_idx=_dev(v_idx, "v_idx", cfg.h_q * cfg.vs_k_vertical * 4, "int32"),
                 s_off=_dev(s_off, "s_off", cfg.h_q * cfg.vs_k_slash * 4, "int32"),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"),
                 cover_pairs=_dev(cover_pairs, "cover_pairs", 8, "int64"),
                 attended_pairs=_dev(attended_pairs, "attended_pairs", 8, "int64"),
                 status=_dev(status, "status", 4, "int32"))
    _check_paged(cache, cfg)
    kc = cache.to_c()
    qb = cfg.n_q * cfg.h_q * cfg.head_dim * 2
    rc = lib().dca_sparse_prefill_paged(_dev(q, "q", qb, "bf16"), ctypes.byref(kc), pos_p, ctypes.byref(c),
                                        _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_sparse_prefill_paged")


# ---------------------------------------------------------------- whole-prompt chunked prefill
def dca_chunk_cost_default(cfg: Config, sparse: bool) -> dca_chunk_cost:
    """The library's MI355X cost coefficients (microseconds) for cfg's heads and budgets."""
    c = cfg.to_c()
    m = dca_chunk_cost()
    rc = lib().dca_chunk_cost_default(ctypes.byref(c), int(bool(sparse)), ctypes.byref(m))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_chunk_cost_default")
    return m


def chunk_cost(per_call=0.0, per_row=0.0, per_index_key=0.0, per_pair=0.0, cover_cap=0) -> dca_chunk_cost:
    m = dca_chunk_cost()
    m.per_call, m.per_row, m.per_index_key, m.per_pair, m.cover_cap = per_call, per_row, per_index_key, per_pair, \
        int(cover_cap)
    return m


def dca_chunk_schedule(n_tokens: int, n_chunks: int, max_rows: int, cost: dca_chunk_cost):
    """Equal-time chunk bounds: returns (bounds list of n_out + 1 ints, largest chunk cost)."""
    b = np.zeros(n_chunks + 1, dtype=np.int32)
    n_out = ctypes.c_int32(0)
    mx = ctypes.c_double(0.0)
    rc = lib().dca_chunk_schedule(int(n_tokens), int(n_chunks), int(max_rows), ctypes.byref(cost),
                                  b.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n_out), ctypes.byref(mx))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_chunk_schedule")
    return [int(x) for x in b[: n_out.value + 1]], float(mx.value)


def _seq_plan(bounds, sparse, index_stream=None, chunk_events=None, index_events=None, cover_pairs=None):
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int32))
    n = len(b) - 1
    keep = [b]
    p = dca_sequence_plan()
    p.bounds = b.ctypes.data_as(ctypes.c_void_p)
    p.n_chunks = n
    p.sparse = int(bool(sparse))
    p.index_stream = int(index_stream) if index_stream is not None else None
    for name, evs in (("chunk_events", chunk_events), ("index_events", index_events)):
        if evs is not None:
            arr = (ctypes.c_void_p * (2 * n))(*[int(e) for e in evs])
            keep.append(arr)
            setattr(p, name, ctypes.cast(arr, ctypes.c_void_p))
    p.cover_pairs = _dev(cover_pairs, "cover_pairs", 8 * n, "int64")
    return p, keep


def dca_prefill_sequence_workspace_size(cfg: Config, bounds, sparse: bool, overlap: bool) -> int:
    """Workspace bytes of dca_prefill_sequence (overlap: an index stream will be passed)."""
    p, _keep = _seq_plan(bounds, sparse, index_stream=1 if overlap else None)
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().dca_prefill_sequence_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_prefill_sequence_workspace_size")
    return int(n.value)


def dca_prefill_sequence(q, k, v, bounds, cfg: Config, cache: KeyCache, out, workspace, sparse: bool = True,
                         index_stream=None, lse_out=None, cover_pairs=None, chunk_events=None, index_events=None,
                         stream=None) -> None:
    """Chunked prefill of a whole prompt (cfg.n_q == cfg.n_k == its length) over the given chunk bounds.
    index_stream: a second stream (int handle) for the index builds, or None to run everything in order."""
    p, _keep = _seq_plan(bounds, sparse, index_stream, chunk_events, index_events, cover_pairs)
    c = cfg.to_c(**_ws(workspace), stream=_stream(stream),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"))
    _check_cache(cache, cfg)
    kc = cache.to_c()
    qb, kb = cfg.n_q * cfg.h_q * cfg.head_dim * 2, cfg.n_k * cfg.h_kv * cfg.head_dim * 2
    rc = lib().dca_prefill_sequence(_dev(q, "q", qb, "bf16"), _dev(k, "k", kb, "bf16"), _dev(v, "v", kb, "bf16"),
                                    ctypes.byref(p), ctypes.byref(c), ctypes.byref(kc), _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_prefill_sequence")


def dca_prefill_sequence_paged_workspace_size(cfg: Config, bounds, sparse: bool, overlap: bool) -> int:
    """Workspace bytes of dca_prefill_sequence_paged (overlap: an index stream will be passed)."""
    p, _keep = _seq_plan(bounds, sparse, index_stream=1 if overlap else None)
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().dca_prefill_sequence_paged_workspace_size(ctypes.byref(c), ctypes.byref(p), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_prefill_sequence_paged_workspace_size")
    return int(n.value)


def dca_prefill_sequence_paged(q, k, v, bounds, cfg: Config, cache: PagedKV, out, workspace, sparse: bool = True,
                               index_stream=None, lse_out=None, cover_pairs=None, chunk_events=None,
                               index_events=None, stream=None) -> None:
    """dca_prefill_sequence whose chunks append into and read from a paged pool."""
    p, _keep = _seq_plan(bounds, sparse, index_stream, chunk_events, index_events, cover_pairs)
    c = cfg.to_c(**_ws(workspace), stream=_stream(stream),
                 lse_out=_dev(lse_out, "lse_out", cfg.h_q * cfg.n_q * 4, "float32"))
    _check_paged(cache, cfg)
    kc = cache.to_c()
    qb, kb = cfg.n_q * cfg.h_q * cfg.head_dim * 2, cfg.n_k * cfg.h_kv * cfg.head_dim * 2
    rc = lib().dca_prefill_sequence_paged(_dev(q, "q", qb, "bf16"), _dev(k, "k", kb, "bf16"),
                                          _dev(v, "v", kb, "bf16"), ctypes.byref(p), ctypes.byref(c),
                                          ctypes.byref(kc), _dev(out, "out", qb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "dca_prefill_sequence_paged")


# ---------------------------------------------------------------- fused MoE layer (include/moe.h)
@dataclasses.dataclass
class MoeConfig:
    n_tokens: int
    n_experts: int
    top_k: int
    d_model: int
    d_ff: int

    def to_c(self, **ptrs) -> moe_cfg:
        c = moe_cfg()
        for f in dataclasses.fields(self):
            setattr(c, f.name, getattr(self, f.name))
        for k, v in ptrs.items():
            setattr(c, k, v)
        return c


def moe_workspace_size(cfg: MoeConfig) -> int:
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    rc = lib().moe_workspace_size(ctypes.byref(c), ctypes.byref(n))
    if rc != DCA_OK:
        raise DcaError(rc, "moe_workspace_size")
    return int(n.value)


def moe_pack_weights(w13, w2, cfg: MoeConfig, w13_packed, w2_packed, stream=None) -> None:
    """Write the packed weight layout moe_forward streams (same shapes as w13 / w2)."""
    c = cfg.to_c(stream=_stream(stream))
    wb = cfg.n_experts * 2 * cfg.d_ff * cfg.d_model * 2
    rc = lib().moe_pack_weights(_dev(w13, "w13", wb, "bf16"), _dev(w2, "w2", wb // 2, "bf16"), ctypes.byref(c),
                                _dev(w13_packed, "w13_packed", wb, "bf16"), _dev(w2_packed, "w2_packed", wb // 2, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "moe_pack_weights")


def moe_forward(x, topk_ids, topk_weights, w13_packed, w2_packed, cfg: MoeConfig, out, workspace, stream=None,
                stage_events: Optional[Sequence[int]] = None) -> None:
    """Fused MoE layer: out [T][d_model] bf16 from x, routing ids / weights and the packed expert weights."""
    ev_arr = None
    if stage_events is not None:
        ev_arr = (ctypes.c_void_p * (2 * MOE_STAGE_COUNT))(*[int(e) for e in stage_events])
    c = cfg.to_c(**_ws(workspace), stream=_stream(stream),
                 stage_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    xb, sb = cfg.n_tokens * cfg.d_model * 2, cfg.n_tokens * cfg.top_k * 4
    wb = cfg.n_experts * 2 * cfg.d_ff * cfg.d_model * 2
    rc = lib().moe_forward(_dev(x, "x", xb, "bf16"), _dev(topk_ids, "topk_ids", sb, "int32"),
                           _dev(topk_weights, "topk_weights", sb, "float32"),
                           _dev(w13_packed, "w13_packed", wb, "bf16"), _dev(w2_packed, "w2_packed", wb // 2, "bf16"),
                           ctypes.byref(c), _dev(out, "out", xb, "bf16"))
    if rc != DCA_OK:
        raise DcaError(rc, "moe_forward")
