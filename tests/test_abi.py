"""Host-side checks of the C ABI (no GPU): exports, struct layout, validation, workspace sizes.

Every call here fails validation (or is pure host arithmetic) before the
library touches the HIP runtime, so these run without a device.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import sparse_dual_chunk_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcasparse.h")

if not os.path.exists(S.LIB_PATH):
    pytest.skip("libdcasparse.so not built (python -m sparse_dual_chunk_amd.build)", allow_module_level=True)


MOE_HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read() + open(MOE_HEADER).read()
    return re.findall(r"DCA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == {"dca_workspace_size", "vs_index_build", "dca_sparse_prefill", "dca_key_cache_append",
                          "dca_sparse_prefill_cached", "dca_decode_workspace_size", "dca_decode", "dca_strerror",
                          "dca_chunk_cost_default", "dca_chunk_schedule", "dca_prefill_sequence_workspace_size",
                          "dca_prefill_sequence", "moe_workspace_size", "moe_forward",
                          "moe_pack_weights", "dca_paged_append", "dca_decode_paged", "dca_sparse_prefill_noalloc",
                          "dca_paged_prefill_workspace_size", "dca_sparse_prefill_paged",
                          "dca_prefill_sequence_paged_workspace_size", "dca_prefill_sequence_paged"}
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(S.lib(), n)


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "%s"\n'
        'int main(void){printf("%%zu", sizeof(dca_cfg));\n' % HEADER
        + "".join('printf(" %%zu", offsetof(dca_cfg, %s));\n' % f for f, _ in S.dca_cfg._fields_)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", str(prog), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(S.dca_cfg)
    assert vals[1:] == [getattr(S.dca_cfg, f).offset for f, _ in S.dca_cfg._fields_]


@pytest.mark.parametrize("name", ["dca_key_cache", "dca_chunk_cost", "dca_sequence_plan", "moe_cfg", "dca_paged_kv"])
def test_other_struct_layouts_match_header(tmp_path, name):
    st = getattr(S, name)
    prog = tmp_path / "st.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "%s"\n'
        'int main(void){printf("%%zu", sizeof(%s));\n' % (MOE_HEADER, name)
        + "".join('printf(" %%zu", offsetof(%s, %s));\n' % (name, f) for f, _ in st._fields_)
        + "return 0;}\n")
    exe = tmp_path / "st"
    subprocess.run(["gcc", str(prog), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(st)
    assert vals[1:] == [getattr(st, f).offset for f, _ in st._fields_]


def _cfg(**kw):
    base = dict(n_q=256, n_k=512, h_q=4, h_kv=2, dca_chunk=128, dca_local=32, rope_base=1e6, yarn_s=4.0)
    base.update(kw)
    return S.Config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), S.DCA_EUNSUPPORTED),
    (dict(dca_chunk=100), S.DCA_EUNSUPPORTED),
    (dict(dca_local=0), S.DCA_EUNSUPPORTED),
    (dict(dca_local=200), S.DCA_EUNSUPPORTED),
    (dict(h_q=5), S.DCA_EINVAL),
    (dict(n_q=0), S.DCA_EINVAL),
    (dict(n_k=100, n_q=200), S.DCA_EINVAL),
    (dict(n_k=500), S.DCA_EUNSUPPORTED),          # p0 = 244 is not a multiple of 64
    (dict(rope_base=1.0), S.DCA_EINVAL),
    (dict(yarn_s=0.0), S.DCA_EINVAL),
    (dict(vs_last_q=65), S.DCA_EUNSUPPORTED),
    (dict(vs_k_vertical=-1), S.DCA_EINVAL),
    (dict(split_k=-2), S.DCA_EINVAL),
])
def test_workspace_size_validation(kw, code):
    with pytest.raises(S.DcaError) as ei:
        S.dca_workspace_size(_cfg(**kw))
    assert ei.value.code == code


def test_workspace_size_grows_with_problem():
    a = S.dca_workspace_size(_cfg())
    b = S.dca_workspace_size(_cfg(n_q=256, n_k=4096))
    assert 0 < a < b
    # 1M-key layer: the K (hi, lo) copies dominate: 2 x 1M x 4 x 128 x 2 bytes
    big = S.dca_workspace_size(_cfg(n_q=32768, n_k=1 << 20, h_q=28, h_kv=4, dca_chunk=262144, dca_local=4096,
                                    vs_k_vertical=4096, vs_k_slash=16384))
    assert big >= 2 * (1 << 20) * 4 * 128 * 2


class _FakeTensor:
    """Stands in for a device tensor: a non-null address that is never dereferenced."""
    def __init__(self, n=1 << 20):
        self._n = n

    def data_ptr(self):
        return 0x1000

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def _call_prefill(cfg, positions=None, ws=None):
    t = _FakeTensor()
    S.dca_sparse_prefill(t, t, t, positions if positions is not None else _FakeTensor(), cfg, t,
                         ws or _FakeTensor(), stream=0)


def test_prefill_rejects_missing_positions_and_misaligned_chunks():
    """positions is a device array checked by a kernel; the host rejects a missing array and
    a chunk start p0 = n_k - n_q off a 64 boundary before anything is enqueued."""
    cfg = _cfg()
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)
    for fn in ("dca_sparse_prefill",):
        rc = getattr(S.lib(), fn)(0x1000, 0x1000, 0x1000, None, ctypes.byref(c), 0x1000)
        assert rc == S.DCA_EINVAL
    rc = S.lib().vs_index_build(0x1000, 0x1000, None, ctypes.byref(c), 0x1000, 0x1000)
    assert rc == S.DCA_EINVAL
    kc = S.dca_key_cache(k_hi=0x1000, k_lo=0x1000, k_flags=0x1000, capacity=1 << 20)
    rc = S.lib().dca_sparse_prefill_cached(0x1000, ctypes.byref(kc), 0x1000, None, ctypes.byref(c), 0x1000)
    assert rc == S.DCA_EINVAL
    with pytest.raises(S.DcaError) as ei:
        _call_prefill(_cfg(n_k=500))          # p0 = 244
    assert ei.value.code == S.DCA_EUNSUPPORTED


def test_noalloc_prefill_rejects_calls_beyond_its_static_scratch():
    """The allocation-free entry point checks the call's scratch need against its static
    array on the host, before any HIP call: a call needing more returns DCA_ESCRATCH."""
    big = _cfg(n_q=32768, n_k=32768 * 4, h_q=28, h_kv=4, dca_chunk=8192, dca_local=1024)
    assert S.dca_workspace_size(big) > S.DCA_STATIC_SCRATCH_BYTES
    c = big.to_c(workspace=None, workspace_bytes=0)
    rc = S.lib().dca_sparse_prefill_noalloc(0x1000, 0x1000, 0x1000, 0x1000, ctypes.byref(c), 0x1000)
    assert rc == S.DCA_ESCRATCH
    # missing positions or keys: rejected like the workspace entry point
    small = _cfg().to_c(workspace=None, workspace_bytes=0)
    assert S.lib().dca_sparse_prefill_noalloc(0x1000, 0x1000, 0x1000, None, ctypes.byref(small), 0x1000) == S.DCA_EINVAL
    assert S.lib().dca_sparse_prefill_noalloc(0x1000, None, 0x1000, 0x1000, ctypes.byref(small), 0x1000) == S.DCA_EINVAL


def test_paged_prefill_checks_the_pool_on_the_host():
    """The paged prefill needs room for the gathered values, a page table that holds n_k keys
    and pages of a multiple of 32 keys; each check fails before anything is enqueued."""
    cfg = _cfg()
    assert S.dca_paged_prefill_workspace_size(cfg) == S.dca_workspace_size(cfg) + cfg.n_k * cfg.h_kv * 128 * 2
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)

    def call(pages=64, page_keys=64, n_table=8, positions=0x1000):
        pk = S.dca_paged_kv(k_hi=0x1000, k_lo=0x1000, v=0x1000, k_flags=0x1000, n_pages=pages, page_keys=page_keys,
                            page_table=0x1000, n_table=n_table)
        return S.lib().dca_sparse_prefill_paged(0x1000, ctypes.byref(pk), positions, ctypes.byref(c), 0x1000)
    assert call(n_table=7) == S.DCA_EINVAL            # 7 * 64 < n_k = 512
    assert call(page_keys=48) == S.DCA_EUNSUPPORTED
    assert call(positions=None) == S.DCA_EINVAL
    assert S.lib().dca_sparse_prefill_paged(0x1000, None, 0x1000, ctypes.byref(c), 0x1000) == S.DCA_EINVAL


def test_prefill_rejects_small_or_missing_workspace():
    cfg = _cfg()
    need = S.dca_workspace_size(cfg)
    with pytest.raises(S.DcaError) as ei:
        _call_prefill(cfg, ws=_FakeTensor(need - 1))
    assert ei.value.code == S.DCA_EWORKSPACE


def test_prefill_rejects_one_sided_pattern_and_nulls():
    cfg = _cfg(vs_k_vertical=8, vs_k_slash=8)
    t = _FakeTensor(S.dca_workspace_size(cfg))
    with pytest.raises(S.DcaError) as ei:
        S.dca_sparse_prefill(t, t, t, _FakeTensor(), cfg, t, t, v_idx=t, s_off=None, stream=0)
    assert ei.value.code == S.DCA_EINVAL
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)
    rc = S.lib().dca_sparse_prefill(None, 0x1000, 0x1000, 0x1000, ctypes.byref(c), 0x1000)
    assert rc == S.DCA_EINVAL
    rc = S.lib().dca_sparse_prefill(0x1000, 0x1000, 0x1000, 0x1000, None, 0x1000)
    assert rc == S.DCA_EINVAL


def test_index_rejects_missing_outputs():
    cfg = _cfg(vs_k_vertical=8, vs_k_slash=8)
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 40)
    rc = S.lib().vs_index_build(0x1000, 0x1000, 0x1000, ctypes.byref(c), None, 0x1000)
    assert rc == S.DCA_EINVAL


def test_binding_checks_device_positions():
    """A torch positions tensor must be int32 and hold n_q entries before its address crosses."""
    torch = pytest.importorskip("torch")
    cfg = _cfg()
    with pytest.raises(ValueError):
        S._dev(torch.zeros(cfg.n_q, dtype=torch.int64), "positions", cfg.n_q * 4, "int32")
    with pytest.raises(ValueError):
        S._dev(torch.zeros(cfg.n_q - 1, dtype=torch.int32), "positions", cfg.n_q * 4, "int32")


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(S.dca_strerror(code), str) and S.dca_strerror(code)



# ---------------------------------------------------------------- decode entry points
def _dcfg(**kw):
    base = dict(n_q=1, n_k=5000, h_q=28, h_kv=4, dca_chunk=1024, dca_local=256, rope_base=1e7, yarn_s=4.0)
    base.update(kw)
    return S.Config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), S.DCA_EUNSUPPORTED),
    (dict(dca_chunk=96), S.DCA_EUNSUPPORTED),
    (dict(dca_local=2000), S.DCA_EUNSUPPORTED),
    (dict(n_q=0), S.DCA_EINVAL),
    (dict(n_q=65, n_k=100), S.DCA_EUNSUPPORTED),
    (dict(n_q=10, n_k=5), S.DCA_EINVAL),
    (dict(h_q=30), S.DCA_EINVAL),
    (dict(split_k=5000), S.DCA_EINVAL),
    (dict(yarn_s=-1.0), S.DCA_EINVAL),
])
def test_decode_workspace_size_validation(kw, code):
    with pytest.raises(S.DcaError) as ei:
        S.dca_decode_workspace_size(_dcfg(**kw))
    assert ei.value.code == code


def test_decode_workspace_holds_the_parts():
    # any positions work (no 64-row alignment); the parts' fp32 partials dominate
    small = S.dca_decode_workspace_size(_dcfg())
    big = S.dca_decode_workspace_size(_dcfg(n_k=1 << 20, dca_chunk=262144, dca_local=4096, n_q=4))
    assert 0 < small < big
    parts = (S.dca_decode_workspace_size(_dcfg(n_k=65536, split_k=64))
             - S.dca_decode_workspace_size(_dcfg(n_k=65536, split_k=32)))
    assert parts >= 32 * 28 * 128 * 4


class _FakeCache(S.KeyCache):
    def __init__(self, capacity):
        t = _FakeTensor()
        super().__init__(k_hi=t, k_lo=t, k_flags=t, capacity=capacity)


def test_decode_rejects_bad_calls_before_any_launch():
    cfg = _dcfg()
    t = _FakeTensor(S.dca_decode_workspace_size(cfg))
    with pytest.raises(S.DcaError) as ei:                      # cache smaller than n_k
        S.dca_decode(t, _FakeCache(4999), t, cfg, t, t, stream=0)
    assert ei.value.code == S.DCA_EINVAL
    with pytest.raises(S.DcaError) as ei:                      # workspace too small
        S.dca_decode(t, _FakeCache(5000), t, cfg, t, _FakeTensor(t.numel() - 1), stream=0)
    assert ei.value.code == S.DCA_EWORKSPACE
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30, v_idx=0x1000)
    kc = _FakeCache(5000).to_c()
    assert S.lib().dca_decode(0x1000, ctypes.byref(kc), 0x1000, ctypes.byref(c), 0x1000) == S.DCA_EINVAL
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)
    assert S.lib().dca_decode(0x1000, None, 0x1000, ctypes.byref(c), 0x1000) == S.DCA_EINVAL


def test_key_cache_append_validation():
    cfg = _dcfg()
    t = _FakeTensor()
    for j0, n, cap, code in [(-1, 4, 100, S.DCA_EINVAL), (0, 0, 100, S.DCA_EINVAL), (90, 20, 100, S.DCA_EINVAL)]:
        c = cfg.to_c(stream=0)
        kc = _FakeCache(cap).to_c()
        assert S.lib().dca_key_cache_append(0x1000, j0, n, ctypes.byref(c), ctypes.byref(kc)) == code
    c = _dcfg(dca_chunk=100).to_c(stream=0)
    kc = _FakeCache(100).to_c()
    assert S.lib().dca_key_cache_append(0x1000, 0, 10, ctypes.byref(c), ctypes.byref(kc)) == S.DCA_EUNSUPPORTED



def test_cached_prefill_rejects_small_cache_before_any_launch():
    cfg = _cfg()
    t = _FakeTensor(S.dca_workspace_size(cfg))
    with pytest.raises(S.DcaError) as ei:
        S.dca_sparse_prefill_cached(t, _FakeCache(511), t, _FakeTensor(), cfg, t, t, stream=0)
    assert ei.value.code == S.DCA_EINVAL
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)
    assert S.lib().dca_sparse_prefill_cached(0x1000, None, 0x1000, 0x1000, ctypes.byref(c), 0x1000) == S.DCA_EINVAL


# ---- whole-prompt chunked prefill
def _scfg(n=960, **kw):
    return _cfg(n_q=n, n_k=n, **kw)


def test_sequence_workspace_size_and_slots():
    cfg = _scfg(vs_k_vertical=24, vs_k_slash=40)
    bounds = [0, 320, 704, 960]
    one = S.dca_prefill_sequence_workspace_size(cfg, bounds, True, overlap=False)
    two = S.dca_prefill_sequence_workspace_size(cfg, bounds, True, overlap=True)
    assert two == 2 * one
    # one slot holds the largest chunk call's workspace
    biggest = max(S.dca_workspace_size(_cfg(n_q=b - a, n_k=b, vs_k_vertical=24, vs_k_slash=40))
                  for a, b in zip(bounds[:-1], bounds[1:]))
    assert one >= biggest


@pytest.mark.parametrize("bounds,code", [([0, 320, 900], S.DCA_EINVAL),        # does not end at n
                                         ([0, 320, 320, 960], S.DCA_EINVAL),   # empty chunk
                                         ([0, 100, 960], S.DCA_EUNSUPPORTED),  # chunk start not a multiple of 64
                                         ([64, 960], S.DCA_EINVAL)])           # does not start at 0
def test_sequence_rejects_bad_bounds(bounds, code):
    with pytest.raises(S.DcaError) as ei:
        S.dca_prefill_sequence_workspace_size(_scfg(), bounds, False, overlap=False)
    assert ei.value.code == code


def test_sequence_rejects_bad_calls_before_any_launch():
    cfg = _scfg()
    bounds = [0, 320, 960]
    ws = S.dca_prefill_sequence_workspace_size(cfg, bounds, False, overlap=False)
    t = _FakeTensor(ws)
    # too small a workspace, too small a cache, n_q != n_k, a pattern pointer in cfg
    with pytest.raises(S.DcaError) as ei:
        S.dca_prefill_sequence(t, t, t, bounds, cfg, _FakeCache(960), t, _FakeTensor(ws - 256), sparse=False,
                               stream=0)
    assert ei.value.code == S.DCA_EWORKSPACE
    with pytest.raises(S.DcaError) as ei:
        S.dca_prefill_sequence(t, t, t, bounds, cfg, _FakeCache(959), t, t, sparse=False, stream=0)
    assert ei.value.code == S.DCA_EINVAL
    with pytest.raises(S.DcaError) as ei:
        S.dca_prefill_sequence(t, t, t, bounds, _cfg(n_q=900, n_k=960), _FakeCache(960), t, t, sparse=False,
                               stream=0)
    assert ei.value.code == S.DCA_EINVAL
    p, _keep = S._seq_plan(bounds, False)
    c = cfg.to_c(workspace=0x1000, workspace_bytes=ws, stream=0, v_idx=0x2000)
    kc = _FakeCache(960).to_c()
    assert S.lib().dca_prefill_sequence(0x1000, 0x1000, 0x1000, ctypes.byref(p), ctypes.byref(c), ctypes.byref(kc),
                                        0x1000) == S.DCA_EINVAL


# ---- fused MoE layer
def _mcfg(**kw):
    base = dict(n_tokens=64, n_experts=64, top_k=8, d_model=3584, d_ff=2560)
    base.update(kw)
    return S.MoeConfig(**base)


@pytest.mark.parametrize("kw,code", [(dict(n_tokens=0), S.DCA_EINVAL), (dict(top_k=0), S.DCA_EINVAL),
                                     (dict(top_k=65), S.DCA_EUNSUPPORTED), (dict(n_experts=1024), S.DCA_EUNSUPPORTED),
                                     (dict(d_model=3500), S.DCA_EUNSUPPORTED), (dict(d_ff=64), S.DCA_EUNSUPPORTED)])
def test_moe_workspace_size_validation(kw, code):
    with pytest.raises(S.DcaError) as ei:
        S.moe_workspace_size(_mcfg(**kw))
    assert ei.value.code == code


def test_moe_workspace_holds_activations_and_outputs():
    n = S.moe_workspace_size(_mcfg())
    slots = 64 * 8
    assert n >= slots * 2560 * 2 + slots * 3584 * 4 + slots * 4 + 65 * 4


def test_moe_rejects_bad_calls_before_any_launch():
    cfg = _mcfg()
    t = _FakeTensor(S.moe_workspace_size(cfg))
    small = _FakeTensor(S.moe_workspace_size(cfg) - 256)
    with pytest.raises(S.DcaError) as ei:
        S.moe_forward(t, t, t, t, t, cfg, t, small, stream=0)
    assert ei.value.code == S.DCA_EWORKSPACE
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 40, stream=0)
    assert S.lib().moe_forward(0x1000, None, 0x1000, 0x1000, 0x1000, ctypes.byref(c), 0x1000) == S.DCA_EINVAL


def test_moe_pack_rejects_overlap_and_bad_shapes():
    cfg = _mcfg(n_experts=2, d_model=256, d_ff=128)
    c = cfg.to_c(stream=0)
    n13 = 2 * 2 * 128 * 256 * 2
    # packed copy overlapping its source
    assert S.lib().moe_pack_weights(0x100000, 0x900000, ctypes.byref(c), 0x100000 + n13 // 2, 0xA00000) == S.DCA_EINVAL
    c2 = _mcfg(d_ff=100).to_c(stream=0)
    assert S.lib().moe_pack_weights(0x1000, 0x2000, ctypes.byref(c2), 0x3000, 0x4000) == S.DCA_EUNSUPPORTED


# ---- paged cache
class _FakePaged(S.PagedKV):
    def __init__(self, n_pages, page_keys, n_table):
        t = _FakeTensor()
        super().__init__(k_hi=t, k_lo=t, v=t, k_flags=t, page_table=_FakeTensor(n_table), n_pages=n_pages,
                         page_keys=page_keys)

    def to_c(self):
        c = super().to_c()
        c.n_table = self.page_table.numel()
        return c


@pytest.mark.parametrize("n_pages,page_keys,n_table,code", [(8, 48, 8, S.DCA_EUNSUPPORTED),   # not a multiple of 32
                                                             (8, 0, 8, S.DCA_EUNSUPPORTED),
                                                             (0, 64, 8, S.DCA_EINVAL),
                                                             (8, 64, 12, S.DCA_EINVAL),      # 768 < 800 keys
                                                             (1 << 20, 1024, 1, S.DCA_EUNSUPPORTED)])  # pool > 4 GiB
def test_paged_decode_validation(n_pages, page_keys, n_table, code):
    cfg = _dcfg(n_q=2, n_k=800)
    t = _FakeTensor(S.dca_decode_workspace_size(cfg))
    with pytest.raises(S.DcaError) as ei:
        S.dca_decode_paged(t, _FakePaged(n_pages, page_keys, n_table), cfg, t, t, stream=0)
    assert ei.value.code == code


def test_paged_append_validation():
    cfg = _dcfg()
    c = cfg.to_c(stream=0)
    for j0, n, code in [(-1, 4, S.DCA_EINVAL), (0, 0, S.DCA_EINVAL), (600, 41, S.DCA_EINVAL)]:
        kc = _FakePaged(8, 64, 10).to_c()                        # 640 keys of table
        assert S.lib().dca_paged_append(0x1000, 0x1000, j0, n, ctypes.byref(c), ctypes.byref(kc)) == code
    kc = _FakePaged(8, 64, 10).to_c()
    assert S.lib().dca_paged_append(0x1000, None, 0, 4, ctypes.byref(c), ctypes.byref(kc)) == S.DCA_EINVAL


# ---- the binding's checks of torch tensors (before any pointer crosses the boundary)
def test_binding_checks_tensors_before_the_call():
    torch = pytest.importorskip("torch")
    cfg = _cfg()                                   # n_q 256, n_k 512, h_q 4, h_kv 2
    pos = _FakeTensor()
    ws = _FakeTensor(S.dca_workspace_size(cfg))
    k = torch.zeros((512, 2, 128), dtype=torch.int16)

    def call(**kw):                                # fakes (unchecked) except the tensor under test
        a = {n: _FakeTensor() for n in ("q", "k", "v", "out")}
        a.update(kw)
        S.dca_sparse_prefill(a["q"], a["k"], a["v"], pos, cfg, a["out"], ws, stream=0)

    with pytest.raises(ValueError, match="q: needs raw bfloat16"):
        call(q=torch.zeros((256, 4, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="k: the tensor must be contiguous"):
        call(k=torch.zeros((2, 512, 128), dtype=torch.int16).transpose(0, 1))
    with pytest.raises(ValueError, match="v: holds"):
        call(v=k[:511])
    with pytest.raises(ValueError, match="out: needs a device tensor"):
        call(out=torch.zeros((256, 4, 128), dtype=torch.bfloat16))   # right size, host memory
    with pytest.raises(ValueError, match="lse_out: needs float32"):
        S.dca_sparse_prefill(_FakeTensor(), _FakeTensor(), _FakeTensor(), pos, cfg, _FakeTensor(), ws,
                             lse_out=torch.zeros((4, 256), dtype=torch.float64), stream=0)
    m = _mcfg(n_tokens=4, n_experts=8, top_k=2, d_model=256, d_ff=128)
    with pytest.raises(ValueError, match="topk_ids: needs int32"):
        S.moe_forward(_FakeTensor(), torch.zeros((4, 2), dtype=torch.int64), _FakeTensor(), _FakeTensor(),
                      _FakeTensor(), m, _FakeTensor(), _FakeTensor(1 << 30), stream=0)
