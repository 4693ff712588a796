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


def _declared_functions():
    src = open(HEADER).read()
    return re.findall(r"DCA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == {"dca_workspace_size", "vs_index_build", "dca_sparse_prefill", "dca_strerror"}
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


def _call_prefill(cfg, positions, ws=None):
    t = _FakeTensor()
    S.dca_sparse_prefill(t, t, t, positions, cfg, t, ws or _FakeTensor(), stream=0)


def test_prefill_rejects_bad_positions_before_any_launch():
    cfg = _cfg()
    pos = np.arange(256, 512, dtype=np.int32)
    pos[10] += 1
    with pytest.raises(S.DcaError) as ei:
        _call_prefill(cfg, pos)
    assert ei.value.code == S.DCA_EINVAL
    with pytest.raises(S.DcaError) as ei:
        _call_prefill(cfg, np.arange(255, 511, dtype=np.int32))
    assert ei.value.code == S.DCA_EINVAL


def test_prefill_rejects_small_or_missing_workspace():
    cfg = _cfg()
    need = S.dca_workspace_size(cfg)
    with pytest.raises(S.DcaError) as ei:
        _call_prefill(cfg, np.arange(256, 512, dtype=np.int32), ws=_FakeTensor(need - 1))
    assert ei.value.code == S.DCA_EWORKSPACE


def test_prefill_rejects_one_sided_pattern_and_nulls():
    cfg = _cfg(vs_k_vertical=8, vs_k_slash=8)
    t = _FakeTensor(S.dca_workspace_size(cfg))
    with pytest.raises(S.DcaError) as ei:
        S.dca_sparse_prefill(t, t, t, np.arange(256, 512, dtype=np.int32), cfg, t, t, v_idx=t, s_off=None, stream=0)
    assert ei.value.code == S.DCA_EINVAL
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 30)
    pos = np.arange(256, 512, dtype=np.int32)
    rc = S.lib().dca_sparse_prefill(None, 0x1000, 0x1000, pos.ctypes.data_as(ctypes.c_void_p), ctypes.byref(c), 0x1000)
    assert rc == S.DCA_EINVAL
    rc = S.lib().dca_sparse_prefill(0x1000, 0x1000, 0x1000, pos.ctypes.data_as(ctypes.c_void_p), None, 0x1000)
    assert rc == S.DCA_EINVAL


def test_index_rejects_missing_outputs():
    cfg = _cfg(vs_k_vertical=8, vs_k_slash=8)
    t = _FakeTensor(S.dca_workspace_size(cfg))
    c = cfg.to_c(workspace=0x1000, workspace_bytes=1 << 40)
    pos = np.arange(256, 512, dtype=np.int32)
    rc = S.lib().vs_index_build(0x1000, 0x1000, pos.ctypes.data_as(ctypes.c_void_p), ctypes.byref(c), None, 0x1000)
    assert rc == S.DCA_EINVAL


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(S.dca_strerror(code), str) and S.dca_strerror(code)
