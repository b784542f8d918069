"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/csa2.h, and rejects bad arguments with
the documented status before any HIP call is made."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

from fp4_kv_cache_csa2_amd import _lib


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_kv_cache_csa2_amd import build
        build.build()
    return _lib.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_version_and_status_strings(lib):
    assert lib.csa2_abi_version() == 3 == _lib.ABI_VERSION
    assert lib.csa2_status_string(_lib.CSA2_EMODE) == b"CSA2_EMODE"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _err(lib):
    return lib.csa2_last_error().decode()


def test_quantize_rejects_bad_D(lib):
    assert lib.csa2_fp4_quantize(FAKE, 0, 4, 24, FAKE, FAKE, None) == _lib.CSA2_EINVAL
    assert "multiple of 16" in _err(lib)
    assert lib.csa2_fp4_quantize(FAKE, 7, 4, 32, FAKE, FAKE, None) == _lib.CSA2_EINVAL
    assert lib.csa2_fp4_quantize(None, 0, 0, 32, None, None, None) == _lib.CSA2_OK  # empty: no-op


def test_topk_argument_errors(lib):
    assert lib.csa2_topk(FAKE, 4, 1000, 0, None, FAKE, None, 0, None) == _lib.CSA2_EINVAL
    assert lib.csa2_topk(FAKE, 4, 1000, 4096, None, FAKE, None, 0, None) == _lib.CSA2_EINVAL
    assert lib.csa2_topk(FAKE, 4, 1001, 16, FAKE, FAKE, None, 0, None) == _lib.CSA2_EINVAL  # pool needs n % 8 == 0
    # large rows need a workspace
    need = lib.csa2_topk_workspace_size(4, 1 << 20, 512)
    assert need > 0
    assert lib.csa2_topk(FAKE, 4, 1 << 20, 512, None, FAKE, None, 0, None) == _lib.CSA2_EWORKSPACE
    assert lib.csa2_topk(FAKE, 4, 1 << 20, 512, None, FAKE, FAKE, need - 1, None) == _lib.CSA2_EWORKSPACE
    assert lib.csa2_topk_workspace_size(64, 16384, 512) == 0  # one-workgroup path
    assert lib.csa2_topk_workspace_size(64, 32768, 512) == 0
    assert lib.csa2_topk_workspace_size(64, 32769, 512) > 0


def test_indexer_argument_errors(lib):
    k = _lib.IdxK(FAKE.value, None, 0, 0, 4096, 96)
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(k), FAKE, 4096, FAKE, None, None) == _lib.CSA2_EUNSUPPORTED
    k = _lib.IdxK(FAKE.value, None, 0, 0, 100, 128)
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(k), FAKE, 4096, FAKE, None, None) == _lib.CSA2_EINVAL
    assert "seq_stride" in _err(lib)
    kp = _lib.IdxK(FAKE.value, FAKE.value, 48, 10, 0, 128)  # page size not a power of two
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(kp), FAKE, 400, FAKE, None, None) == _lib.CSA2_EUNSUPPORTED
    kp = _lib.IdxK(FAKE.value, FAKE.value, 12, 10, 0, 128)  # not a multiple of 8
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(kp), FAKE, 100, FAKE, None, None) == _lib.CSA2_EINVAL
    kp = _lib.IdxK(FAKE.value, FAKE.value, 64, 2, 0, 128)   # 2 pages cannot hold 4096 entries
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(kp), FAKE, 4096, FAKE, None, None) == _lib.CSA2_EINVAL
    assert lib.csa2_index_full(FAKE, 1, 1, 0, ctypes.byref(k), FAKE, 100, FAKE, None, None) == _lib.CSA2_EINVAL
    # scores may be left out when block maxima are asked for, not both
    assert lib.csa2_index_full(FAKE, 1, 1, 8, ctypes.byref(k), FAKE, 100, None, None, None) == _lib.CSA2_EINVAL
    assert "block maxima" in _err(lib)


def test_attention_argument_errors(lib):
    kv = _lib.Fp4KV(FAKE.value, FAKE.value, None, 0, 0, 4096, 512)
    args = (FAKE, 1, 1, 1, 8, ctypes.byref(kv), FAKE, 512, 0.1, FAKE, FAKE, None, 0, None)
    assert lib.csa2_sparse_attn_fp4(*args) == _lib.CSA2_EUNSUPPORTED  # H = 8
    kv.D = 100
    assert lib.csa2_sparse_attn_fp4(FAKE, 1, 1, 1, 64, ctypes.byref(kv), FAKE, 512, 0.1, FAKE, FAKE, None, 0,
                                    None) == _lib.CSA2_EUNSUPPORTED
    # few rows split the keys over workgroups: a workspace is required
    assert lib.csa2_attn_workspace_size(4, 1, 64, 512) > 0
    assert lib.csa2_swa_attn(FAKE, 1, 4, 1, 64, 512, FAKE, 128, FAKE, 128, 0.1, 0, FAKE, FAKE, None, 0,
                             None) == _lib.CSA2_EWORKSPACE
    assert lib.csa2_swa_attn(FAKE, 1, 4, 1, 64, 512, FAKE, 128, FAKE, 0, 0.1, 0, FAKE, FAKE, None, 0,
                             None) == _lib.CSA2_EINVAL
    # a window longer than the ring would make two of its tokens share a row
    big = 1 << 30
    assert lib.csa2_swa_attn(FAKE, 1, 4, 1, 64, 512, FAKE, 100, FAKE, 128, 0.1, 0, FAKE, FAKE, FAKE, big,
                             None) == _lib.CSA2_EINVAL
    assert "ring" in _err(lib)


def _layer_args(ws_bytes=1 << 40):
    kv = _lib.Fp4KV(FAKE.value, FAKE.value, None, 0, 0, 4096, 512)
    kk = _lib.IdxK(FAKE.value, None, 0, 0, 4096, 128)
    a = _lib.LayerArgs(1, 1, 64, 8, 512, 2048, FAKE.value, 1, FAKE.value, FAKE.value, 128, FAKE.value, 128, 0.1,
                       FAKE.value, FAKE.value, ctypes.pointer(kv), ctypes.pointer(kk), FAKE.value, 4096, 0,
                       0x100000, ws_bytes)
    return a, kv, kk


def test_layer_mode_errors(lib):
    a, kv, kk = _layer_args()
    st = _lib.GroupState(FAKE.value, FAKE.value, 0, 0, 0, 0, None, 0, 0)
    assert lib.csa2_layer_forward(_lib.CSA2_REUSE, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EMODE
    assert "Reuse" in _err(lib)
    assert lib.csa2_layer_forward(_lib.CSA2_REINDEX, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EMODE
    st.has_idx = 1
    assert lib.csa2_layer_forward(_lib.CSA2_REINDEX, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EMODE
    assert lib.csa2_layer_forward(7, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EINVAL
    a.K = 0
    assert lib.csa2_layer_forward(_lib.CSA2_FULL, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EINVAL
    a, kv, kk = _layer_args(ws_bytes=16)
    assert lib.csa2_layer_forward(_lib.CSA2_FULL, ctypes.byref(a), ctypes.byref(st), None) == _lib.CSA2_EWORKSPACE
    assert st.has_idx == 1 and st.has_pool == 0  # failed calls leave the state alone


def test_layer_workspace_size_covers_parts(lib):
    n, rows = 1 << 20, 4
    total = lib.csa2_layer_workspace_size(rows, 1, 64, 512, n, 512, 2048)
    assert total >= rows * n * 4 + lib.csa2_topk_workspace_size(rows, n, 512) + lib.csa2_attn_workspace_size(
        rows, 1, 64, 512)


def test_replay_and_append_argument_errors(lib):
    arr = (_lib.P * 1)(FAKE.value)
    a = _lib.ReplayArgs(2, 8, 100, 512, 128, FAKE.value, 1, arr, arr, arr)  # d_model not a multiple of 32
    assert lib.csa2_swa_replay(ctypes.byref(a), None) == _lib.CSA2_EINVAL
    assert "multiple of 64" in _err(lib)
    a = _lib.ReplayArgs(2, 200, 128, 512, 128, FAKE.value, 1, arr, arr, arr)  # n > T
    assert lib.csa2_swa_replay(ctypes.byref(a), None) == _lib.CSA2_EINVAL
    a = _lib.ReplayArgs(2, 8, 128, 500, 128, FAKE.value, 1, arr, arr, arr)  # D not a multiple of 16
    assert lib.csa2_swa_replay(ctypes.byref(a), None) == _lib.CSA2_EINVAL
    a = _lib.ReplayArgs(2, 8, 128, 512, 128, FAKE.value, 49, arr, arr, arr)  # too many layers
    assert lib.csa2_swa_replay(ctypes.byref(a), None) == _lib.CSA2_EINVAL
    a = _lib.ReplayArgs(0, 8, 128, 512, 128, None, 1, None, None, None)  # nothing to do
    assert lib.csa2_swa_replay(ctypes.byref(a), None) == _lib.CSA2_OK
    kv = _lib.Fp4KV(FAKE.value, FAKE.value, None, 0, 0, 4096, 24)  # D not a multiple of 16
    ap = _lib.AppendArgs(1, FAKE.value, 0, FAKE.value, ctypes.pointer(kv), None, None, 0, None, None, 0, None)
    assert lib.csa2_append_token(ctypes.byref(ap), None) == _lib.CSA2_EINVAL
    kv = _lib.Fp4KV(FAKE.value, FAKE.value, None, 0, 0, 4096, 512)
    ap = _lib.AppendArgs(1, FAKE.value, 0, FAKE.value, ctypes.pointer(kv), None, None, 33, arr, arr, 128, FAKE.value)
    assert lib.csa2_append_token(ctypes.byref(ap), None) == _lib.CSA2_EINVAL  # too many layers
    ap = _lib.AppendArgs(1, FAKE.value, 0, FAKE.value, ctypes.pointer(kv), FAKE.value, None, 0, None, None, 0, None)
    assert lib.csa2_append_token(ctypes.byref(ap), None) == _lib.CSA2_EINVAL  # key without a K view
