"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and rejects bad arguments before any HIP
call. Fake device addresses are never dereferenced: every call here fails
validation first (and carries an undersized workspace as a second guard)."""

import ctypes
import os

import pytest

import long_context_kv_snapkv_amd as skv
from long_context_kv_snapkv_amd import snapkv as binding


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from long_context_kv_snapkv_amd.build import build
        build()
    return skv.load_library()


def test_exports_every_declared_function(lib):
    names = skv.header_functions()
    assert len(names) == 20, names
    assert "snapkv_compress_staged" in names
    assert "snapkv_compress_with_scores" in names
    assert "snapkv_compress_static" in names
    assert "snapkv_compress_from_lse" in names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert skv.snapkv_status_string(0) == "ok"
    assert skv.snapkv_status_string(1) == "invalid argument"
    assert skv.snapkv_status_string(2) == "unsupported"
    assert skv.snapkv_status_string(3) == "workspace too small"
    assert skv.snapkv_status_string(4) == "HIP error"
    assert skv.snapkv_status_string(99) == "unknown status"


def test_stage_names(lib):
    names = [skv.snapkv_stage_name(i) for i in range(skv.SNAPKV_NUM_STAGES)]
    assert names == ["snapkv_score_stats", "snapkv_score_vote", "snapkv_select", "snapkv_gather"]
    assert skv.snapkv_stage_name(-1) is None and skv.snapkv_stage_name(4) is None


FAKE = 0x10000  # 16-byte aligned address that is never dereferenced


def _compress(lib, **over):
    a = dict(batch=1, hq=4, hkv=2, d=128, q=FAKE, k=FAKE, v=FAKE, lens=[100], window=8,
             kernel=5, pool=0, budget=32, ok=FAKE, ov=FAKE, oi=FAKE, ws=FAKE, ws_bytes=1,
             stream=None)
    a.update(over)
    lens = (ctypes.c_int32 * max(1, len(a["lens"])))(*a["lens"])
    st = lib.snapkv_compress(a["batch"], a["hq"], a["hkv"], a["d"], a["q"], a["k"], a["v"],
                             lens, a["window"], a["kernel"], a["pool"], a["budget"], a["ok"],
                             a["ov"], a["oi"], a["ws"], a["ws_bytes"], a["stream"])
    return st, skv.snapkv_last_error()


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(oi=None), 1),
    (dict(q=FAKE + 2), 1), (dict(ok=FAKE + 8), 1),
    (dict(batch=0, lens=[]), 1), (dict(batch=257, lens=[10] * 257), 1),
    (dict(hq=5), 1), (dict(hkv=0), 1), (dict(window=0), 1),
    (dict(budget=8), 1), (dict(budget=3), 1),
    (dict(kernel=4), 1), (dict(kernel=0), 1), (dict(kernel=-3), 1), (dict(pool=2), 1),
    (dict(lens=[0]), 1), (dict(batch=2, lens=[5, -1]), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(hq=32, hkv=2, window=64), 2),
    (dict(kernel=2051), 2),
    (dict(ws_bytes=1), 3), (dict(ws=None, ws_bytes=10**9), 3), (dict(ws=FAKE + 4, ws_bytes=10**9), 3),
])
def test_compress_validation(lib, over, status):
    st, msg = _compress(lib, **over)
    assert st == status, msg
    assert msg


def test_window_scores_validation(lib):
    lens = (ctypes.c_int32 * 1)(100)
    st = lib.snapkv_window_scores(1, 4, 2, 128, FAKE, FAKE, lens, 8, 5, 0, FAKE, 91, FAKE,
                                  1 << 30, None)
    assert st == 1 and "scores_len" in skv.snapkv_last_error()
    st = lib.snapkv_window_scores(1, 4, 2, 128, FAKE, FAKE, lens, 8, 6, 0, FAKE, 92, FAKE,
                                  1, None)
    assert st == 1


def test_workspace_size_host_logic(lib):
    small = skv.snapkv_workspace_size(32, 8, 128, [16384], 32)
    big = skv.snapkv_workspace_size(32, 8, 128, [131072], 32)
    assert 0 < small < big
    # the pooled score vectors alone need 8 heads * P floats
    assert small >= 8 * (16384 - 32) * 4
    assert skv.snapkv_workspace_size(32, 8, 128, [16384, 100], 32) >= small
    with pytest.raises(skv.SnapKVError) as e:
        skv.snapkv_workspace_size(32, 8, 100, [16384], 32)
    assert e.value.status == skv.SNAPKV_ERR_UNSUPPORTED


def test_pooling_names_match_page_snippet():
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "glossary_snippet_params.json")) as f:
        p = json.load(f)
    assert skv.pool_mode_code(p["pooling"]) == skv.SNAPKV_POOL_AVG
    assert skv.pool_mode_code("maxpool") == skv.SNAPKV_POOL_MAX
    import inspect
    params = inspect.signature(skv.compress).parameters
    for name in ("window_size", "max_capacity_prompt", "kernel_size", "pooling"):
        assert name in params


def test_compress_from_lse_validation(lib):
    lens = (ctypes.c_int32 * 1)(100)

    def call(lse, ws_bytes=1, kernel=5):
        return lib.snapkv_compress_from_lse(1, 4, 2, 128, FAKE, FAKE, FAKE, lens, 8, lse,
                                            kernel, 0, 32, FAKE, FAKE, FAKE, FAKE,
                                            ws_bytes, None)

    assert call(None) == 1 and "window_lse" in skv.snapkv_last_error()
    assert call(FAKE + 2) == 1 and "window_lse" in skv.snapkv_last_error()
    assert call(FAKE, kernel=4) == 1
    # a 4-byte aligned normaliser buffer passes; the undersized workspace stops the call
    assert call(FAKE + 4) == 3


def test_compress_with_scores_validation(lib):
    lens = (ctypes.c_int32 * 1)(100)

    def call(sc=FAKE, slen=92, lse=None, ws_bytes=1):
        return lib.snapkv_compress_with_scores(1, 4, 2, 128, FAKE, FAKE, FAKE, lens, 8, lse, 5,
                                               0, 32, FAKE, FAKE, FAKE, sc, slen, FAKE,
                                               ws_bytes, None)

    assert call(sc=None) == 1 and "out_scores" in skv.snapkv_last_error()
    assert call(sc=FAKE + 4) == 1 and "out_scores" in skv.snapkv_last_error()
    assert call(slen=91) == 1 and "scores_len" in skv.snapkv_last_error()
    assert call(lse=FAKE + 2) == 1 and "window_lse" in skv.snapkv_last_error()
    # valid arguments: the undersized workspace stops the call
    assert call() == 3
    assert call(lse=FAKE + 4) == 3


def test_compress_static_rejects_before_any_device_call(lib):
    # no workspace argument: shapes whose scratch exceeds the fixed area are
    # refused on the host, like every other invalid argument
    def call(lens, hq=64, hkv=8, budget=1024, kernel=7, ok=FAKE):
        arr = (ctypes.c_int32 * len(lens))(*lens)
        return lib.snapkv_compress_static(len(lens), hq, hkv, 128, FAKE, FAKE, FAKE, arr, 64,
                                          kernel, 1, budget, ok, FAKE, FAKE, None)

    assert skv.SNAPKV_STATIC_SCRATCH_BYTES == 32 << 20
    assert call([131072] * 8) == 3 and "static area" in skv.snapkv_last_error()
    assert skv.snapkv_workspace_size(64, 8, 128, [131072] * 8, 64) > skv.SNAPKV_STATIC_SCRATCH_BYTES
    assert call([131072], budget=64) == 1
    assert call([131072], kernel=4) == 1
    assert call([131072], ok=None) == 1
    assert call([131072], hq=63) == 1
    # every benchmark workload fits the area
    for lens, hq, w in (([131072], 64, 64), ([32768] * 8, 32, 64), ([16384], 32, 32)):
        assert skv.snapkv_workspace_size(hq, 8, 128, lens, w) <= skv.SNAPKV_STATIC_SCRATCH_BYTES


def test_prefill_attention_validation(lib):
    def call(lens=(100,), hq=4, hkv=2, d=128, q=FAKE, out=FAKE, window=8, lse=FAKE, qw=FAKE):
        arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
        return lib.snapkv_prefill_attention(len(lens), hq, hkv, d, q, FAKE, FAKE, arr, window,
                                            out, lse, qw, None)

    assert call(q=None) == 1 and "NULL" in skv.snapkv_last_error()
    assert call(out=FAKE + 8) == 1
    assert call(qw=FAKE + 8) == 1
    assert call(lse=FAKE + 2) == 1 and "window_lse" in skv.snapkv_last_error()
    assert call(lens=()) == 1
    assert call(lens=(5, 0)) == 1
    assert call(hq=6, hkv=4) == 1
    assert call(window=0) == 1 and "window" in skv.snapkv_last_error()
    assert call(d=96) == 2
    assert call(lens=(10,) * 256, hq=512, hkv=8) == 2


def test_compress_int4_validation(lib):
    lens = (ctypes.c_int32 * 1)(100)

    def call(ks=FAKE, vs=FAKE, kq=FAKE, lse=None, ws_bytes=1):
        return lib.snapkv_compress_int4(1, 4, 2, 128, FAKE, FAKE, FAKE, lens, 8, lse, 5, 0, 32,
                                        kq, ks, FAKE, vs, FAKE, FAKE, ws_bytes, None)

    assert call(ks=None) == 1 and "scale" in skv.snapkv_last_error()
    assert call(vs=FAKE + 4) == 1
    assert call(kq=None) == 1
    assert call(lse=FAKE + 2) == 1 and "window_lse" in skv.snapkv_last_error()
    # valid pointers: the undersized workspace stops the call
    assert call() == 3
    assert call(lse=FAKE + 4) == 3


def test_decode_validation_and_workspace(lib):
    def ws(lens, layout=0, cap=1024, hq=32, hkv=8, d=128):
        arr = (ctypes.c_int32 * len(lens))(*lens)
        out = ctypes.c_size_t(0)
        st = lib.snapkv_decode_workspace_size(len(lens), hq, hkv, d, layout, cap, arr,
                                              ctypes.byref(out))
        return st, out.value

    st, small = ws([1024])
    assert st == 0 and small >= 8 * 4 * 130 * 4
    st, full = ws([16384], layout=1)
    assert st == 0 and full >= small
    assert ws([1025])[0] == 1          # above the capacity
    assert ws([0])[0] == 1
    assert ws([10], layout=2)[0] == 1
    assert ws([10], cap=0)[0] == 1
    assert ws([10], d=96)[0] == 2
    assert ws([10], hq=72, hkv=8)[0] == 2  # 9 query heads per KV head
    assert ws([10], hq=30, hkv=8)[0] == 1
    lens = (ctypes.c_int32 * 1)(100)
    st = lib.snapkv_decode_attention(1, 32, 8, 128, FAKE, FAKE, FAKE + 8, 0, 128, lens, FAKE,
                                     FAKE, 1 << 30, None)
    assert st == 1 and "aligned" in skv.snapkv_last_error()
    st = lib.snapkv_decode_attention(1, 32, 8, 128, FAKE, None, FAKE, 0, 128, lens, FAKE,
                                     FAKE, 1 << 30, None)
    assert st == 1
    st = lib.snapkv_decode_attention(1, 32, 8, 128, FAKE, FAKE, FAKE, 0, 128, lens, FAKE,
                                     FAKE, 1, None)
    assert st == 3
    # the timed form validates the same way before touching its events
    st = lib.snapkv_decode_attention_timed(1, 32, 8, 128, FAKE, FAKE, FAKE + 8, 0, 128, lens,
                                           FAKE, FAKE, 1 << 30, None, None, None)
    assert st == 1 and "aligned" in skv.snapkv_last_error()
    st = lib.snapkv_decode_attention_timed(1, 32, 8, 128, FAKE, FAKE, FAKE, 0, 128, lens, FAKE,
                                           FAKE, 1, None, None, None)
    assert st == 3


def test_decode_kernel_count(lib):
    # one launch while no prompt has more than 16 chunks of rows (chunks of
    # at least 128 rows, about 1024 chunk items per call), else two
    comp = skv.SNAPKV_CACHE_COMPRESSED
    packed = skv.SNAPKV_CACHE_PACKED
    assert skv.snapkv_decode_kernels(32, 8, 128, [1024], comp, 1024) == 1
    assert skv.snapkv_decode_kernels(32, 8, 128, [4096] * 8, comp, 4096) == 1
    assert skv.snapkv_decode_kernels(32, 8, 128, [16384], packed) == 2
    assert skv.snapkv_decode_kernels(8, 8, 64, [2048], packed) == 1   # 16 chunks of 128
    assert skv.snapkv_decode_kernels(8, 8, 64, [2049], packed) == 2   # 17
    with pytest.raises(skv.SnapKVError):
        skv.snapkv_decode_kernels(32, 8, 96, [10], comp, 16)


def test_select_kernels_host_logic(lib):
    # no device here (no CU count): nothing runs inside the gather and the
    # sliced selection takes its three kernels; a prefix of up to 32768
    # positions is one workgroup per head, a longer one is sliced, and a
    # call that compresses nothing selects nothing
    import torch
    if torch.cuda.is_available():
        pytest.skip("host logic without a device")
    assert skv.snapkv_select_kernels(32, 8, 128, [16384], 32, 1024) == 1
    assert skv.snapkv_select_kernels(32, 8, 128, [32768 + 32], 32, 1024) == 1
    assert skv.snapkv_select_kernels(32, 8, 128, [32768 + 33], 32, 1024) == 3
    assert skv.snapkv_select_kernels(64, 8, 128, [131072], 64, 1024) == 3
    assert skv.snapkv_select_kernels(32, 8, 128, [1000, 500], 32, 1024) == 0
    with pytest.raises(skv.SnapKVError):
        skv.snapkv_select_kernels(32, 8, 128, [16384], 32, 32)  # budget <= window
    n = ctypes.c_int32(0)
    lens = (ctypes.c_int32 * 1)(16384)
    assert (lib.snapkv_select_kernels(1, 32, 8, 128, lens, 32, 1024, None)
            == skv.SNAPKV_ERR_INVALID_ARGUMENT)


def test_score_kernels_host_logic(lib):
    # no device here: the fused score kernel needs the device's CU count, so
    # the two-kernel path is reported; shape errors follow snapkv_compress
    assert skv.snapkv_score_kernels(32, 8, 128, [16384], 32, 7) in (1, 2, 3)
    with pytest.raises(skv.SnapKVError):
        skv.snapkv_score_kernels(32, 8, 96, [16384], 32, 7)
    with pytest.raises(skv.SnapKVError):
        skv.snapkv_score_kernels(32, 8, 128, [16384], 32, 4)
    n = ctypes.c_int32(0)
    lens = (ctypes.c_int32 * 1)(16384)
    assert lib.snapkv_score_kernels(1, 32, 8, 128, lens, 32, 7, None) == skv.SNAPKV_ERR_INVALID_ARGUMENT
    assert lib.snapkv_score_kernels(1, 32, 8, 128, lens, 32, 7, ctypes.byref(n)) == skv.SNAPKV_OK


def test_gather_selects_host_logic(lib):
    # no device here: the selection inside the gather needs the device's CU
    # count, so the separate selection kernel is reported off the GPU
    assert skv.snapkv_gather_selects(32, 8, 128, [16384], 32, 1024) in (0, 1)
    with pytest.raises(skv.SnapKVError):
        skv.snapkv_gather_selects(32, 8, 128, [16384], 32, 32)
    lens = (ctypes.c_int32 * 1)(16384)
    assert lib.snapkv_gather_selects(1, 32, 8, 128, lens, 32, 1024, None) == skv.SNAPKV_ERR_INVALID_ARGUMENT
