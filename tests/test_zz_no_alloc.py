"""snapkv_compress_static, the entry point that allocates nothing: its
intermediates go to the library's fixed scratch area. Called through the C
ABI, its outputs must equal snapkv_compress's (with a caller workspace) bit
for bit, on two calls in a row, the second with a smaller input (the area
keeps the first call's contents)."""

import ctypes

import pytest
import torch

import long_context_kv_snapkv_amd as skv
from parity import bits_from_device, check_structure_and_gather, upload
from synth import WORKLOADS, make_custom, make_layer

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _compare(x, window, kernel, pool, budget):
    q, k, v = upload(x)
    lens = x.seq_lens.tolist()
    ref = skv.snapkv_compress(q, k, v, lens, window, kernel, pool, budget)
    # outputs pre-filled with a pattern, so that every element must be written
    out = [torch.full_like(ref[0], 3.0), torch.full_like(ref[1], -2.0),
           torch.full_like(ref[2], 77)]
    got = skv.snapkv_compress_static(q, k, v, lens, window, kernel, pool, budget,
                                     out_k=out[0], out_v=out[1], out_idx=out[2])
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    res = dict(out_k=bits_from_device(got[0]), out_v=bits_from_device(got[1]),
               out_idx=got[2].cpu().numpy())
    check_structure_and_gather(res, x, window, budget)


@needs_gpu
def test_static_scratch_matches_workspace_path_on_two_calls():
    w = WORKLOADS["llama3_8b_16k"]
    print("[no_alloc] call 1: llama3_8b_16k", flush=True)
    _compare(make_layer(w), w.window, w.kernel, w.pool, w.budget)
    # a smaller second call on the same area (its first call's contents stay)
    print("[no_alloc] call 2: ragged, smaller", flush=True)
    x = make_custom([3000, 700, 40, 2500], 16, 4, 128, 32, seed=5)
    _compare(x, 32, 5, "avg", 512)


@needs_gpu
def test_static_scratch_rejects_a_shape_beyond_the_area():
    # the need is computed on the host: a shape whose scratch exceeds the
    # area is refused before anything is enqueued
    x = make_custom([300], 8, 2, 128, 16, seed=2)
    q, k, v = upload(x)
    big_lens = [131072] * 8
    assert skv.snapkv_workspace_size(64, 8, 128, big_lens, 64) > skv.SNAPKV_STATIC_SCRATCH_BYTES
    lib = skv.load_library()
    arr = (ctypes.c_int32 * 8)(*big_lens)
    st = lib.snapkv_compress_static(8, 64, 8, 128, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    arr, 64, 7, 1, 1024, k.data_ptr(), v.data_ptr(),
                                    k.data_ptr(), None)
    assert st == skv.SNAPKV_ERR_WORKSPACE, skv.snapkv_last_error()
    assert "static area" in skv.snapkv_last_error()
    torch.cuda.synchronize()
