"""GPU parity of snapkv_compress_fp8: the compressed cache stored as OCP FP8
E4M3 bytes with a float32 scale per row.

Codes and scales must equal the oracle's quantisation bit for bit (the
float32 product decides the code; the oracle encodes it by the format's
definition, the kernel with the conversion instruction), for the input rows
the GPU's index list names on every head, and the oracle's whole 8-bit cache
where its own selection is unambiguous. The index list must equal
snapkv_compress's.
"""

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
import oracle
from parity import check_index_sets, run_gpu, upload
from synth import WORKLOADS, make_custom, make_layer
from test_int4_gpu import _rows_at

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _run_fp8(x, window, kernel, pool, budget, lse=None):
    q, k, v = upload(x)
    lt = None if lse is None else torch.from_numpy(np.ascontiguousarray(lse, np.float32)).cuda()
    kq, ks, vq, vs, idx = skv.snapkv_compress_fp8(q, k, v, x.seq_lens.tolist(), window, kernel,
                                                  pool, budget, window_lse=lt)
    torch.cuda.synchronize()
    return dict(kq=kq.cpu().numpy(), ks=ks.cpu().numpy(), vq=vq.cpu().numpy(),
                vs=vs.cpu().numpy(), idx=idx.cpu().numpy())


def _check_fp8(x, window, kernel, pool, budget, res):
    lens = x.seq_lens.tolist()
    plain = run_gpu(x, window, kernel, pool, budget)
    np.testing.assert_array_equal(res["idx"], plain["out_idx"])
    want = oracle.quantize_cache_fp8(_rows_at(x.k, x, res["idx"], budget),
                                     _rows_at(x.v, x, res["idx"], budget), res["idx"])
    for key in ("kq", "ks", "vq", "vs"):
        np.testing.assert_array_equal(res[key], getattr(want, key), err_msg=key)
    ref = oracle.compress(x.q_win, x.k, x.v, lens, window, kernel, pool, budget)
    full = oracle.quantize_cache_fp8(ref.out_k, ref.out_v, ref.out_idx)
    check_index_sets(res["idx"], ref.pooled, lens, window, budget)
    m = budget - window
    for b, length in enumerate(lens):
        for h in range(res["idx"].shape[1]):
            if length > budget:
                o = np.sort(ref.pooled[b][h])[::-1]
                if o[m - 1] - o[m] <= 1e-3 * o[m - 1] + 1e-6 * o[0]:
                    continue
            for key in ("kq", "ks", "vq", "vs"):
                np.testing.assert_array_equal(res[key][b, h], getattr(full, key)[b, h])


CASES = [
    # lens, h_q, h_kv, d, window, kernel, pool, budget
    ([1000], 8, 8, 64, 32, 5, "avg", 256),
    ([3000, 2500], 16, 4, 128, 64, 5, "avg", 1024),
    ([64, 300, 65, 5, 1000], 8, 2, 128, 32, 5, "avg", 96),
    # prefixes past the register-resident selection, one prompt kept whole:
    # the sliced selection and the gather in one launch
    ([40000, 3000, 400, 35000, 4100], 8, 2, 128, 16, 5, "avg", 512),
    ([36000], 4, 4, 64, 16, 7, "max", 1500),            # D = 64
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_fp8_matches_oracle(case):
    lens, hq, hkv, d, window, kernel, pool, budget = case
    print(f"[fp8] {case}", flush=True)
    x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 79)
    _check_fp8(x, window, kernel, pool, budget, _run_fp8(x, window, kernel, pool, budget))


@needs_gpu
def test_fp8_llama3_8b_16k():
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    print("[fp8] llama3_8b_16k", flush=True)
    res = _run_fp8(x, w.window, w.kernel, w.pool, w.budget)
    _check_fp8(x, w.window, w.kernel, w.pool, w.budget, res)
    deq = oracle.e4m3_decode(res["kq"]) * res["ks"].astype(np.float64)[..., None]
    kept = oracle.bf16_bits_to_f64(_rows_at(x.k, x, res["idx"], w.budget))
    bound = np.maximum(np.abs(kept) * 2.0 ** -4, res["ks"][..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - kept) <= bound).all()


@needs_gpu
def test_fp8_with_caller_normalisers_and_extremes():
    x = make_custom([5000, 3000], 32, 8, 128, 32, seed=41)
    x.k[:300] = 0                      # zero rows: codes 0, scale 0
    x.v[4990:5000, :, 7] = 0x4780      # window rows with one dominant entry (65536)
    lse = oracle.window_lse(x.q_win, x.k, x.seq_lens, 32).astype(np.float32)
    res = _run_fp8(x, 32, 7, "max", 512, lse=lse)
    want = oracle.quantize_cache_fp8(_rows_at(x.k, x, res["idx"], 512),
                                     _rows_at(x.v, x, res["idx"], 512), res["idx"])
    for key in ("kq", "ks", "vq", "vs"):
        np.testing.assert_array_equal(res[key], getattr(want, key), err_msg=key)
    assert (res["vq"][0][:, -10:, 7] == 0x7E).all()
