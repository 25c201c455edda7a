"""GPU parity of snapkv_compress_int4: the compressed cache stored at 4 bits
per value with a float32 scale per row.

Integer outputs are compared bit for bit. The index list must equal
snapkv_compress's on the same inputs (same selection kernels). Codes and
scales must equal the oracle's quantisation (float32 decisions, as the
kernel takes them): for every head, of the input K/V rows the index list
names; and, where the oracle's own selection is unambiguous, the oracle's
whole 4-bit cache (compress_int4) for that head.
"""

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
import oracle
from parity import check_index_sets, check_structure_and_gather, run_gpu, upload
from synth import WORKLOADS, make_custom, make_layer

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = [
    # lens, h_q, h_kv, d, window, kernel, pool, budget
    ([1000], 8, 8, 64, 32, 5, "avg", 256),              # MHA, D = 64
    ([3000, 2500], 16, 4, 128, 64, 5, "avg", 1024),
    ([64, 300, 65, 5, 1000], 8, 2, 128, 32, 5, "avg", 96),  # ragged, kept whole, L < W
    ([700], 6, 2, 64, 24, 9, "max", 80),
    ([257], 4, 2, 128, 16, 5, "max", 256),              # L = B + 1
    # prefixes past the register-resident selection, one prompt kept whole:
    # the sliced selection and the gather in one launch
    ([40000, 3000, 400, 35000, 4100], 8, 2, 128, 16, 5, "avg", 512),
    ([36000], 4, 4, 64, 16, 7, "max", 1500),            # D = 64
]


def _run_int4(x, window, kernel, pool, budget, lse=None):
    q, k, v = upload(x)
    lt = None if lse is None else torch.from_numpy(np.ascontiguousarray(lse, np.float32)).cuda()
    kq, ks, vq, vs, idx = skv.snapkv_compress_int4(q, k, v, x.seq_lens.tolist(), window, kernel,
                                                   pool, budget, window_lse=lt)
    torch.cuda.synchronize()
    return dict(kq=kq.cpu().numpy(), ks=ks.cpu().numpy(), vq=vq.cpu().numpy(),
                vs=vs.cpu().numpy(), idx=idx.cpu().numpy())


def _rows_at(bits, x, idx, budget):
    """Input rows named by an index list (zero rows where it holds -1)."""
    batch, hkv = idx.shape[:2]
    out = np.zeros((batch, hkv, budget, bits.shape[2]), dtype=np.uint16)
    for b in range(batch):
        for h in range(hkv):
            sel = idx[b, h] >= 0
            out[b, h, sel] = bits[x.offsets[b] + idx[b, h, sel], h]
    return out


def _check_int4(x, window, kernel, pool, budget, res, lse=None):
    lens = x.seq_lens.tolist()
    plain = run_gpu(x, window, kernel, pool, budget)
    np.testing.assert_array_equal(res["idx"], plain["out_idx"])
    check_structure_and_gather(plain, x, window, budget)
    # each stored row is the quantisation of the input row its index names
    want = oracle.quantize_cache(_rows_at(x.k, x, res["idx"], budget),
                                 _rows_at(x.v, x, res["idx"], budget), res["idx"])
    for key, ref in (("kq", want.kq), ("ks", want.ks), ("vq", want.vq), ("vs", want.vs)):
        np.testing.assert_array_equal(res[key], ref, err_msg=key)
    # heads whose oracle selection is unambiguous match the oracle's 4-bit cache
    ref = oracle.compress(x.q_win, x.k, x.v, lens, window, kernel, pool, budget, lse=lse)
    full = oracle.quantize_cache(ref.out_k, ref.out_v, ref.out_idx)
    check_index_sets(res["idx"], ref.pooled, lens, window, budget)
    m = budget - window
    matched = 0
    for b, length in enumerate(lens):
        for h in range(res["idx"].shape[1]):
            if length > budget:
                o = np.sort(ref.pooled[b][h])[::-1]
                if o[m - 1] - o[m] <= 1e-3 * o[m - 1] + 1e-6 * o[0]:
                    continue
            for key in ("kq", "ks", "vq", "vs"):
                np.testing.assert_array_equal(res[key][b, h], getattr(full, key)[b, h])
            matched += 1
    return matched


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_int4_matches_oracle(case):
    lens, hq, hkv, d, window, kernel, pool, budget = case
    print(f"[int4] {case}", flush=True)
    x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 83)
    res = _run_int4(x, window, kernel, pool, budget)
    _check_int4(x, window, kernel, pool, budget, res)


@needs_gpu
def test_int4_llama3_8b_16k():
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    print(f"[int4] llama3_8b_16k lens={x.seq_lens.tolist()}", flush=True)
    res = _run_int4(x, w.window, w.kernel, w.pool, w.budget)
    _check_int4(x, w.window, w.kernel, w.pool, w.budget, res)
    # the stored values are within half a step of the kept rows
    deq = oracle.dequantize_int4(res["kq"], res["ks"])
    kept = oracle.bf16_bits_to_f64(_rows_at(x.k, x, res["idx"], w.budget))
    assert (np.abs(deq - kept) <= res["ks"][..., None] * (0.5 + 1e-5)).all()


@needs_gpu
def test_int4_with_caller_normalisers():
    x = make_custom([6000, 4100], 32, 8, 128, 32, seed=21)
    lse = oracle.window_lse(x.q_win, x.k, x.seq_lens, 32).astype(np.float32)
    print("[int4] with normalisers", flush=True)
    res = _run_int4(x, 32, 7, "avg", 512, lse=lse)
    want = oracle.quantize_cache(_rows_at(x.k, x, res["idx"], 512),
                                 _rows_at(x.v, x, res["idx"], 512), res["idx"])
    np.testing.assert_array_equal(res["kq"], want.kq)
    np.testing.assert_array_equal(res["vs"], want.vs)
    ref = oracle.compress(x.q_win, x.k, x.v, x.seq_lens.tolist(), 32, 7, "avg", 512,
                          lse=lse.astype(np.float64))
    check_index_sets(res["idx"], ref.pooled, x.seq_lens.tolist(), 32, 512)


@needs_gpu
def test_int4_zero_and_extreme_rows():
    # zero K rows quantise to codes 0 / scale 0; window rows (always kept)
    # with one dominant V entry store 7 there and 0 elsewhere
    x = make_custom([600], 8, 2, 128, 16, seed=22)
    x.k[:200] = 0
    x.v[590:600, :, 5] = 0x4780  # bf16 65536
    res = _run_int4(x, 16, 5, "avg", 300)
    _check_int4(x, 16, 5, "avg", 300, res)
    assert (res["idx"][0] < 200).any()
    assert (res["ks"][0][res["idx"][0] < 200] == 0).all()
    codes = oracle.unpack_int4(res["vq"][0][:, -10:])
    assert (codes[..., 5] == 7).all() and (np.delete(codes, 5, axis=-1) == 0).all()
    np.testing.assert_array_equal(res["vs"][0][:, -10:], np.float32(65536.0) / np.float32(7.0))


@needs_gpu
def test_int4_repeatable_and_bytes_sized():
    x = make_custom([9000], 32, 8, 128, 32, seed=23)
    a = _run_int4(x, 32, 7, "max", 1024)
    b = _run_int4(x, 32, 7, "max", 1024)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    assert a["kq"].shape == (1, 8, 1024, 64) and a["kq"].dtype == np.uint8
