"""The Python binding rejects malformed tensors before anything reaches the C ABI.

The ABI takes raw pointers, so a short K/V, a K/V of another dtype, a strided
innermost dimension or an undersized idx/counts buffer would make a kernel read or
write past an allocation.  Each case here must raise ValueError on the host; these
run on the CPU (shape, dtype and capacity checks come before the device check).
"""
import pytest
import torch

import block_sparse_long_pooled_amd as fp

L, HQ, HKV, D = 300, 4, 2, 128
NB = -(-L // 128)
TRI = NB * (NB + 1) // 2


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def qkv():
    return bf(L, HQ, D), bf(L, HKV, D), bf(L, HKV, D)


def lists(heads=HQ):
    return torch.zeros(heads * TRI, dtype=torch.int32), torch.zeros((heads, NB), dtype=torch.int32)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_attention_rejects_mismatched_kv():
    q, k, v = qkv()
    idx, counts = lists()
    raises(lambda: fp.sparse_attn(q, bf(L - 1, HKV, D), v, idx, counts), "tokens")
    raises(lambda: fp.sparse_attn(q, k, bf(L, HKV + 1, D), idx, counts), "heads")
    raises(lambda: fp.sparse_attn(q, bf(L, 3, D), bf(L, 3, D), idx, counts), "multiple")
    raises(lambda: fp.sparse_attn(q, bf(L, HKV, 64), v, idx, counts), "head dim")
    raises(lambda: fp.sparse_attn(q, k.to(torch.float8_e4m3fn), v, idx, counts), "dtype")


def test_attention_rejects_strided_innermost_dim():
    q, k, v = qkv()
    idx, counts = lists()
    wide = bf(L, HQ, 2 * D)[..., ::2]
    assert wide.shape == q.shape and wide.stride(2) == 2
    raises(lambda: fp.sparse_attn(wide, k, v, idx, counts), "unit innermost stride")
    raises(lambda: fp.dense_attn(q, k, v, out=bf(L, HQ, 2 * D)[..., ::2]), "unit innermost stride")


def test_attention_rejects_short_or_wrong_lists():
    q, k, v = qkv()
    idx, counts = lists()
    raises(lambda: fp.sparse_attn(q, k, v, idx[:-1], counts), "idx holds")
    raises(lambda: fp.sparse_attn(q, k, v, idx.to(torch.int64), counts), "idx must be")
    raises(lambda: fp.sparse_attn(q, k, v, idx, counts[:, :-1]), "counts must have shape")
    raises(lambda: fp.sparse_attn(q, k, v, idx, counts.t().contiguous().t()), "contiguous")
    raises(lambda: fp.sparse_attn_grouped(q, k, v, *lists(HKV - 1)), "idx holds")
    raises(lambda: fp.sparse_attn_masked(q, k, v, torch.zeros((HQ, NB, 2), dtype=torch.int32)), "mask")


def test_attention_rejects_bad_out_and_fp8_scales():
    q, k, v = qkv()
    idx, counts = lists()
    raises(lambda: fp.sparse_attn(q, k, v, idx, counts, out=bf(L, HQ - 1, D)), "heads")
    raises(lambda: fp.sparse_attn(q, k, v, idx, counts, out=torch.zeros((L, HQ, D))), "bfloat16")
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
    s_q, s_kv = torch.ones(HQ), torch.ones(HKV)
    raises(lambda: fp.sparse_attn(q8, k8, v8, idx, counts), "fp8 inputs need q_scale")
    raises(lambda: fp.sparse_attn(q8, k8, v8, idx, counts, s_q, s_q, s_kv), "k_scale")
    raises(lambda: fp.sparse_attn(q8, k8, v8, idx, counts, s_q, s_kv, s_kv.double()), "v_scale")


def test_selection_rejects_short_buffers():
    pq = torch.zeros((HQ, NB, D), dtype=torch.float64)
    pk = torch.zeros((HKV, NB, D), dtype=torch.float64)
    idx, counts = lists()
    raises(lambda: fp.threshold_compact(pq, pk, 0.1, 1, 4, idx=idx[:5], counts=counts), "idx holds")
    raises(lambda: fp.threshold_compact(pq, pk, 0.1, 1, 4, idx=idx, counts=counts[:1]), "counts")
    raises(lambda: fp.threshold_compact(pq.float(), pk, 0.1, 1, 4, idx=idx, counts=counts), "pooled_q")
    raises(lambda: fp.threshold_compact(pq, pk[:, :-1], 0.1, 1, 4, idx=idx, counts=counts), "pooled_k")
    raises(lambda: fp.threshold_compact(pq, pk, 0.1, 1, 4, idx=idx, counts=counts,
                                        scores=torch.zeros((HQ, NB, NB - 1), dtype=torch.float64)), "scores")
    raises(lambda: fp.threshold_mask(pq, pk, 0.1, 1, 4, mask=torch.zeros((HQ, NB, 2), dtype=torch.int32)), "mask")
    raises(lambda: fp.union_compact(torch.zeros((HQ, NB, 1), dtype=torch.int32), 3), "multiple")


def test_discover_and_pool_reject_bad_outputs():
    q, k, _ = qkv()
    raises(lambda: fp.discover(q, bf(L + 1, HKV, D)), "tokens")
    raises(lambda: fp.discover(q, k, pooled_q=torch.zeros((HQ, NB - 1, D), dtype=torch.float64)), "pooled_q")
    raises(lambda: fp.pool(q, pooled=torch.zeros((HQ, NB, D), dtype=torch.float32)), "pooled")


def test_mean_correct_rejects_bad_buffers():
    q, _, _ = qkv()
    pk = torch.zeros((HKV, NB, D), dtype=torch.float64)
    idx, counts = lists()
    out = bf(L, HQ, D)
    lse = torch.zeros((HQ, L))
    ws = torch.zeros(16, dtype=torch.uint8)
    raises(lambda: fp.mean_correct(q, pk, pk, idx, counts, out, lse, workspace=ws), "workspace")
    raises(lambda: fp.mean_correct(q, pk, pk, idx, counts, out, lse[:, :-1]), "lse")
    raises(lambda: fp.mean_correct(q, pk, pk[:1], idx, counts, out, lse), "pooled_v")


def test_packed_batch_rejects_mismatches():
    batch = fp.VarlenBatch([200, 300], torch.device("cpu"))
    T = batch.total_tokens
    q, k, v = bf(T, HQ, D), bf(T, HKV, D), bf(T, HKV, D)
    idx = torch.zeros(HQ * batch.total_tri, dtype=torch.int32)
    counts = torch.zeros((HQ, batch.total_blocks), dtype=torch.int32)
    raises(lambda: fp.sparse_attn_paged(bf(T - 1, HQ, D), k, v, batch, idx, counts), "tokens")
    raises(lambda: fp.sparse_attn_paged(q, k, v, batch, idx[:-1], counts), "idx holds")
    raises(lambda: fp.sparse_attn_paged(q, k, v, batch, idx, None), "both")
    pages = bf(6, 128, HKV, D)
    table = torch.zeros((2, 2), dtype=torch.int32)
    raises(lambda: fp.sparse_attn_paged(q, pages, pages, batch, idx, counts, page_table=table), "pages per sequence")
    raises(lambda: fp.sparse_attn_paged(q, pages, bf(5, 128, HKV, D), batch, idx, counts,
                                        page_table=torch.zeros((2, 3), dtype=torch.int32)), "pages")
    raises(lambda: fp.discover_paged(q, bf(T, HKV, D), batch,
                                     pooled_k=torch.zeros((HKV, 1, D), dtype=torch.float64)), "pooled_k")
    cb = fp.ChunkedBatch([100], [400], torch.device("cpu"))
    raises(lambda: fp.sparse_attn_chunked(bf(99, HQ, D), bf(400, HKV, D), bf(400, HKV, D), cb), "tokens")


def test_valid_cpu_tensors_fail_only_on_the_device_check():
    q, k, v = qkv()
    idx, counts = lists()
    raises(lambda: fp.sparse_attn(q, k, v, idx, counts), "CUDA device")
    raises(lambda: fp.discover(q, k), "CUDA device")
