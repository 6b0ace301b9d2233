"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Sizes are ones the oracle finishes in seconds but that still span several tiles
(the threshold kernel tiles 64 query blocks; attention visits many blocks) and a
ragged tail.  Rules:
  * pooled means: bit-exact (fp64 sums of exact inputs);
  * lists: exact except non-forced blocks within 1e-6 relative of alpha;
  * attention: the oracle attends over the GPU's own lists; max-abs error
    <= 2e-2 (bf16) / 6e-2 (fp8) against fp64;
  * self-consistency: reruns, alpha = 0 vs dense, GQA vs MHA, paged vs packed are
    bit-exact on the GPU.
"""
import functools
import math

import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
import synth
from helpers import (TOL_BF16, TOL_FP8, check_lists, oracle_inputs, record_margin, to_device, to_device_paged,
                     unpack_lists)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@functools.lru_cache(maxsize=None)
def workload(name):
    if name == "tiny":
        return synth.make_config(0)
    if name == "gqa_ragged":  # 71 blocks: two 64-row threshold tiles, ragged tail of 37
        return synth.make_workload(name, 8, 2, [128 * 70 + 37], seed=21, alphas=(0.05, 0.1, 0.3),
                                   n_sink=1, n_local=3)
    if name == "fp8_ragged":
        return synth.make_workload(name, 8, 2, [128 * 40 + 100], seed=22, dtype="fp8", alphas=(0.1,),
                                   n_sink=1, n_local=4)
    if name == "mha_one_block":  # a single partial block
        return synth.make_workload(name, 2, 2, [100], seed=23, alphas=(0.1,), n_sink=1, n_local=1)
    if name == "gqa7":  # Qwen2.5-7B head ratio (28/4 -> 7), short
        return synth.make_workload(name, 7, 1, [128 * 20 + 1], seed=24, alphas=(0.2,), n_sink=2, n_local=2)
    if name == "structured":  # the sparser structured recipe: peaked rows, heads sharing blocks
        return synth.make_structured(L=128 * 90 + 57, hq=8, hkv=2, seed=25)
    if name == "gqa28x4_short":  # hq not a multiple of 8: KV groups on XCD pairs (10 query blocks)
        return synth.make_workload(name, 28, 4, [128 * 9 + 17], seed=26, alphas=(0.2,), n_sink=1, n_local=2)
    raise KeyError(name)


@functools.lru_cache(maxsize=None)
def oracle_selection(name, alpha):
    wl = workload(name)
    q, k, _ = oracle_inputs(wl)
    return O.select_blocks(q, k, 128, alpha, wl.n_sink, wl.n_local)


CASES = ["tiny", "gqa_ragged", "fp8_ragged", "mha_one_block", "gqa7", "structured", "gqa28x4_short"]


def run_gpu(wl, alpha):
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=True)
    torch.cuda.synchronize()
    return dict(pq=pq.cpu().numpy(), pk=pk.cpu().numpy(), idx=idx.cpu().numpy(), counts=counts.cpu().numpy(),
                out=out.float().cpu().numpy(), lse=lse.cpu().numpy())


@pytest.mark.parametrize("name", CASES)
def test_discover_bit_exact(name):
    wl = workload(name)
    print(f"[case] discover {name} L={wl.L} hq={wl.hq} hkv={wl.hkv} {wl.dtype}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    torch.cuda.synchronize()
    oq, ok_, _ = oracle_inputs(wl)
    assert np.array_equal(pq.cpu().numpy(), O.pool(oq, 128))
    assert np.array_equal(pk.cpu().numpy(), O.pool(ok_, 128))


@pytest.mark.parametrize("name", CASES)
def test_lists_and_attention_match_oracle(name):
    wl = workload(name)
    for alpha in wl.alphas:
        print(f"[case] select+attn {name} alpha={alpha}", flush=True)
        r = run_gpu(wl, alpha)
        sel = oracle_selection(name, alpha)
        nb = -(-wl.L // 128)
        tri = nb * (nb + 1) // 2
        lists = [unpack_lists(r["idx"], r["counts"], h, nb, tri) for h in range(wl.hq)]
        check_lists(lists, sel, alpha, wl.n_sink, wl.n_local)
        q, k, v = oracle_inputs(wl)
        ref, ref_lse = O.sparse_attention(q, k, v, lists, 128, want_lse=True)
        err = np.max(np.abs(r["out"] - ref))
        tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
        msg = f"{name} alpha={alpha}: full output max-abs {err:.3e} (bound {tol}), density {r['counts'].sum() / (wl.hq * tri):.3f}"
        print("  " + msg, flush=True)
        record_margin(msg)
        assert err <= tol
        assert np.max(np.abs(r["lse"] - ref_lse.astype(np.float32))) <= 1e-3 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("name", CASES)
def test_scores_match_oracle(name):
    """The debug score output: fp64 pooled scores on the fp64 matrix core against the
    oracle's score map (same pooled means, bit-exact inputs; only the summation order
    differs), written for j <= i only; lists are the same with and without it."""
    wl = workload(name)
    print(f"[case] scores {name}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    hq, nb, _ = pq.shape
    sc = torch.full((hq, nb, nb), float("nan"), dtype=torch.float64, device=q.device)
    alpha = wl.alphas[0]
    idx1, cnt1 = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local, scores=sc)
    idx0, cnt0 = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    torch.cuda.synchronize()
    ref = O.block_scores(pq.cpu().numpy(), pk.cpu().numpy(), 1.0 / math.sqrt(128))
    got = sc.cpu().numpy()
    low = np.tril(np.ones((nb, nb), dtype=bool))
    assert np.all(np.isnan(got[:, ~low]))
    diff = np.abs(got[:, low] - ref[:, low])
    assert np.all(diff <= 1e-12 * np.maximum(1.0, np.abs(ref[:, low])))
    assert torch.equal(cnt0, cnt1) and torch.equal(idx0, idx1)


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "fp8_ragged", "mha_one_block", "gqa28x4_short"])
def test_dense_matches_oracle(name):
    wl = workload(name)
    print(f"[case] dense {name}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    out = fp.dense_attn(q, k, v, qs, ks, vs)
    torch.cuda.synchronize()
    oq, ok_, ov = oracle_inputs(wl)
    ref = O.dense_attention(oq, ok_, ov)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= tol


def test_alpha_zero_equals_dense_bit_exact():
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    pq, pk = fp.discover(q, k)
    idx, counts = fp.threshold_compact(pq, pk, 0.0, 1, 1)
    sp = fp.sparse_attn(q, k, v, idx, counts)
    de = fp.dense_attn(q, k, v)
    torch.cuda.synchronize()
    nb = pq.shape[1]
    assert torch.equal(counts.cpu(), torch.arange(1, nb + 1, dtype=torch.int32).repeat(wl.hq, 1))
    assert torch.equal(sp, de)


def test_alpha_above_one_keeps_forced_blocks_only():
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    pq, pk = fp.discover(q, k)
    idx, counts = fp.threshold_compact(pq, pk, 1.5, 2, 3)
    nb = pq.shape[1]
    idx, counts = idx.cpu().numpy(), counts.cpu().numpy()
    for h in range(wl.hq):
        for i, lst in enumerate(unpack_lists(idx, counts, h, nb, nb * (nb + 1) // 2)):
            want = sorted(set(range(min(2, i + 1))) | set(range(max(0, i - 2), i + 1)))
            assert lst.tolist() == want


def test_huge_sink_and_window_keep_everything():
    """n_sink and n_local far beyond the sequence (no overflow in i - n_local): every
    causal block is forced, so the sparse output equals the dense kernel bit for bit."""
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    pq, pk = fp.discover(q, k)
    nb = pq.shape[1]
    for ns, nl in [(10 ** 6, 1), (0, 2 ** 31 - 1)]:
        idx, counts = fp.threshold_compact(pq, pk, 1.5, ns, nl)
        sp = fp.sparse_attn(q, k, v, idx, counts)
        de = fp.dense_attn(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(counts.cpu(), torch.arange(1, nb + 1, dtype=torch.int32).repeat(wl.hq, 1)), (ns, nl)
        assert torch.equal(sp, de), (ns, nl)


def test_rerun_is_bit_identical():
    wl = workload("gqa_ragged")
    a = run_gpu(wl, 0.1)
    b = run_gpu(wl, 0.1)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_gqa_equals_mha_with_repeated_kv():
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    g = wl.hq // wl.hkv
    kr = k.repeat_interleave(g, dim=1).contiguous()
    vr = v.repeat_interleave(g, dim=1).contiguous()
    o1, i1, c1 = fp.prefill(q, k, v, 0.1, 1, 3)
    o2, i2, c2 = fp.prefill(q, kr, vr, 0.1, 1, 3)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(i1, i2) and torch.equal(o1, o2)


def test_strided_inputs_match_contiguous():
    """[H, L, d] head-major views (non-default strides) give the same bits."""
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    qh = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    kh = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    vh = v.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    o1, i1, c1 = fp.prefill(q, k, v, 0.1, 1, 3)
    o2, i2, c2 = fp.prefill(qh, kh, vh, 0.1, 1, 3)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(i1, i2) and torch.equal(o1, o2)


# ----------------------------------------------------------------- varlen / paged
@functools.lru_cache(maxsize=None)
def batch_workload(dtype="bf16"):
    # ragged lengths: partial tails, one single-block sequence, one > 64 blocks
    return synth.make_workload("paged_small", 8, 2, [1000, 128, 65, 8300, 3000], seed=31, paged=True,
                               dtype=dtype, alphas=(0.1,), n_sink=1, n_local=4)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_paged_matches_oracle_and_packed(dtype):
    wl = batch_workload(dtype)
    print(f"[case] paged {dtype} lengths={wl.lengths}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    kc, vc, table = to_device_paged(wl)
    batch = fp.VarlenBatch(wl.lengths, q.device)
    pq1, pk1 = fp.discover_paged(q, k, batch, q_scale=qs, k_scale=ks)
    pq2, pk2 = fp.discover_paged(q, kc, batch, page_table=table, q_scale=qs, k_scale=ks)
    idx, counts = fp.threshold_compact_varlen(pq2, pk2, batch, 0.1, wl.n_sink, wl.n_local)
    sc = dict(q_scale=qs, k_scale=ks, v_scale=vs)
    o_packed = fp.sparse_attn_paged(q, k, v, batch, idx, counts, **sc)
    o_paged, lse = fp.sparse_attn_paged(q, kc, vc, batch, idx, counts, page_table=table, return_lse=True, **sc)
    d_paged = fp.sparse_attn_paged(q, kc, vc, batch, page_table=table, **sc)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP8
    assert torch.equal(pq1, pq2) and torch.equal(pk1, pk2)
    assert torch.equal(o_packed, o_paged)

    oq, ok_, ov = oracle_inputs(wl)
    cu = wl.cu_seqlens
    sels = O.select_blocks_varlen(oq, ok_, cu, 128, 0.1, wl.n_sink, wl.n_local)
    pq_np, pk_np = pq2.cpu().numpy(), pk2.cpu().numpy()
    idx_np, cnt_np = idx.cpu().numpy(), counts.cpu().numpy()
    out = o_paged.float().cpu().numpy()
    dout = d_paged.float().cpu().numpy()
    for s in range(wl.n_seqs):
        b0, b1 = batch.cu_blocks[s], batch.cu_blocks[s + 1]
        assert np.array_equal(pq_np[:, b0:b1], sels[s]["pq"])
        assert np.array_equal(pk_np[:, b0:b1], sels[s]["pk"])
        nb = b1 - b0
        lists = [unpack_lists(idx_np, cnt_np, h, nb, batch.total_tri, batch.cu_tri[s], b0) for h in range(wl.hq)]
        check_lists(lists, sels[s], 0.1, wl.n_sink, wl.n_local)
        a, b = cu[s], cu[s + 1]
        ref = O.sparse_attention(oq[a:b], ok_[a:b], ov[a:b], lists, 128)
        assert np.max(np.abs(out[a:b] - ref)) <= tol, s
        dref = O.dense_attention(oq[a:b], ok_[a:b], ov[a:b])
        assert np.max(np.abs(dout[a:b] - dref)) <= tol, s


def test_varlen_single_sequence_equals_contiguous_api():
    wl = workload("gqa_ragged")
    q, k, v, *_ = to_device(wl)
    batch = fp.VarlenBatch([wl.L], q.device)
    pq1, pk1 = fp.discover(q, k)
    pq2, pk2 = fp.discover_paged(q, k, batch)
    i1, c1 = fp.threshold_compact(pq1, pk1, 0.1, 1, 3)
    i2, c2 = fp.threshold_compact_varlen(pq2, pk2, batch, 0.1, 1, 3)
    o1 = fp.sparse_attn(q, k, v, i1, c1)
    o2 = fp.sparse_attn_paged(q, k, v, batch, i2, c2)
    torch.cuda.synchronize()
    assert torch.equal(pq1, pq2) and torch.equal(i1, i2) and torch.equal(c1, c2) and torch.equal(o1, o2)


def test_invalid_page_gives_nan_not_fault():
    """A page id outside [0, num_pages) is never dereferenced; that sequence's
    pooled K and attention rows that need it come out NaN, the others are intact."""
    wl = batch_workload()
    q, k, v, *_ = to_device(wl)
    kc, vc, table = to_device_paged(wl)
    bad = table.clone()
    bad[1, 0] = kc.shape[0] + 5  # sequence 1 (one block) points past the cache
    batch = fp.VarlenBatch(wl.lengths, q.device)
    pq, pk = fp.discover_paged(q, kc, batch, page_table=bad)
    out = fp.sparse_attn_paged(q, kc, vc, batch, page_table=bad)
    good = fp.sparse_attn_paged(q, kc, vc, batch, page_table=table)
    torch.cuda.synchronize()
    cu = wl.cu_seqlens
    b1 = batch.cu_blocks[1]
    assert torch.isnan(pk[:, b1]).all()
    assert torch.isnan(out[cu[1]:cu[2]].float()).all()
    keep = torch.ones(out.shape[0], dtype=torch.bool)
    keep[cu[1]:cu[2]] = False
    assert torch.equal(out[keep], good[keep])


def test_empty_and_zero_length_sequences():
    wl = batch_workload()
    q, k, v, *_ = to_device(wl)
    lengths = [wl.lengths[0], 0, wl.lengths[1]]
    T = lengths[0] + lengths[2]
    qq, kk, vv = q[:T].contiguous(), k[:T].contiguous(), v[:T].contiguous()
    batch = fp.VarlenBatch(lengths, q.device)
    pq, pk = fp.discover_paged(qq, kk, batch)
    idx, counts = fp.threshold_compact_varlen(pq, pk, batch, 0.1, 1, 4)
    out = fp.sparse_attn_paged(qq, kk, vv, batch, idx, counts)
    ref_batch = fp.VarlenBatch([lengths[0], lengths[2]], q.device)
    pq2, pk2 = fp.discover_paged(qq, kk, ref_batch)
    idx2, c2 = fp.threshold_compact_varlen(pq2, pk2, ref_batch, 0.1, 1, 4)
    out2 = fp.sparse_attn_paged(qq, kk, vv, ref_batch, idx2, c2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(idx, idx2)
    # L = 0 contiguous call is a no-op
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=q.device)
    pq0, pk0 = fp.discover(e, e[:, :2])
    assert pq0.shape == (8, 0, 128)


def test_list_without_diagonal_gives_nan_rows():
    """A caller list that does not end with the diagonal block is rejected in the
    kernel: that (head, query block) comes out NaN, every other row is unchanged."""
    wl = workload("gqa_ragged")
    print("[case] list without its diagonal block", flush=True)
    q, k, v, *_ = to_device(wl)
    pq, pk = fp.discover(q, k)
    idx, counts = fp.threshold_compact(pq, pk, 0.1, wl.n_sink, wl.n_local)
    good = fp.sparse_attn(q, k, v, idx, counts)
    h, i = 3, 40
    cut = counts.clone()
    cut[h, i] -= 1  # drops the last entry, which is block i
    out = fp.sparse_attn(q, k, v, idx, cut)
    torch.cuda.synchronize()
    assert int(counts[h, i]) >= 2
    rows = slice(i * 128, (i + 1) * 128)
    assert torch.isnan(out[rows, h].float()).all()
    keep = torch.ones(out.shape[:2], dtype=torch.bool, device=out.device)
    keep[rows, h] = False
    assert torch.equal(out[keep], good[keep])
