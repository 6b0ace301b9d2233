"""Parity at the full workload sizes, in the launch configuration bench.py times.

Pooled means are compared bit-exactly everywhere and lists on every row (the
oracle's pooled score map is cheap).  Attention is checked on a stratified sample
of query blocks the oracle computes one by one, over the GPU's own lists: for every
head its first 4 and last 4 query blocks, plus the 8 rows (past the first four) with
the fewest listed blocks, where rounding of the probabilities weighs most, and a few
seeded random rows.  Each test prints its worst max-abs and LSE error against the
bound.  Paged == packed is checked bit-exactly on the full output of the paged batch,
and its sample takes every sequence's first and last query block for every head.
"""
import functools

import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
import synth
from helpers import (TOL_BF16, TOL_FP8, check_lists, oracle_inputs, record_margin, to_device, to_device_paged,
                     unpack_lists)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@functools.lru_cache(maxsize=1)
def cfg(k):
    return synth.make_config(k)


def sample_rows(hq, nb, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (hq - 1, nb - 1), (hq // 2, nb // 2)}
    while len(rows) < n:
        rows.add((int(rng.integers(hq)), int(rng.integers(nb))))
    return sorted(rows)


def stratified_rows(counts, seed, n_random=8):
    """Every head's first 4 and last 4 query blocks, the 8 sparsest rows past the
    first four blocks, and n_random seeded random rows."""
    hq, nb = counts.shape
    rows = set()
    for h in range(hq):
        for i in list(range(min(4, nb))) + list(range(max(0, nb - 4), nb)):
            rows.add((h, i))
    if nb > 4:
        order = np.argsort(counts[:, 4:], axis=None, kind="stable")[:8]
        for f in order:
            rows.add((int(f // (nb - 4)), int(f % (nb - 4)) + 4))
    rows.update(sample_rows(hq, nb, n_random, seed))
    return sorted(rows)


def check_rows(oq, ok_, ov, lists, out_np, lse_np, rows, tol, label):
    """Attention and LSE of the given (head, query block) rows against the oracle over
    the same lists; returns (worst max-abs, worst LSE error)."""
    worst = worst_lse = 0.0
    for h, i in rows:
        ref, ref_lse = O.attend_block(oq, ok_, ov, lists[h][i], h, i, 128, want_lse=True)
        got = out_np[i * 128:i * 128 + ref.shape[0], h]
        err = float(np.max(np.abs(got - ref)))
        worst = max(worst, err)
        assert err <= tol, f"{label}: row ({h}, {i}) max-abs {err:.3e} > {tol}"
        if lse_np is not None:
            lerr = float(np.max(np.abs(lse_np[h, i * 128:i * 128 + ref.shape[0]] - ref_lse)))
            worst_lse = max(worst_lse, lerr)
            assert lerr <= 1e-3 * max(1.0, float(np.abs(ref_lse).max())), f"{label}: row ({h}, {i}) LSE {lerr:.3e}"
    return worst, worst_lse


@pytest.mark.parametrize("k", [1, 2, 3])
def test_single_sequence_config(k):
    wl = cfg(k)
    print(f"[case] full-size config {k} {wl.name}", flush=True)
    q, kk, v, qs, ks, vs = to_device(wl)
    oq, ok_, ov = oracle_inputs(wl)
    pq_ref, pk_ref = O.pool(oq, 128), O.pool(ok_, 128)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    for alpha in wl.alphas:
        pq, pk = fp.discover(q, kk, qs, ks)
        idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
        out, lse = fp.sparse_attn(q, kk, v, idx, counts, qs, ks, vs, return_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(pq.cpu().numpy(), pq_ref)
        assert np.array_equal(pk.cpu().numpy(), pk_ref)
        s = O.block_scores(pq_ref, pk_ref, 1 / np.sqrt(128))
        P = O.reweight(s)
        del s
        keep = O.keep_mask(P, alpha, wl.n_sink, wl.n_local)
        nb = pq.shape[1]
        tri = nb * (nb + 1) // 2
        idx_np, cnt_np = idx.cpu().numpy(), counts.cpu().numpy()
        lists = [unpack_lists(idx_np, cnt_np, h, nb, tri) for h in range(wl.hq)]
        n_amb = check_lists(lists, dict(P=P, keep=keep), alpha, wl.n_sink, wl.n_local)
        del P, keep
        out_np = out.float().cpu().numpy()
        lse_np = lse.cpu().numpy()
        rows = stratified_rows(cnt_np, seed=100 + k)
        worst, worst_lse = check_rows(oq, ok_, ov, lists, out_np, lse_np, rows, tol, f"{wl.name} alpha={alpha}")
        msg = (f"{wl.name} alpha={alpha}: density {cnt_np.sum() / (wl.hq * tri):.4f}, in-band {n_amb}, "
               f"{len(rows)} sampled rows: max-abs {worst:.3e} (bound {tol}), LSE {worst_lse:.3e}")
        print("  " + msg, flush=True)
        record_margin(msg)


@pytest.mark.parametrize("k", [2, 3])
def test_dense_sampled_rows(k):
    """The same-GPU dense kernel at 128K bf16 and 256K fp8, sampled query blocks."""
    wl = cfg(k)
    print(f"[case] dense {wl.name} sampled rows", flush=True)
    q, kk, v, qs, ks, vs = to_device(wl)
    out = fp.dense_attn(q, kk, v, qs, ks, vs)
    torch.cuda.synchronize()
    oq, ok_, ov = oracle_inputs(wl)
    out_np = out.float().cpu().numpy()
    del out
    nb = -(-wl.L // 128)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    full = [np.arange(i + 1) for i in range(nb)]
    rows = sorted({(h, i) for h in range(wl.hq) for i in (0, 1, nb - 1)} | set(sample_rows(wl.hq, nb, 4, seed=7)))
    worst, _ = check_rows(oq, ok_, ov, [full] * wl.hq, out_np, None, rows, tol, f"dense {wl.name}")
    msg = f"dense {wl.name}: {len(rows)} sampled rows, max-abs {worst:.3e} (bound {tol})"
    print("  " + msg, flush=True)
    record_margin(msg)


def test_paged_batch_config():
    wl = cfg(4)
    print(f"[case] paged batch lengths={wl.lengths}", flush=True)
    q, kk, v, *_ = to_device(wl)
    kc, vc, table = to_device_paged(wl)
    batch = fp.VarlenBatch(wl.lengths, q.device)
    pq, pk = fp.discover_paged(q, kc, batch, page_table=table)
    idx, counts = fp.threshold_compact_varlen(pq, pk, batch, 0.1, wl.n_sink, wl.n_local)
    o_paged = fp.sparse_attn_paged(q, kc, vc, batch, idx, counts, page_table=table)
    o_packed = fp.sparse_attn_paged(q, kk, v, batch, idx, counts)
    torch.cuda.synchronize()
    assert torch.equal(o_paged, o_packed)
    oq, ok_, ov = oracle_inputs(wl)
    pq_np, pk_np = pq.cpu().numpy(), pk.cpu().numpy()
    idx_np, cnt_np = idx.cpu().numpy(), counts.cpu().numpy()
    out_np = o_paged.float().cpu().numpy()
    cu = wl.cu_seqlens
    worst = 0.0
    for s in range(wl.n_seqs):
        a, b = cu[s], cu[s + 1]
        b0, b1 = batch.cu_blocks[s], batch.cu_blocks[s + 1]
        sel = O.select_blocks(oq[a:b], ok_[a:b], 128, 0.1, wl.n_sink, wl.n_local)
        assert np.array_equal(pq_np[:, b0:b1], sel["pq"])
        assert np.array_equal(pk_np[:, b0:b1], sel["pk"])
        nb = b1 - b0
        lists = [unpack_lists(idx_np, cnt_np, h, nb, batch.total_tri, batch.cu_tri[s], b0) for h in range(wl.hq)]
        check_lists(lists, sel, 0.1, wl.n_sink, wl.n_local)
        rows = [(h, i) for h in range(wl.hq) for i in sorted({0, nb - 1})]
        err, _ = check_rows(oq[a:b], ok_[a:b], ov[a:b], lists, out_np[a:b], None, rows, TOL_BF16,
                            f"paged batch sequence {s}")
        worst = max(worst, err)
    msg = (f"paged batch: {wl.n_seqs} sequences x {wl.hq} heads x first/last block, max-abs {worst:.3e} "
           f"(bound {TOL_BF16})")
    print("  " + msg, flush=True)
    record_margin(msg)
