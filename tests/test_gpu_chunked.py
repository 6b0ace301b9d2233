"""Chunked / prefix-cached prefill on the GPU against the fp64 oracle, through the
C ABI.  Each sequence brings len_q new queries (the last len_q positions) against a
K/V cache of len_k tokens; the cases mix a chunk that starts inside a block, a
block-aligned chunk, a whole sequence and a single query, with packed and paged
K/V, bf16 and fp8.  Rules as in the prefill parity tests: pooled means bit-exact,
lists exact outside the 1e-6 band, attention within 2e-2 (bf16) / 6e-2 (fp8) of the
oracle over the GPU's own lists; whole-sequence chunks equal the prefill call bit
for bit, paged equals packed bit for bit."""
import functools

import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
import synth
from helpers import BAND_REL, TOL_BF16, TOL_FP8, oracle_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ALPHA = 0.1


@functools.lru_cache(maxsize=None)
def case(name):
    if name == "bf16_paged":
        lk = [128 * 9 + 50, 128 * 20, 128 * 5 + 1, 700]
        lq = [300, 128 * 3, 128 * 5 + 1, 1]
        wl = synth.make_workload(name, 8, 2, lk, seed=31, paged=True, n_sink=1, n_local=3)
    elif name == "fp8":
        lk = [128 * 12 + 3, 128 * 4]
        lq = [200, 128 * 4]
        wl = synth.make_workload(name, 8, 2, lk, seed=32, dtype="fp8", paged=True, n_sink=1, n_local=4)
    else:
        raise KeyError(name)
    return wl, lq


def chunk_rows(wl, lq):
    """Row indices of the packed Q that form each sequence's chunk."""
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    return [np.arange(cu[s + 1] - n, cu[s + 1]) for s, n in enumerate(lq)]


def to_dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def run(name, paged=False, dense=False):
    wl, lq = case(name)
    rows = np.concatenate(chunk_rows(wl, lq))
    qc = to_dev(wl.q[rows], wl.dtype)
    k, v = to_dev(wl.k, wl.dtype), to_dev(wl.v, wl.dtype)
    sc = [None] * 3 if wl.dtype == "bf16" else [torch.from_numpy(x).cuda() for x in (wl.q_scale, wl.k_scale, wl.v_scale)]
    pt = None
    if paged:
        kc, vc, pt = synth.device_pages(wl)
        k, v = kc, vc
    batch = fp.ChunkedBatch(lq, wl.lengths, torch.device("cuda"))
    pq, pk = fp.discover_chunked(qc, k, batch, page_table=pt, q_scale=sc[0], k_scale=sc[1])
    idx, counts = fp.threshold_compact_chunked(pq, pk, batch, ALPHA, wl.n_sink, wl.n_local)
    if dense:
        idx = counts = None
    out, lse = fp.sparse_attn_chunked(qc, k, v, batch, idx, counts, page_table=pt, q_scale=sc[0], k_scale=sc[1],
                                      v_scale=sc[2], return_lse=True)
    torch.cuda.synchronize()
    res = dict(batch=batch, pq=pq.cpu().numpy(), pk=pk.cpu().numpy(), out=out.float().cpu().numpy(),
               lse=lse.cpu().numpy())
    if idx is not None:
        res.update(idx=idx.cpu().numpy(), counts=counts.cpu().numpy())
    return wl, lq, res


def seq_inputs(wl, lq, s):
    q, k, v = oracle_inputs(wl)
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    a, b = cu[s], cu[s + 1]
    return q[b - lq[s]:b], k[a:b], v[a:b]


def gpu_lists(res, h, s):
    bt = res["batch"]
    out = []
    for r in range(bt.nq[s]):
        I = bt.I0[s] + r
        o = h * bt.total_tri + bt.row_offset(s, I)
        c = int(res["counts"][h, bt.cu_qblocks[s] + r])
        out.append(res["idx"][o:o + c].astype(np.int64))
    return out


@pytest.mark.parametrize("name,paged", [("bf16_paged", False), ("bf16_paged", True), ("fp8", False), ("fp8", True)])
def test_chunked_discover_bit_exact(name, paged):
    print(f"[case] chunked discover {name} paged={paged}", flush=True)
    wl, lq, res = run(name, paged)
    bt = res["batch"]
    for s in range(wl.n_seqs):
        qc, k, _ = seq_inputs(wl, lq, s)
        q0, q1 = bt.cu_qblocks[s], bt.cu_qblocks[s + 1]
        k0, k1 = bt.cu_kblocks[s], bt.cu_kblocks[s + 1]
        assert np.array_equal(res["pq"][:, q0:q1], O.pool_chunk(qc, wl.lengths[s], 128)), s
        assert np.array_equal(res["pk"][:, k0:k1], O.pool(k, 128)), s


@pytest.mark.parametrize("name,paged", [("bf16_paged", False), ("bf16_paged", True), ("fp8", False), ("fp8", True)])
def test_chunked_lists_and_attention_match_oracle(name, paged):
    print(f"[case] chunked lists + attention {name} paged={paged}", flush=True)
    wl, lq, res = run(name, paged)
    bt = res["batch"]
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    for s in range(wl.n_seqs):
        qc, k, v = seq_inputs(wl, lq, s)
        sel = O.select_blocks_chunked(qc, k, 128, ALPHA, wl.n_sink, wl.n_local)
        assert sel["I0"] == bt.I0[s] and sel["nq"] == bt.nq[s]
        lists = []
        for h in range(wl.hq):
            got = gpu_lists(res, h, s)
            lists.append(got)
            for r, lst in enumerate(got):
                I = bt.I0[s] + r
                assert lst.size >= 1 and np.all(np.diff(lst) > 0) and lst[-1] == I, (s, h, r, lst)
                g = np.zeros(I + 1, dtype=bool)
                g[lst] = True
                diff = np.nonzero(g != sel["keep"][h, r, :I + 1])[0]
                j = np.arange(I + 1)
                forced = (j < wl.n_sink) | (j > I - wl.n_local)
                band = np.abs(sel["P"][h, r, :I + 1] - ALPHA) <= BAND_REL * ALPHA
                assert all(band[x] and not forced[x] for x in diff), (s, h, r, diff)
        ref, ref_lse = O.sparse_attention_chunked(qc, k, v, lists, 128, want_lse=True)
        got = res["out"][cu_q[s]:cu_q[s + 1]]
        err = np.max(np.abs(got - ref))
        assert err <= tol, (s, err)
        # same LSE rule as the prefill parity test (bf16 sums the bf16-rounded P:
        # up to 2^-9 relative on the sum)
        lerr = np.max(np.abs(res["lse"][:, cu_q[s]:cu_q[s + 1]] - ref_lse))
        assert lerr <= 1e-3 * max(1.0, np.abs(ref_lse).max()), (s, lerr)


def test_chunked_dense_matches_oracle():
    wl, lq, res = run("bf16_paged", dense=True)
    print("[case] chunked dense", flush=True)
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    for s in range(wl.n_seqs):
        qc, k, v = seq_inputs(wl, lq, s)
        I0, nq = O.chunk_blocks(lq[s], wl.lengths[s], 128)
        full = [[np.arange(I0 + r + 1) for r in range(nq)] for _ in range(wl.hq)]
        ref = O.sparse_attention_chunked(qc, k, v, full, 128)
        assert np.max(np.abs(res["out"][cu_q[s]:cu_q[s + 1]] - ref)) <= TOL_BF16, s


@pytest.mark.parametrize("name", ["bf16_paged", "fp8"])
def test_chunked_paged_equals_packed_bit_exact(name):
    print(f"[case] chunked paged vs packed {name}", flush=True)
    _, _, a = run(name, paged=False)
    _, _, b = run(name, paged=True)
    for key in ("pq", "pk", "idx", "counts", "out", "lse"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_whole_sequence_chunk_equals_prefill_bit_exact():
    """Sequence 2 of the case is a whole sequence (len_q = len_k): its chunked output
    equals the single-sequence prefill call on the same tokens."""
    print("[case] whole-sequence chunk vs prefill", flush=True)
    wl, lq, res = run("bf16_paged")
    s = 2
    assert lq[s] == wl.lengths[s]
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    a, b = cu[s], cu[s + 1]
    q, k, v = (to_dev(x[a:b], "bf16") for x in (wl.q, wl.k, wl.v))
    pq, pk = fp.discover(q, k)
    idx, counts = fp.threshold_compact(pq, pk, ALPHA, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, return_lse=True)
    torch.cuda.synchronize()
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    assert np.array_equal(res["out"][cu_q[s]:cu_q[s + 1]], out.float().cpu().numpy())
    assert np.array_equal(res["lse"][:, cu_q[s]:cu_q[s + 1]], lse.cpu().numpy())
