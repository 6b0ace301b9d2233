"""The V2 mean correction, GPU side (an assumption kept outside the oracle-checked
core; its definition is oracle.mean_correction): pooled V is bit-exact; the
corrected output and LSE match the oracle's definition over the GPU's own lists;
with nothing pruned (alpha = 0) the pass leaves output and LSE unchanged."""
import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
from helpers import TOL_BF16, TOL_FP8, oracle_inputs, to_device, unpack_lists
import synth
from test_gpu_parity import workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("name", ["gqa_ragged", "fp8_ragged"])
def test_pool_v_bit_exact(name):
    wl = workload(name)
    print(f"[case] pool V {name}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pv = fp.pool(v, vs)
    torch.cuda.synchronize()
    _, _, ov = oracle_inputs(wl)
    assert np.array_equal(pv.cpu().numpy(), O.pool(ov, 128))


@pytest.mark.parametrize("name,alpha", [("tiny", 0.1), ("gqa_ragged", 0.3), ("fp8_ragged", 0.1), ("gqa7", 0.2)])
def test_mean_correction_matches_definition(name, alpha):
    wl = workload(name)
    print(f"[case] mean correction {name} alpha={alpha}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    pv = fp.pool(v, vs)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=True)
    fp.mean_correct(q, pk, pv, idx, counts, out, lse, q_scale=qs)
    torch.cuda.synchronize()
    nb = -(-wl.L // 128)
    lists = [unpack_lists(idx.cpu().numpy(), counts.cpu().numpy(), h, nb, nb * (nb + 1) // 2) for h in range(wl.hq)]
    oq, ok_, ov = oracle_inputs(wl)
    ref, ref_lse = O.mean_correction(oq, ok_, ov, lists, 128, want_lse=True)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= tol
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3 * max(1.0, np.abs(ref_lse).max())


def test_mean_correction_is_noop_without_pruning():
    wl = workload("gqa_ragged")
    print(f"[case] mean correction alpha=0 L={wl.L}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    pv = fp.pool(v, vs)
    idx, counts = fp.threshold_compact(pq, pk, 0.0, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=True)
    o2, l2 = out.clone(), lse.clone()
    fp.mean_correct(q, pk, pv, idx, counts, o2, l2, q_scale=qs)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("L", [100, 129, 128 * 33 + 5])
def test_mean_correction_edge_lengths(L):
    """One partial block (nothing below the diagonal), two blocks, and a ragged
    33-block sequence with alpha > 1, no sink and a 1-block window, so every
    off-diagonal block is pruned and enters through its mean."""
    wl = synth.make_workload(f"mc_edge_{L}", 4, 2, [L], seed=41, alphas=(1.5,), n_sink=0, n_local=1)
    print(f"[case] mean correction edge L={L}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    pv = fp.pool(v, vs)
    idx, counts = fp.threshold_compact(pq, pk, 1.5, 0, 1)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=True)
    o0, l0 = out.clone(), lse.clone()
    fp.mean_correct(q, pk, pv, idx, counts, out, lse, q_scale=qs)
    torch.cuda.synchronize()
    nb = -(-L // 128)
    assert torch.equal(counts.cpu(), torch.ones((wl.hq, nb), dtype=torch.int32))
    lists = [unpack_lists(idx.cpu().numpy(), counts.cpu().numpy(), h, nb, nb * (nb + 1) // 2) for h in range(wl.hq)]
    oq, ok_, ov = oracle_inputs(wl)
    ref, ref_lse = O.mean_correction(oq, ok_, ov, lists, 128, want_lse=True)
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= TOL_BF16
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3 * max(1.0, np.abs(ref_lse).max())
    # block 0 has nothing to correct: its rows are untouched
    assert torch.equal(out[:min(L, 128)], o0[:min(L, 128)]) and torch.equal(lse[:, :min(L, 128)], l0[:, :min(L, 128)])


@pytest.mark.parametrize("dtype,paged", [("bf16", True), ("fp8", False)])
def test_mean_correction_varlen_matches_definition_per_sequence(dtype, paged):
    """Packed batch (ragged lengths, an empty and a single-block sequence): pooled V per
    sequence is bit-exact (paged or packed V), and the corrected output and LSE of every
    sequence match oracle.mean_correction on that sequence over the GPU's own lists."""
    lengths = [128 * 23 + 77, 0, 100, 128 * 9, 128 * 40 + 3]
    wl = synth.make_workload(f"mc_varlen_{dtype}", 8, 2, lengths, seed=47, dtype=dtype, paged=True,
                             alphas=(0.2,), n_sink=1, n_local=3)
    print(f"[case] mean correction varlen {dtype} paged={paged} lengths={lengths}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    kc, vc, table = synth.device_pages(wl)
    batch = fp.VarlenBatch(wl.lengths, q.device)
    kk, vv, pt = (kc, vc, table) if paged else (k, v, None)
    pq, pk = fp.discover_paged(q, kk, batch, page_table=pt, q_scale=qs, k_scale=ks)
    pv = fp.pool_varlen(vv, batch, page_table=pt, scale=vs)
    idx, counts = fp.threshold_compact_varlen(pq, pk, batch, 0.2, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn_paged(q, kk, vv, batch, idx, counts, page_table=pt, q_scale=qs, k_scale=ks,
                                    v_scale=vs, return_lse=True)
    fp.mean_correct_varlen(q, pk, pv, batch, idx, counts, out, lse, q_scale=qs)
    torch.cuda.synchronize()
    oq, ok_, ov = oracle_inputs(wl)
    idx_np, cnt_np = idx.cpu().numpy(), counts.cpu().numpy()
    pv_np, out_np, lse_np = pv.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_FP8
    cu = wl.cu_seqlens
    for s in range(wl.n_seqs):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        b0, b1 = batch.cu_blocks[s], batch.cu_blocks[s + 1]
        assert np.array_equal(pv_np[:, b0:b1], O.pool(ov[a:b], 128)), s
        lists = [unpack_lists(idx_np, cnt_np, h, b1 - b0, batch.total_tri, batch.cu_tri[s], b0) for h in range(wl.hq)]
        ref, ref_lse = O.mean_correction(oq[a:b], ok_[a:b], ov[a:b], lists, 128, want_lse=True)
        assert np.max(np.abs(out_np[a:b] - ref)) <= tol, s
        assert np.max(np.abs(lse_np[:, a:b] - ref_lse)) <= 1e-3 * max(1.0, np.abs(ref_lse).max()), s


def test_mean_correction_varlen_single_sequence_equals_contiguous():
    """A one-sequence batch gives bit for bit what the single-sequence call gives."""
    wl = workload("gqa_ragged")
    print(f"[case] mean correction varlen == single L={wl.L}", flush=True)
    q, k, v, *_ = to_device(wl)
    batch = fp.VarlenBatch([wl.L], q.device)
    pq, pk = fp.discover(q, k)
    pv = fp.pool(v)
    assert torch.equal(fp.pool_varlen(v, batch), pv)
    idx, counts = fp.threshold_compact(pq, pk, 0.3, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, return_lse=True)
    o1, l1 = out.clone(), lse.clone()
    o2, l2 = out.clone(), lse.clone()
    fp.mean_correct(q, pk, pv, idx, counts, o1, l1)
    fp.mean_correct_varlen(q, pk, pv, batch, idx, counts, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert not torch.equal(o1, out)
