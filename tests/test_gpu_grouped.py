"""Group-shared lists on the GPU: one list per KV-head group, the union of its
query heads' lists; every head of the group attends over it.

  * the union lists equal the union of the GPU's own per-head lists exactly, and
    the oracle's group union outside the 1e-6 band of any head of the group;
  * attention matches the oracle over the GPU's group lists (2e-2 bf16, 6e-2 fp8);
  * with one query head per KV head the grouped call equals the per-head call,
    and with alpha = 0 it equals the dense kernel, bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
import synth
from helpers import BAND_REL, TOL_BF16, TOL_FP8, oracle_inputs, to_device, unpack_lists
from test_gpu_parity import workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [("gqa_ragged", 0.05), ("fp8_ragged", 0.1), ("gqa7", 0.2)]


def grouped(name, alpha):
    wl = workload(name)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    mask = fp.threshold_mask(pq, pk, alpha, wl.n_sink, wl.n_local)
    gidx, gcounts = fp.union_compact(mask, wl.hkv)
    torch.cuda.synchronize()
    return wl, (q, k, v, qs, ks, vs), idx, counts, gidx, gcounts


@pytest.mark.parametrize("name,alpha", CASES)
def test_union_lists(name, alpha):
    print(f"[case] union lists {name} alpha={alpha}", flush=True)
    wl, _, idx, counts, gidx, gcounts = grouped(name, alpha)
    nb = -(-wl.L // 128)
    tri = nb * (nb + 1) // 2
    G = wl.hq // wl.hkv
    idx_h, counts_h = idx.cpu().numpy(), counts.cpu().numpy()
    gi, gc = gidx.cpu().numpy(), gcounts.cpu().numpy()
    per_head = [unpack_lists(idx_h, counts_h, h, nb, tri) for h in range(wl.hq)]
    q, k, _ = oracle_inputs(wl)
    sel = O.select_blocks_grouped(q, k, 128, alpha, wl.n_sink, wl.n_local)
    P = sel["heads"]["P"]
    for g in range(wl.hkv):
        lists = unpack_lists(gi, gc, g, nb, tri)
        for i in range(nb):
            want = sorted(set().union(*[set(int(x) for x in per_head[h][i]) for h in range(g * G, (g + 1) * G)]))
            assert [int(x) for x in lists[i]] == want, (g, i)
            got = np.zeros(i + 1, dtype=bool)
            got[lists[i]] = True
            diff = np.nonzero(got != sel["keep"][g, i, :i + 1])[0]
            for j in diff:
                assert any(abs(P[h, i, j] - alpha) <= BAND_REL * alpha for h in range(g * G, (g + 1) * G)), (g, i, j)


@pytest.mark.parametrize("name,alpha", CASES)
def test_grouped_attention_matches_oracle(name, alpha):
    print(f"[case] grouped attention {name} alpha={alpha}", flush=True)
    wl, (q, k, v, qs, ks, vs), _, _, gidx, gcounts = grouped(name, alpha)
    out, lse = fp.sparse_attn_grouped(q, k, v, gidx, gcounts, qs, ks, vs, return_lse=True)
    torch.cuda.synchronize()
    nb = -(-wl.L // 128)
    tri = nb * (nb + 1) // 2
    G = wl.hq // wl.hkv
    gi, gc = gidx.cpu().numpy(), gcounts.cpu().numpy()
    glists = [unpack_lists(gi, gc, g, nb, tri) for g in range(wl.hkv)]
    lists = [glists[h // G] for h in range(wl.hq)]
    oq, ok_, ov = oracle_inputs(wl)
    ref, ref_lse = O.sparse_attention(oq, ok_, ov, lists, 128, want_lse=True)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_FP8
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= tol
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3 * max(1.0, np.abs(ref_lse).max())


def test_grouped_with_one_head_per_group_equals_per_head():
    wl = workload("mha_one_block")
    assert wl.hq == wl.hkv
    print(f"[case] grouped MHA L={wl.L}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, 0.1, wl.n_sink, wl.n_local)
    mask = fp.threshold_mask(pq, pk, 0.1, wl.n_sink, wl.n_local)
    gidx, gcounts = fp.union_compact(mask, wl.hkv)
    a = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs)
    b = fp.sparse_attn_grouped(q, k, v, gidx, gcounts, qs, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(gcounts, counts)
    assert torch.equal(a, b)


def test_grouped_alpha_zero_equals_dense():
    wl = workload("gqa_ragged")
    print(f"[case] grouped alpha=0 L={wl.L}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    mask = fp.threshold_mask(pq, pk, 0.0, wl.n_sink, wl.n_local)
    gidx, gcounts = fp.union_compact(mask, wl.hkv)
    a = fp.dense_attn(q, k, v, qs, ks, vs)
    b = fp.sparse_attn_grouped(q, k, v, gidx, gcounts, qs, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
