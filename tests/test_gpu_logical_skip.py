"""Logical-skip ablation, GPU side (FlashPrefill Method 3 contrasts a masked loop
over every block with the physical jumps over compacted lists).

  * the bit-packed mask holds exactly the decisions of the lists (same fp64 scores,
    same threshold), and the bits above the diagonal are zero;
  * the masked loop visits the same blocks in the same order as the list kernel, so
    outputs and LSE are bit-identical (bf16 and fp8), and alpha = 0 equals the
    dense kernel;
  * a row whose mask is empty gives NaN output, not a fault.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import oracle as O
from helpers import TOL_BF16, oracle_inputs, to_device, unpack_lists
from test_gpu_parity import workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [("tiny", 0.1), ("gqa_ragged", 0.05), ("fp8_ragged", 0.1), ("mha_one_block", 0.1), ("gqa7", 0.2)]


def mask_bits(mask, nb):
    """[hq, nb, W] int32 words -> bool [hq, nb, 32 W] (bit j%32 of word j//32)."""
    w = mask.cpu().numpy().astype(np.uint32)
    bits = (w[..., None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[0], nb, -1).astype(bool)


def select_both(name, alpha):
    wl = workload(name)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    mask = fp.threshold_mask(pq, pk, alpha, wl.n_sink, wl.n_local)
    torch.cuda.synchronize()
    return wl, (q, k, v, qs, ks, vs), idx, counts, mask


@pytest.mark.parametrize("name,alpha", CASES)
def test_mask_equals_lists(name, alpha):
    print(f"[case] mask vs lists {name} alpha={alpha}", flush=True)
    wl, _, idx, counts, mask = select_both(name, alpha)
    nb = -(-wl.L // 128)
    bits = mask_bits(mask, nb)
    idx_h, counts_h = idx.cpu().numpy(), counts.cpu().numpy()
    for h in range(wl.hq):
        lists = unpack_lists(idx_h, counts_h, h, nb, nb * (nb + 1) // 2)
        for i in range(nb):
            want = np.zeros(bits.shape[-1], dtype=bool)
            want[lists[i]] = True
            # every word that covers some j <= i is written: compare it whole
            upto = ((i >> 5) + 1) * 32
            assert np.array_equal(bits[h, i, :upto], want[:upto]), (h, i)


@pytest.mark.parametrize("name,alpha", CASES)
def test_masked_attention_bit_identical_to_lists(name, alpha):
    print(f"[case] masked attention {name} alpha={alpha}", flush=True)
    wl, (q, k, v, qs, ks, vs), idx, counts, mask = select_both(name, alpha)
    for want_lse in (False, True):
        a = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=want_lse)
        b = fp.sparse_attn_masked(q, k, v, mask, qs, ks, vs, return_lse=want_lse)
        torch.cuda.synchronize()
        if want_lse:
            assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        else:
            assert torch.equal(a, b)


def test_masked_alpha_zero_equals_dense():
    wl = workload("gqa_ragged")
    print(f"[case] masked alpha=0 vs dense L={wl.L}", flush=True)
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    mask = fp.threshold_mask(pq, pk, 0.0, wl.n_sink, wl.n_local)
    a = fp.dense_attn(q, k, v, qs, ks, vs)
    b = fp.sparse_attn_masked(q, k, v, mask, qs, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_masked_attention_matches_oracle():
    wl = workload("tiny")
    print(f"[case] masked attention vs oracle L={wl.L}", flush=True)
    alpha = 0.1
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    mask = fp.threshold_mask(pq, pk, alpha, wl.n_sink, wl.n_local)
    out = fp.sparse_attn_masked(q, k, v, mask, qs, ks, vs)
    torch.cuda.synchronize()
    nb = -(-wl.L // 128)
    bits = mask_bits(mask, nb)
    lists = [[np.nonzero(bits[h, i, :i + 1])[0] for i in range(nb)] for h in range(wl.hq)]
    oq, ok_, ov = oracle_inputs(wl)
    ref = O.sparse_attention(oq, ok_, ov, lists, 128)
    err = np.max(np.abs(out.float().cpu().numpy() - ref))
    assert err <= TOL_BF16, err


def test_empty_mask_row_gives_nan():
    wl = workload("gqa_ragged")
    print(f"[case] empty mask row L={wl.L}", flush=True)
    alpha = 0.1
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    mask = fp.threshold_mask(pq, pk, alpha, wl.n_sink, wl.n_local)
    h, i = 1, 5
    mask[h, i].zero_()
    a = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs)
    b = fp.sparse_attn_masked(q, k, v, mask, qs, ks, vs)
    torch.cuda.synchronize()
    rows = slice(128 * i, 128 * (i + 1))
    assert torch.isnan(b[rows, h].float()).all()
    b[rows, h] = a[rows, h]
    assert torch.equal(a, b)
