"""Guard zones around every output buffer: no entry point writes outside its extent.

Each output (pooled means, idx, counts, score map, block mask, attention output,
LSE, mean-correction workspace, single sequence and packed batch) is carved out of a larger allocation whose leading
and trailing guard zones hold a fixed byte pattern.  After the calls the guards
must still hold that pattern, for single-sequence, fp8, packed-batch (packed and
paged K/V) and chunked-prefill runs.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import synth
from helpers import to_device, to_device_paged

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GUARD_BYTES = 4096
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape`/`dtype` inside a byte buffer with guard zones on both sides."""

    def __init__(self, shape, dtype, device="cuda"):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((GUARD_BYTES + n + GUARD_BYTES,), PATTERN, dtype=torch.uint8, device=device)
        self.n = n
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)

    def intact(self) -> bool:
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.n:]
        return bool((head == PATTERN).all().item()) and bool((tail == PATTERN).all().item())


def assert_intact(bufs: dict):
    torch.cuda.synchronize()
    bad = [name for name, b in bufs.items() if not b.intact()]
    assert not bad, f"guard zone overwritten next to {bad}"


def zeroed(shape, dtype):
    g = Guarded(shape, dtype)
    g.t.zero_()
    return g


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_single_sequence_outputs_stay_in_bounds(dtype):
    print(f"[case] canary single sequence {dtype}", flush=True)
    wl = synth.make_workload("canary", 8, 2, [128 * 21 + 45], seed=41, dtype=dtype, alphas=(0.1,))
    q, k, v, qs, ks, vs = to_device(wl)
    L, hq, hkv, d = wl.L, wl.hq, wl.hkv, 128
    nb = -(-L // 128)
    b = {
        "pooled_q": Guarded((hq, nb, d), torch.float64), "pooled_k": Guarded((hkv, nb, d), torch.float64),
        "idx": zeroed((fp.idx_capacity(hq, nb),), torch.int32), "counts": Guarded((hq, nb), torch.int32),
        "scores": Guarded((hq, nb, nb), torch.float64),
        "out": Guarded((L, hq, d), torch.bfloat16), "lse": Guarded((hq, L), torch.float32),
        "dense_out": Guarded((L, hq, d), torch.bfloat16),
    }
    fp.discover(q, k, qs, ks, pooled_q=b["pooled_q"].t, pooled_k=b["pooled_k"].t)
    fp.threshold_compact(b["pooled_q"].t, b["pooled_k"].t, 0.1, wl.n_sink, wl.n_local, idx=b["idx"].t,
                         counts=b["counts"].t, scores=b["scores"].t)
    fp.sparse_attn(q, k, v, b["idx"].t, b["counts"].t, qs, ks, vs, out=b["out"].t, lse=b["lse"].t)
    fp.dense_attn(q, k, v, qs, ks, vs, out=b["dense_out"].t)
    assert_intact(b)
    assert torch.isfinite(b["out"].t.float()).all()


def test_mask_union_grouped_masked_and_mean_correction_stay_in_bounds():
    print("[case] canary mask / union / grouped / masked / mean correction", flush=True)
    wl = synth.make_workload("canary2", 8, 2, [128 * 19 + 7], seed=42, alphas=(0.1,))
    q, k, v, *_ = to_device(wl)
    L, hq, hkv, d = wl.L, wl.hq, wl.hkv, 128
    nb = -(-L // 128)
    pq, pk = fp.discover(q, k)
    b = {
        "mask": zeroed((hq, nb, fp.mask_words(nb)), torch.int32),
        "gidx": zeroed((fp.idx_capacity(hkv, nb),), torch.int32), "gcounts": Guarded((hkv, nb), torch.int32),
        "gout": Guarded((L, hq, d), torch.bfloat16), "mout": Guarded((L, hq, d), torch.bfloat16),
        "pooled_v": Guarded((hkv, nb, d), torch.float64),
        "workspace": Guarded((int(fp.load().fp_mean_correct_workspace_bytes(L, hkv)),), torch.uint8),
        "corr_out": Guarded((L, hq, d), torch.bfloat16), "corr_lse": Guarded((hq, L), torch.float32),
    }
    fp.threshold_mask(pq, pk, 0.1, wl.n_sink, wl.n_local, mask=b["mask"].t)
    fp.union_compact(b["mask"].t, hkv, idx=b["gidx"].t, counts=b["gcounts"].t)
    fp.sparse_attn_grouped(q, k, v, b["gidx"].t, b["gcounts"].t, out=b["gout"].t)
    fp.sparse_attn_masked(q, k, v, b["mask"].t, out=b["mout"].t)
    idx, counts = fp.threshold_compact(pq, pk, 0.1, wl.n_sink, wl.n_local)
    fp.sparse_attn(q, k, v, idx, counts, out=b["corr_out"].t, lse=b["corr_lse"].t)
    fp.pool(v, pooled=b["pooled_v"].t)
    fp.mean_correct(q, pk, b["pooled_v"].t, idx, counts, b["corr_out"].t, b["corr_lse"].t,
                    workspace=b["workspace"].t)
    assert_intact(b)


@pytest.mark.parametrize("paged", [False, True])
def test_packed_batch_outputs_stay_in_bounds(paged):
    print(f"[case] canary packed batch paged={paged}", flush=True)
    wl = synth.make_workload("canary3", 8, 2, [700, 0, 128 * 5, 1333], seed=43, alphas=(0.1,), paged=True)
    q, k, v, *_ = to_device(wl)
    kc, vc, table = to_device_paged(wl)
    kk, vv, pt = (kc, vc, table) if paged else (k, v, None)
    batch = fp.VarlenBatch(wl.lengths, q.device)
    hq, hkv, d = wl.hq, wl.hkv, 128
    b = {
        "pooled_q": Guarded((hq, batch.total_blocks, d), torch.float64),
        "pooled_k": Guarded((hkv, batch.total_blocks, d), torch.float64),
        "idx": zeroed((hq * batch.total_tri,), torch.int32), "counts": Guarded((hq, batch.total_blocks), torch.int32),
        "out": Guarded((batch.total_tokens, hq, d), torch.bfloat16),
        "lse": Guarded((hq, batch.total_tokens), torch.float32),
        "dense_out": Guarded((batch.total_tokens, hq, d), torch.bfloat16),
        "pooled_v": Guarded((hkv, batch.total_blocks, d), torch.float64),
        "mc_workspace": Guarded((int(fp.load().fp_mean_correct_varlen_workspace_bytes(batch.total_blocks,
                                                                                       batch.n_seqs, hkv)),),
                                torch.uint8),
    }
    fp.discover_paged(q, kk, batch, page_table=pt, pooled_q=b["pooled_q"].t, pooled_k=b["pooled_k"].t)
    fp.threshold_compact_varlen(b["pooled_q"].t, b["pooled_k"].t, batch, 0.1, wl.n_sink, wl.n_local,
                                idx=b["idx"].t, counts=b["counts"].t)
    fp.sparse_attn_paged(q, kk, vv, batch, b["idx"].t, b["counts"].t, page_table=pt, out=b["out"].t,
                         lse=b["lse"].t)
    fp.sparse_attn_paged(q, kk, vv, batch, page_table=pt, out=b["dense_out"].t)
    fp.pool_varlen(vv, batch, page_table=pt, pooled=b["pooled_v"].t)
    fp.mean_correct_varlen(q, b["pooled_k"].t, b["pooled_v"].t, batch, b["idx"].t, b["counts"].t, b["out"].t,
                           b["lse"].t, workspace=b["mc_workspace"].t)
    assert_intact(b)


@pytest.mark.parametrize("paged", [False, True])
def test_chunked_outputs_stay_in_bounds(paged):
    print(f"[case] canary chunked paged={paged}", flush=True)
    lens = [128 * 9 + 30, 500, 128 * 4]
    wl = synth.make_workload("canary4", 8, 2, lens, seed=44, alphas=(0.1,), paged=True)
    q, k, v, *_ = to_device(wl)
    kc, vc, table = to_device_paged(wl)
    kk, vv, pt = (kc, vc, table) if paged else (k, v, None)
    q_lens = [300, 1, 128 * 2]
    cu = wl.cu_seqlens
    qc = torch.cat([q[cu[s + 1] - n:cu[s + 1]] for s, n in enumerate(q_lens)])
    batch = fp.ChunkedBatch(q_lens, lens, q.device)
    hq, hkv, d = wl.hq, wl.hkv, 128
    b = {
        "pooled_q": Guarded((hq, batch.total_qblocks, d), torch.float64),
        "pooled_k": Guarded((hkv, batch.total_kblocks, d), torch.float64),
        "idx": zeroed((hq * batch.total_tri,), torch.int32), "counts": Guarded((hq, batch.total_qblocks), torch.int32),
        "out": Guarded((batch.total_q, hq, d), torch.bfloat16),
        "lse": Guarded((hq, batch.total_q), torch.float32),
    }
    fp.discover_chunked(qc, kk, batch, page_table=pt, pooled_q=b["pooled_q"].t, pooled_k=b["pooled_k"].t)
    fp.threshold_compact_chunked(b["pooled_q"].t, b["pooled_k"].t, batch, 0.1, wl.n_sink, wl.n_local,
                                 idx=b["idx"].t, counts=b["counts"].t)
    fp.sparse_attn_chunked(qc, kk, vv, batch, b["idx"].t, b["counts"].t, page_table=pt, out=b["out"].t,
                           lse=b["lse"].t)
    assert_intact(b)
