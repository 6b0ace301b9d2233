"""The no-allocation mean correction, fp_mean_correct_noalloc (the library's static
per-GPU scratch), against fp_mean_correct with a caller workspace, through the C ABI.
Two calls in a row on one GPU, the second with a smaller input (the scratch still
holds the first call's tile images), bf16 and fp8: corrected outputs and LSE must be
bit-identical to the workspace entry point's."""
import pytest
import torch

import block_sparse_long_pooled_amd as fp
import synth
from helpers import to_device

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def corrected_both_ways(wl, alpha):
    q, k, v, qs, ks, vs = to_device(wl)
    pq, pk = fp.discover(q, k, qs, ks)
    idx, counts = fp.threshold_compact(pq, pk, alpha, wl.n_sink, wl.n_local)
    out, lse = fp.sparse_attn(q, k, v, idx, counts, qs, ks, vs, return_lse=True)
    pv = fp.pool(v, vs)
    o_ws, l_ws = out.clone(), lse.clone()
    fp.mean_correct(q, pk, pv, idx, counts, o_ws, l_ws, q_scale=qs)
    o_na, l_na = out.clone(), lse.clone()
    fp.mean_correct_noalloc(q, pk, pv, idx, counts, o_na, l_na, q_scale=qs)
    torch.cuda.synchronize()
    return out, o_ws, l_ws, o_na, l_na


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_equals_workspace_entry_point_two_calls(dtype):
    for n, L in enumerate([128 * 40 + 77, 128 * 9 + 5]):  # second call smaller
        print(f"[case] mean_correct_noalloc {dtype} call {n + 1} L={L}", flush=True)
        wl = synth.make_workload(f"noalloc{n}", 8, 2, [L], seed=60 + n, dtype=dtype, alphas=(0.2,))
        out, o_ws, l_ws, o_na, l_na = corrected_both_ways(wl, 0.2)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
        assert not torch.equal(o_ws, out)  # the correction changed something
        assert torch.isfinite(o_na.float()).all() and torch.isfinite(l_na).all()
