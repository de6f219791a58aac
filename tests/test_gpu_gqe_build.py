"""The GQE output build on the GPU (kept experts concatenated, the weighted-sum
slot per group, the shared head) against the float64 oracle: indices
bit-exact, gates within 1e-6, every output within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_GATE, dev, max_abs, np64, sample_tokens, say
from workloads import gqe_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _inputs(B, h, g, T, d, seed, device="cpu"):
    q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=seed, device=device)
    qs = prefill_inputs(B, 1, 1, T, d, "bf16", seed=seed + 1, device=device)[0][:, 0].contiguous()
    return q, qs, k, v, lg


@pytest.mark.parametrize("B,h,g,T,d,top_k,skv,out_dt", [
    (2, 16, 8, 200, 128, 1, 0, torch.float32),    # the pages' shape: 8 routed + 1 shared
    (1, 8, 2, 300, 128, 2, 1, torch.bfloat16),
    (2, 12, 4, 129, 64, 3, 3, torch.float32),
    (1, 32, 8, 520, 128, 4, 7, torch.float32),    # every expert kept
])
def test_gqe_build_shapes(B, h, g, T, d, top_k, skv, out_dt):
    import gqa_routed_query_amd as gq

    dv = dev()
    say(f"gqe build B={B} h={h} g={g} T={T} d={d} k={top_k} shared_kv={skv} out={out_dt}")
    q, qs, k, v, lg = _inputs(B, h, g, T, d, seed=900 + T)
    concat, wsum, shared, idx, gate = gq.gqe_prefill_build(
        q.to(dv), qs.to(dv), k.to(dv), v.to(dv), lg.to(dv), top_k, shared_kv=skv, out_dtype=out_dt)
    torch.cuda.synchronize()
    rc, rw, rs, ridx, rgate = oracle.gqe_build_ref(q, qs, k, v, lg, top_k, shared_kv=skv)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    assert max_abs(concat, rc) <= TOL_BF16
    assert max_abs(wsum, rw) <= TOL_BF16
    assert max_abs(shared, rs) <= TOL_BF16


def test_gqe_build_wsum_is_routed_output_summed_over_group():
    """The weighted-sum slot of a group equals gqe_routed_prefill's output
    (gate x row for kept heads, 0 for the others) summed over the group's
    heads, both on the GPU."""
    import gqa_routed_query_amd as gq

    dv = dev()
    B, h, g, T, d = 2, 16, 4, 257, 128
    say("gqe build vs routed prefill")
    q, qs, k, v, lg = _inputs(B, h, g, T, d, seed=920, device=dv)
    _, wsum, _, idx, gate = gq.gqe_prefill_build(q, qs, k, v, lg, 2, out_dtype=torch.float32)
    out, idx2, gate2 = gq.gqe_routed_prefill(q, k, v, lg, 2, out_dtype=torch.float32,
                                             workspace=None)  # same arithmetic: no key splits
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(gate, gate2)
    grp = out.view(B, g, h // g, T, d).sum(2).permute(0, 2, 1, 3)   # [B,T,g,d]
    assert max_abs(wsum, grp) <= 1e-4


@pytest.mark.parametrize("h,top_k", [(16, 1), (32, 2)])
def test_gqe_build_long_sequence(h, top_k):
    """B=2, T=4096, g=8, d=128 (the pages' 16-head shape with k=1, and the
    32-head shape with k=2): all indices bit-exact, sampled tokens of every
    output against the oracle's rows."""
    import gqa_routed_query_amd as gq

    dv = dev()
    B, g, T, d = 2, 8, 4096, 128
    say(f"gqe build long h={h} k={top_k}")
    q, qs, k, v, lg = _inputs(B, h, g, T, d, seed=930 + h, device=dv)
    concat, wsum, shared, idx, gate = gq.gqe_prefill_build(q, qs, k, v, lg, top_k, shared_kv=5,
                                                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ridx, rgate = oracle.gqe_topk_ref(lg.cpu(), g, top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    qc, qsc, kc, vc = q.cpu(), qs.cpu(), k.cpu(), v.cpu()
    worst = 0.0
    for t in sample_tokens(T, 12, seed=931):
        for b in range(B):
            for gam in (0, 3, g - 1):
                acc = 0.0
                for j in range(top_k):
                    row = oracle.gqa_ref_row(qc, kc, vc, b, int(ridx[b, t, gam, j]), t)
                    worst = max(worst, float(np.abs(np64(concat[b, t, gam, j]) - row).max()))
                    acc = acc + rgate[b, t, gam, j] * row
                worst = max(worst, float(np.abs(np64(wsum[b, t, gam]) - acc).max()))
            srow = oracle.gqa_ref_row(qsc[:, None], kc[:, 5:6], vc[:, 5:6], b, 0, t)
            worst = max(worst, float(np.abs(np64(shared[b, t]) - srow).max()))
    assert worst <= TOL_BF16, worst
