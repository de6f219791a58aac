"""GQE routed prefill on the GPU against the float64 oracle: router indices
bit-exact, gates within 1e-6, outputs within the dtype tolerance, unselected
rows exactly zero."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, TOL_GATE, dev, max_abs, np64, sample_tokens, say
from workloads import WORKLOADS, gqe_inputs, gqe_sweep_points, prefill_inputs

pytestmark = pytest.mark.gpu


def _run(q, k, v, lg, top_k, causal=True, out_dtype=torch.float32, workspace=True):
    """The routed call into an output filled with NaN beforehand, so every row
    the launch leaves unwritten (a kept row or a zero row) shows."""
    import gqa_routed_query_amd as gq

    d = dev()
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=d)
    res = gq.gqe_routed_prefill(q.to(d), k.to(d), v.to(d), lg.to(d), top_k, causal=causal,
                                out=out, workspace=workspace)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("B,h,g,T,d,top_k,ties,dt", [
    (2, 8, 2, 300, 128, 1, False, "bf16"),
    (2, 8, 2, 300, 128, 2, False, "bf16"),
    (1, 8, 2, 300, 128, 4, False, "bf16"),   # all experts kept: gated dense
    (2, 8, 2, 129, 128, 2, True, "bf16"),    # many tied logits
    (1, 12, 4, 100, 64, 3, True, "bf16"),
    (1, 32, 1, 80, 128, 5, False, "bf16"),   # one group of 32 experts
    (1, 4, 2, 40, 16, 1, False, "f32"),
    (1, 8, 2, 70, 32, 2, True, "f32"),
    (2, 8, 2, 90, 16, 1, False, "bf16"),    # bf16 below the MFMA tiles: fp32 arithmetic
    (1, 8, 4, 150, 32, 2, True, "bf16"),
])
def test_gqe_shapes(B, h, g, T, d, top_k, ties, dt):
    say(f"gqe B={B} h={h} g={g} T={T} d={d} k={top_k} ties={ties} {dt}")
    q, k, v, lg = gqe_inputs(B, h, g, T, d, dt, seed=400 + T + top_k, ties=ties)
    out, idx, gate = _run(q, k, v, lg, top_k)
    ref, ridx, rgate = oracle.gqe_ref(q, k, v, lg, top_k, causal=True)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert max_abs(out, ref) <= tol
    # a row is nonzero iff the router kept its head for its token
    assert torch.equal((out.cpu() != 0).any(-1), torch.from_numpy((ref != 0).any(-1)))


def test_gqe_top1_rows_equal_dense_rows():
    """With k = 1 the gate is 1 and a kept row is the dense GQA row, to the bit
    when both run the same arithmetic (no workspace: no key splits)."""
    import gqa_routed_query_amd as gq

    d = dev()
    say("gqe k=1 vs dense prefill")
    q, k, v, lg = gqe_inputs(1, 8, 2, 260, 128, "bf16", seed=61)
    out, idx, gate = _run(q, k, v, lg, 1, workspace=None)
    dense = gq.gqa_prefill(q.to(d), k.to(d), v.to(d), causal=True, out_dtype=torch.float32)
    assert bool((gate == 1.0).all())
    idx_c = idx.cpu()
    for t in range(0, 260, 7):
        for gam in range(2):
            i = int(idx_c[0, t, gam, 0])
            assert max_abs(out[0, i, t], dense[0, i, t]) <= 1e-6


@pytest.mark.parametrize("top_k", WORKLOADS["gqe"].top_k)
def test_gqe_headline_shape(top_k):
    """B=2, T=4096, h=32, g=8, d=128, logits N(0,1) (seed 5), drawn on the GPU,
    bf16 output with the workspace, the launch the benchmark times: all router
    indices bit-exact, gates within 1e-6, and every element of the output
    against the oracle (kept rows gate x dense row, every other row zero)."""
    w = WORKLOADS["gqe"]
    d = dev()
    say(f"gqe headline shape k={top_k}, full output")
    q, k, v, lg = gqe_inputs(w.B, w.h, w.g, w.T, w.d, "bf16", seed=w.seed, device=d)
    out, idx, gate = _run(q, k, v, lg, top_k, out_dtype=torch.bfloat16)
    ref, ridx, rgate = oracle.gqe_ref(q.cpu(), k.cpu(), v.cpu(), lg.cpu(), top_k, causal=True)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    oc = out.cpu()
    # structure: a row is nonzero iff its head was kept for its token
    assert torch.equal((oc != 0).any(-1), torch.from_numpy((ref != 0).any(-1)))
    err = max_abs(oc, ref)
    say(f"gqe headline k={top_k}: max|err| {err:.3e}")
    assert err <= TOL_BF16, err


def test_gqe_large_grid_ragged():
    """B=16, h=32, g=8, T=2000, k=2: the routed rows fill the large-grid
    configuration (1408 workgroups of 384 rows) and the last 32-key tile is
    partial. Indices bit-exact, zero rows exactly where heads were dropped, and
    sampled kept rows (the last tokens among them) equal gate x the oracle's row."""
    B, h, g, T, d, top_k = 16, 32, 8, 2000, 128, 2
    dv = dev()
    say(f"gqe large grid B={B} h={h} g={g} T={T} k={top_k}")
    q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=77, device=dv)
    out, idx, gate = _run(q, k, v, lg, top_k, out_dtype=torch.bfloat16)
    ridx, rgate = oracle.gqe_topk_ref(lg.cpu(), g, top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    kept = torch.zeros(B, T, h, dtype=torch.bool, device=dv)
    kept.scatter_(2, idx.view(B, T, -1).long(), True)
    assert torch.equal((out != 0).any(-1).permute(0, 2, 1), kept)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    worst = 0.0
    for t in sample_tokens(T, 12, seed=78, tile=32):
        for bb in (0, B - 1):
            for gam in (0, 3, g - 1):
                for j in range(top_k):
                    i = int(ridx[bb, t, gam, j])
                    ref = rgate[bb, t, gam, j] * oracle.gqa_ref_row(qc, kc, vc, bb, i, t)
                    worst = max(worst, float(np.abs(np64(out[bb, i, t]) - ref).max()))
    assert worst <= TOL_BF16, worst


@pytest.mark.parametrize("B,h,g,T,d,top_k,out_dt", [
    (2, 32, 8, 4096, 128, 1, torch.bfloat16),   # the GQE workload at k=1: one round of jobs
    (2, 8, 2, 300, 128, 2, torch.float32),
    (1, 12, 4, 333, 64, 3, torch.bfloat16),
    (1, 12, 4, 333, 64, 3, torch.float32),      # d = 64 with fp32 output
    (17, 20, 10, 700, 128, 1, torch.bfloat16),  # 170 problems, 3 row tiles: one split (the cap keeps the
                                                # 170 waiting second parts below the CU count)
])
def test_gqe_key_split_matches_unsplit(B, h, g, T, d, top_k, out_dt):
    """With a workspace, a causal grid of less than two blocks per CU splits the
    key range of its heaviest row tiles over two jobs and merges their partial
    results. The router outputs are identical, and the output equals the launch
    without a workspace within the bf16 tolerance (as it equals the oracle)."""
    import gqa_routed_query_amd as gq

    dv = dev()
    say(f"gqe key split B={B} h={h} g={g} T={T} d={d} k={top_k} out={out_dt}")
    assert gq.gqe_workspace_bytes(B, h, g, T, d, top_k) > 0
    q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=300 + T, device=dv)
    nan = float("nan")
    a, ia, ga = gq.gqe_routed_prefill(q, k, v, lg, top_k, out=torch.full(q.shape, nan, dtype=out_dt, device=dv),
                                      workspace=True)
    b, ib, gb = gq.gqe_routed_prefill(q, k, v, lg, top_k, out=torch.full(q.shape, nan, dtype=out_dt, device=dv),
                                      workspace=None)
    assert not a.isnan().any() and not b.isnan().any()
    torch.cuda.synchronize()
    assert torch.equal(ia, ib) and torch.equal(ga, gb)
    # The same rows are all zero (the heads the router did not keep). Single
    # elements of a kept row may sum to exactly 0.0 in one order of additions
    # and not in the other, so the check is per row.
    assert torch.equal((a == 0).all(-1), (b == 0).all(-1))
    # The probabilities are rounded to bf16 against each part's own reference
    # max, so the two launches differ at bf16 precision even with fp32 output.
    assert max_abs(a, b) <= TOL_BF16, max_abs(a, b)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ridx, rgate = ia.cpu().numpy(), ga.cpu().numpy()
    worst = 0.0
    for t in sample_tokens(T, 10, seed=T):
        for bb in {0, B - 1}:
            for gam in (0, g - 1):
                for j in range(top_k):
                    i = int(ridx[bb, t, gam, j])
                    ref = rgate[bb, t, gam, j] * oracle.gqa_ref_row(qc, kc, vc, bb, i, t)
                    worst = max(worst, float(np.abs(np64(a[bb, i, t]) - ref).max()))
    assert worst <= TOL_BF16, worst


@pytest.mark.parametrize("B,h,g,T,d,ks,seed", gqe_sweep_points(),
                         ids=lambda x: str(x) if not isinstance(x, tuple) else "k" + "".join(map(str, x)))
def test_gqe_sweep_point(B, h, g, T, d, ks, seed):
    """The GQE-vs-GQA sequence-length sweep (2k .. 64k tokens per sequence):
    for each k, all router indices bit-exact, gates within 1e-6, a row is
    nonzero iff its head was kept, and sampled kept rows equal gate x the
    oracle's dense row; the dense GQA output the sweep compares against is
    checked on sampled rows as well."""
    import gqa_routed_query_amd as gq

    dv = dev()
    say(f"gqe sweep B={B} h={h} g={g} T={T} k={ks}")
    q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=seed, device=dv)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    toks = sample_tokens(T, 6, seed=seed)
    for top_k in ks:
        out, idx, gate = _run(q, k, v, lg, top_k, out_dtype=torch.bfloat16)
        ridx, rgate = oracle.gqe_topk_ref(lg.cpu(), g, top_k)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert max_abs(gate, rgate) <= TOL_GATE
        kept = torch.zeros(B, T, h, dtype=torch.bool, device=dv)
        kept.scatter_(2, idx.view(B, T, -1).long(), True)
        assert torch.equal((out != 0).any(-1).permute(0, 2, 1), kept)
        worst = 0.0
        for t in toks:
            for bb in {0, B - 1}:
                for gam in (0, g - 1):
                    for j in range(top_k):
                        i = int(ridx[bb, t, gam, j])
                        ref = rgate[bb, t, gam, j] * oracle.gqa_ref_row(qc, kc, vc, bb, i, t)
                        worst = max(worst, float(np.abs(np64(out[bb, i, t]) - ref).max()))
        assert worst <= TOL_BF16, (top_k, worst)
        del out, idx, gate, kept
    dense = gq.gqa_prefill(q, k, v, causal=True, out_dtype=torch.bfloat16)
    worst = 0.0
    for t in toks:
        for i in (0, h // 2, h - 1):
            ref = oracle.gqa_ref_row(qc, kc, vc, B - 1, i, t)
            worst = max(worst, float(np.abs(np64(dense[B - 1, i, t]) - ref).max()))
    assert worst <= TOL_BF16, worst
    del q, k, v, lg, dense
    torch.cuda.empty_cache()


def test_gqe_split_wait_timeout_writes_nan(monkeypatch):
    """The second part of a key-split row tile waits for the first part's
    partial result with a bounded wait. With the bound set to zero polls
    (GQA_SPLIT_WAIT_POLLS=0) it gives up at once: every kernel still ends, the
    split tile's kept rows come out NaN (a loud failure, not a silent one) and
    every other row equals the normal launch. B=2, h=8, g=2, T=300, k=2: 600
    rows per (batch, group), two 384-row tiles, the second one split."""
    import gqa_routed_query_amd as gq

    B, h, g, T, d, top_k = 2, 8, 2, 300, 128, 2
    dv = dev()
    say("gqe split wait: timeout path")
    assert gq.gqe_workspace_bytes(B, h, g, T, d, top_k) > 0
    q, k, v, lg = gqe_inputs(B, h, g, T, d, "bf16", seed=901, device=dv)

    def call():
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dv)
        res = gq.gqe_routed_prefill(q, k, v, lg, top_k, out=out, workspace=True)
        torch.cuda.synchronize()
        return res

    ref, ridx, rgate = call()
    monkeypatch.setenv("GQA_SPLIT_WAIT_POLLS", "0")
    bad, bidx, bgate = call()
    monkeypatch.delenv("GQA_SPLIT_WAIT_POLLS")
    again, aidx, agate = call()
    assert torch.equal(ridx, bidx) and torch.equal(rgate, bgate)
    # the launch after the timed-out one is whole again, bit for bit
    assert torch.equal(again, ref) and torch.equal(aidx, ridx) and torch.equal(agate, rgate)
    assert not ref.isnan().any()
    # kept row rho = t*k + j of (b, group) lies in row tile rho // 384
    idx_c = ridx.cpu()
    in_split = torch.zeros(B, h, T, dtype=torch.bool)
    for b in range(B):
        for t in range(T):
            for gam in range(g):
                for j in range(top_k):
                    in_split[b, int(idx_c[b, t, gam, j]), t] = (t * top_k + j) // 384 == 1
    bad_c, ref_c = bad.cpu(), ref.cpu()
    nan_rows = bad_c.isnan().all(-1)
    assert torch.equal(nan_rows, in_split), int((nan_rows != in_split).sum())
    assert in_split.any()
    keep = ~in_split
    assert torch.equal(bad_c[keep], ref_c[keep])


def test_gqe_split_graph_replays():
    """The key-split launch captured in a HIP graph and replayed with new inputs
    each time: a replay reuses the captured launch's flag value, so each second
    part must wait for its own first part (the flag is cleared after use).
    Every replay equals an eager call on the same inputs, bit for bit, with
    eager work and synchronisation between the replays. GQE workload shape
    (B=2, T=4096, h=32, g=8, d=128), k=1."""
    import gqa_routed_query_amd as gq

    w = WORKLOADS["gqe"]
    dv = dev()
    say("gqe split launch in a graph, replays")
    assert gq.gqe_workspace_bytes(w.B, w.h, w.g, w.T, w.d, 1) > 0
    q, k, v, lg = gqe_inputs(w.B, w.h, w.g, w.T, w.d, "bf16", seed=950, device=dv)
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gq.gqe_routed_prefill(q, k, v, lg, 1, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="relaxed"):
        _, gidx, ggate = gq.gqe_routed_prefill(q, k, v, lg, 1, out=out)
    for rep in range(3):
        q2, k2, v2, lg2 = gqe_inputs(w.B, w.h, w.g, w.T, w.d, "bf16", seed=960 + rep, device=dv)
        q.copy_(q2), k.copy_(k2), v.copy_(v2), lg.copy_(lg2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dv)
        e_out, e_idx, e_gate = gq.gqe_routed_prefill(q, k, v, lg, 1, out=e_out)
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        assert torch.equal(gidx, e_idx) and torch.equal(ggate, e_gate)
        assert torch.equal(out, e_out)
