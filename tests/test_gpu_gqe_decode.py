"""GQE routed decode on the GPU against the float64 oracle: router indices
bit-exact, gates within 1e-6, outputs within the bf16 tolerance, rows of heads
the router did not keep (and of empty sequences) exactly zero."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, TOL_GATE, dev, max_abs, say
from workloads import WORKLOADS, decode_inputs, router_logits

pytestmark = pytest.mark.gpu


def _run(q, kc, vc, lens, lg, top_k, out_dtype=torch.float32, workspace=None):
    """The call into an output filled with NaN beforehand, so any row the
    launch leaves unwritten (kept or zero) fails the comparison."""
    import gqa_routed_query_amd as gq

    d = dev()
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=d)
    res = gq.gqe_routed_decode(q.to(d), kc.to(d), vc.to(d), lens.to(d), lg.to(d), top_k,
                               out=out, workspace=workspace)
    torch.cuda.synchronize()
    return res


def _check(out, idx, gate, q, kc, vc, lens, lg, top_k, tol=TOL_BF16):
    ref, ridx, rgate = oracle.gqe_decode_ref(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu(), lg.cpu(), top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert max_abs(gate, rgate) <= TOL_GATE
    assert torch.isfinite(out).all()
    assert max_abs(out, ref) <= tol
    # a row is nonzero iff its head was kept and its sequence has cached keys
    assert torch.equal((out.cpu() != 0).any(-1), torch.from_numpy((ref != 0).any(-1)))


@pytest.mark.parametrize("B,h,g,T_max,d,top_k,ties,out_dt", [
    (5, 8, 2, 1000, 128, 1, False, torch.float32),
    (5, 8, 2, 1000, 128, 2, True, torch.bfloat16),
    (3, 32, 1, 700, 128, 4, False, torch.float32),    # 32 experts in one group
    (3, 16, 16, 300, 128, 1, False, torch.float32),   # one expert per group: k = h/g = 1
    (4, 16, 2, 400, 64, 3, True, torch.float32),      # d = 64
    (2, 64, 1, 130, 128, 5, False, torch.float32),    # 64 heads per group
    (3, 8, 2, 500, 128, 4, False, torch.float32),     # every expert kept
    (2, 32, 1, 300, 128, 20, True, torch.float32),    # 20 of 32 kept: the 32-column kernel
    (3, 16, 4, 500, 32, 2, False, torch.float32),     # d = 32
    (2, 32, 1, 400, 32, 9, True, torch.bfloat16),     # d = 32, 9 of 32 kept
    (3, 16, 4, 500, 16, 2, False, torch.float32),     # d = 16
    (2, 32, 1, 300, 16, 5, True, torch.bfloat16),     # d = 16, 5 of 32 kept
])
def test_gqe_decode_shapes_poisoned_padding(B, h, g, T_max, d, top_k, ties, out_dt):
    say(f"gqe decode B={B} h={h} g={g} T_max={T_max} d={d} k={top_k} ties={ties} out={out_dt}")
    q, kc, vc, lens = decode_inputs(B, h, g, T_max, d, (1, T_max), seed=700 + h + top_k,
                                    poison_padding=True)
    lens[0] = T_max
    lens[-1] = 1
    kc[0] = kc[0].nan_to_num(0.0)
    vc[0] = vc[0].nan_to_num(0.0)
    lg = router_logits(B, 1, h, seed=701 + h, ties=ties)[:, 0].contiguous()
    out, idx, gate = _run(q, kc, vc, lens, lg, top_k, out_dt)
    _check(out, idx, gate, q, kc, vc, lens, lg, top_k)


@pytest.mark.parametrize("B,h,g,T_max,d,top_k,ties,out_dt", [
    (5, 8, 2, 1000, 128, 1, False, torch.float32),
    (5, 8, 2, 1000, 128, 2, True, torch.bfloat16),
    (2, 64, 1, 130, 128, 40, False, torch.float32),   # 40 of 64 kept: three 16-row blocks
    (4, 16, 2, 400, 64, 3, True, torch.float32),      # d = 64
    (3, 16, 4, 500, 16, 2, False, torch.float32),     # d = 16
])
def test_gqe_decode_fp32_cache(B, h, g, T_max, d, top_k, ties, out_dt):
    """fp32 q and caches through the routed decode: fp32 accuracy."""
    say(f"gqe decode fp32 cache B={B} h={h} g={g} T_max={T_max} d={d} k={top_k} out={out_dt}")
    q, kc, vc, lens = decode_inputs(B, h, g, T_max, d, (1, T_max), dtype="f32", seed=720 + h + top_k,
                                    poison_padding=True)
    lens[0] = T_max
    lens[-1] = 1
    kc[0] = kc[0].nan_to_num(0.0)
    vc[0] = vc[0].nan_to_num(0.0)
    lg = router_logits(B, 1, h, seed=721 + h, ties=ties)[:, 0].contiguous()
    out, idx, gate = _run(q, kc, vc, lens, lg, top_k, out_dt)
    _check(out, idx, gate, q, kc, vc, lens, lg, top_k,
           tol=TOL_F32 if out_dt == torch.float32 else TOL_BF16)


def test_gqe_decode_edge_lengths():
    """Empty caches give zero rows for every head; lengths around the 32-key
    sub-block and 128-key step boundaries."""
    lens_list = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 0, 512]
    B = len(lens_list)
    say("gqe decode edge lengths")
    q, kc, vc, _ = decode_inputs(B, 8, 2, 512, 128, (1, 1), seed=71, poison_padding=False)
    lens = torch.tensor(lens_list, dtype=torch.int32)
    for b, n in enumerate(lens_list):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    lg = router_logits(B, 1, 8, seed=72)[:, 0].contiguous()
    for top_k in (1, 2):
        out, idx, gate = _run(q, kc, vc, lens, lg, top_k)
        assert float(out[0].abs().max()) == 0.0 and float(out[10].abs().max()) == 0.0
        _check(out, idx, gate, q, kc, vc, lens, lg, top_k)


def test_gqe_decode_share_invariance(monkeypatch):
    """The result does not depend on how the key range is shared out over
    workgroups (one, a few, many, the default)."""
    q, kc, vc, lens = decode_inputs(6, 16, 4, 3000, 128, (1, 3000), seed=73)
    lg = router_logits(6, 1, 16, seed=74)[:, 0].contiguous()
    outs = []
    for units in ("1", "3", "200", None):
        say(f"gqe decode units={units}")
        if units:
            monkeypatch.setenv("GQA_DECODE_UNITS", units)
        else:
            monkeypatch.delenv("GQA_DECODE_UNITS", raising=False)
        out, idx, gate = _run(q, kc, vc, lens, lg, 2)
        _check(out, idx, gate, q, kc, vc, lens, lg, 2)
        outs.append(out)
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 1e-3


def test_gqe_decode_kept_rows_equal_plain_decode():
    """k = 1: the gate is 1 and a kept row is the plain GQA decode row of its
    head (both on the GPU); the workspace is reused between the two calls."""
    import gqa_routed_query_amd as gq

    d = dev()
    say("gqe decode vs gqa decode")
    q, kc, vc, lens = decode_inputs(8, 32, 8, 2048, 128, (1, 2048), seed=75, device=d)
    lg = router_logits(8, 1, 32, seed=76, device=d)[:, 0].contiguous()
    ws = torch.empty(gq.gqa_decode_workspace_bytes(8, 32, 8, 2048, 128), dtype=torch.uint8, device=d)
    plain = gq.gqa_decode(q, kc, vc, lens, out_dtype=torch.float32, workspace=ws)
    out, idx, gate = gq.gqe_routed_decode(q, kc, vc, lens, lg, 1, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert bool((gate == 1.0).all())
    for b in range(8):
        for gam in range(8):
            i = int(idx[b, gam, 0])
            assert max_abs(out[b, i], plain[b, i]) <= 1e-3


@pytest.mark.parametrize("top_k", (1, 2))
def test_gqe_decode_headline_shape(top_k):
    """The decode workload (B=64, h=32, g=8, d=128, cache lengths uniform in
    [1024, 8192], seed 3) with router logits [64, 32] ~ N(0,1): all indices
    bit-exact and gates checked, every unselected row zero, every sequence in
    full against the oracle (one at a time, its valid cache positions only)."""
    w = WORKLOADS["decode"]
    d = dev()
    say(f"gqe decode headline shape k={top_k}")
    q, kc, vc, lens = decode_inputs(w.B, w.h, w.g, w.T, w.d, w.lens, seed=w.seed, device=d)
    lg = router_logits(w.B, 1, w.h, seed=w.seed + 100, device=d)[:, 0].contiguous()
    out, idx, gate = _run(q, kc, vc, lens, lg, top_k, torch.bfloat16)
    ridx, rgate = oracle.gqe_topk_ref(lg.cpu().view(w.B, 1, w.h), w.g, top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx[:, 0])
    assert max_abs(gate, rgate[:, 0]) <= TOL_GATE
    kept = torch.zeros(w.B, w.h, dtype=torch.bool, device=d)
    kept.scatter_(1, idx.view(w.B, -1).long(), True)
    assert torch.equal((out != 0).any(-1), kept)
    lens_c = lens.cpu()
    oc = out.cpu()
    for b in range(w.B):
        n = int(lens_c[b])
        ref, _, _ = oracle.gqe_decode_ref(q[b:b + 1].cpu(), kc[b:b + 1, :, :n].cpu(),
                                          vc[b:b + 1, :, :n].cpu(), np.array([n]),
                                          lg[b:b + 1].cpu(), top_k)
        assert max_abs(oc[b:b + 1], ref) <= TOL_BF16, b
