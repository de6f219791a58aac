"""The fused router projection + top-k on the GPU. Logits are checked against
the float64 oracle within the worst-case float32 dot-product bound; the top-k
decision is checked bit-exact against the oracle's selection applied to the
kernel's own float32 logits (both sides decide in the kernel's precision), and
the gates within 1e-6."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_GATE, dev, max_abs, np64, say
from workloads import ROUTER_D_MODEL, WORKLOADS, gqe_inputs, router_inputs

pytestmark = pytest.mark.gpu


def _check(x, w, g, top_k):
    import gqa_routed_query_amd as gq

    d = dev()
    logits, idx, gate = gq.gqe_router(x.to(d), w.to(d), g, top_k)
    _, idx2, gate2 = gq.gqe_router(x.to(d), w.to(d), g, top_k, return_logits=False)
    torch.cuda.synchronize()
    ref, bound, _, _ = oracle.gqe_router_ref(x.cpu(), w.cpu(), g, top_k)
    err = np.abs(np64(logits) - ref)
    assert np.all(err <= bound), float((err - bound).max())
    n, h = ref.shape
    ridx, rgate = oracle.gqe_topk_ref(logits.cpu().view(1, n, h), g, top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx[0])
    assert max_abs(gate, rgate[0]) <= TOL_GATE
    assert torch.equal(idx, idx2) and torch.equal(gate, gate2)
    _check_against_f64_selection(ref, bound, idx.cpu().numpy().reshape(n, g, top_k), g, top_k)
    return logits, idx, gate


def _check_against_f64_selection(ref, bound, idx, g, top_k, min_frac=0.8):
    """Independent of the kernel's logits: where the float64 logits fix the
    ranked top-k of a group beyond both error bounds (each kept expert's
    logit minus its bound exceeds every lower-ranked expert's logit plus its
    bound), every float32 evaluation within the bound ranks them the same, so
    the kernel's indices must equal the oracle's selection on the float64
    logits. Most groups are decided that way; the rest are left to the
    same-precision check above."""
    n, h = ref.shape
    r = h // g
    ridx, _ = oracle.gqe_topk_ref(ref.reshape(1, n, h), g, top_k)
    sel = ridx[0] - (np.arange(g) * r)[None, :, None]              # [n, g, k] local experts
    lo = (ref - bound).reshape(n, g, r)
    hi = (ref + bound).reshape(n, g, r)
    beats = lo[..., :, None] > hi[..., None, :]                      # [n, g, r, r]
    sure = np.ones((n, g), dtype=bool)
    taken = np.zeros((n, g, r), dtype=bool)
    ii, gg = np.meshgrid(np.arange(n), np.arange(g), indexing="ij")
    for j in range(top_k):
        a = sel[..., j]
        taken[ii, gg, a] = True
        row = beats[ii, gg, a]                                       # [n, g, r]: a vs each expert
        sure &= np.all(row | taken, axis=-1)
    assert sure.mean() >= min_frac, sure.mean()
    assert np.array_equal(idx[sure], ridx[0][sure])


@pytest.mark.parametrize("n,dm,h,g,k", [
    (100, 128, 8, 2, 1),
    (257, 256, 16, 8, 1),     # ragged token tile, the pages' 16 heads over 8 groups
    (64, 1024, 32, 8, 2),
    (33, 4096, 32, 8, 1),
    (70, 512, 64, 8, 3),      # two head blocks of 32
    (50, 384, 12, 4, 2),      # h not a multiple of 32
    (31, 128, 64, 1, 5),      # one group of 64 experts
])
def test_router_shapes(n, dm, h, g, k):
    say(f"router n={n} d_model={dm} h={h} g={g} k={k}")
    x, w = router_inputs(n, dm, h, seed=800 + n)
    _check(x, w, g, k)


def test_router_feeds_routed_prefill():
    """The router's logits drive gqe_routed_prefill to the same kept heads and
    gates ([B, T, d_model] tokens of one batch)."""
    import gqa_routed_query_amd as gq

    d = dev()
    B, T, h, g, hd = 2, 96, 16, 4, 64
    say("router -> routed prefill")
    x, w = router_inputs(B * T, h * hd, h, seed=810, device=d)
    logits, idx, gate = gq.gqe_router(x.view(B, T, h * hd), w, g, 2)
    q, k, v, _ = gqe_inputs(B, h, g, T, hd, "bf16", seed=811, device=d)
    out, idx_p, gate_p = gq.gqe_routed_prefill(q, k, v, logits, 2)
    torch.cuda.synchronize()
    assert idx.shape == (B, T, g, 2)
    assert torch.equal(idx, idx_p) and torch.equal(gate, gate_p)


@pytest.mark.parametrize("top_k", WORKLOADS["gqe"].top_k)
def test_router_headline_shape(top_k):
    """The GQE workload's 8192 tokens (B=2, T=4096) from d_model = 4096 to
    h = 32 heads in 8 groups: every logit within its bound, every kept index
    bit-exact, every gate checked."""
    w8 = WORKLOADS["gqe"]
    d = dev()
    say(f"router headline k={top_k}")
    x, w = router_inputs(w8.B * w8.T, ROUTER_D_MODEL, w8.h, seed=w8.seed + 200, device=d)
    _check(x, w, w8.g, top_k)
