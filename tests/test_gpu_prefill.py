"""GQA prefill on the GPU against the float64 oracle, element by element."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, dev, max_abs, np64, sample_tokens, say
from workloads import WORKLOADS, prefill_inputs

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal=True, out_dtype=None, scale=None):
    """The call into an output filled with NaN beforehand, so any element the
    launch leaves unwritten fails the comparison."""
    import gqa_routed_query_amd as gq

    d = dev()
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=d)
    out = gq.gqa_prefill(q.to(d), k.to(d), v.to(d), causal=causal, out=out, scale=scale)
    torch.cuda.synchronize()
    return out


def test_tiny_fp32_gqa_mha_mqa():
    """B=1, h=4, T=16, d=16 fp32, causal, at g=2 (GQA), g=4 (MHA), g=1 (MQA):
    one draw, the same q and the first g KV heads."""
    w = WORKLOADS["tiny_f32"]
    q, k4, v4 = prefill_inputs(w.B, w.h, 4, w.T, w.d, "f32", seed=w.seed)
    for g in w.g_sweep:
        k, v = k4[:, :g].contiguous(), v4[:, :g].contiguous()
        say(f"tiny fp32 g={g}")
        out = _run(q, k, v, causal=True)
        err = max_abs(out, oracle.gqa_ref(q, k, v, causal=True))
        assert err <= TOL_F32, (g, err)


@pytest.mark.parametrize("B,h,g,T,d,causal", [
    (1, 4, 2, 1, 16, True),        # T = 1: output is V
    (2, 8, 2, 77, 16, True),
    (1, 6, 3, 130, 32, False),
    (2, 4, 1, 97, 64, True),       # MQA
    (1, 4, 4, 300, 128, True),     # MHA, several tiles, ragged tail
    (1, 8, 2, 259, 128, False),
])
def test_fp32_shapes(B, h, g, T, d, causal):
    say(f"fp32 B={B} h={h} g={g} T={T} d={d} causal={causal}")
    q, k, v = prefill_inputs(B, h, g, T, d, "f32", seed=100 + T)
    out = _run(q, k, v, causal=causal)
    err = max_abs(out, oracle.gqa_ref(q, k, v, causal=causal))
    assert err <= TOL_F32, err


@pytest.mark.parametrize("B,h,g,T,d,causal,out_dt", [
    (1, 4, 2, 1, 128, True, torch.float32),        # T = 1
    (2, 8, 2, 300, 128, True, torch.float32),      # several row and key tiles, ragged tail
    (2, 8, 2, 300, 128, True, torch.bfloat16),
    (1, 8, 2, 300, 128, False, torch.float32),
    (1, 4, 4, 130, 128, True, torch.float32),      # MHA
    (1, 8, 1, 257, 128, True, torch.float32),      # MQA
    (1, 32, 8, 520, 128, True, torch.bfloat16),    # the headline head layout
    (2, 6, 3, 190, 64, True, torch.float32),       # d = 64
    (1, 12, 4, 333, 64, False, torch.bfloat16),
    (1, 2, 1, 64, 128, True, torch.float32),       # exactly one tile
    (1, 4, 2, 65, 128, True, torch.float32),       # one tile plus one key
])
def test_bf16_shapes(B, h, g, T, d, causal, out_dt):
    say(f"bf16 B={B} h={h} g={g} T={T} d={d} causal={causal} out={out_dt}")
    q, k, v = prefill_inputs(B, h, g, T, d, "bf16", seed=200 + T + h)
    out = _run(q, k, v, causal=causal, out_dtype=out_dt)
    err = max_abs(out, oracle.gqa_ref(q, k, v, causal=causal))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("B,h,g,T,d,causal,out_dt", [
    (2, 8, 2, 77, 16, True, torch.float32),
    (1, 6, 3, 130, 32, False, torch.float32),
    (1, 4, 1, 300, 32, True, torch.bfloat16),      # MQA, several key tiles, ragged tail
    (1, 4, 4, 1, 16, True, torch.float32),         # T = 1
])
def test_bf16_small_head_dims(B, h, g, T, d, causal, out_dt):
    """bf16 inputs at d 16 and 32 (below the MFMA kernel's tiles) run in fp32
    arithmetic on the exact upcast inputs: fp32 tolerance for fp32 output."""
    say(f"bf16 small d B={B} h={h} g={g} T={T} d={d} causal={causal} out={out_dt}")
    q, k, v = prefill_inputs(B, h, g, T, d, "bf16", seed=250 + T + d)
    out = _run(q, k, v, causal=causal, out_dtype=out_dt)
    err = max_abs(out, oracle.gqa_ref(q, k, v, causal=causal))
    assert err <= (TOL_F32 if out_dt == torch.float32 else TOL_BF16), err


def test_bf16_explicit_scale():
    say("bf16 explicit scale 0.3")
    q, k, v = prefill_inputs(1, 8, 2, 150, 128, "bf16", seed=7)
    out = _run(q, k, v, causal=True, out_dtype=torch.float32, scale=0.03)
    err = max_abs(out, oracle.gqa_ref(q, k, v, causal=True, scale=0.03))
    assert err <= TOL_BF16, err


def test_bf16_headline_shape_full():
    """B=4, h=32, g=8, T=2048, d=128, causal, inputs drawn on the GPU (seed 2)
    and bf16 output, the launch the benchmark times: every element of the
    output against the oracle, one batch element at a time."""
    w = WORKLOADS["prefill"]
    d = dev()
    say("prefill headline shape, full output")
    q, k, v = prefill_inputs(w.B, w.h, w.g, w.T, w.d, "bf16", seed=w.seed, device=d)
    out = _run(q, k, v, causal=True)
    assert out.dtype == torch.bfloat16
    qc, kc, vc, oc = q.cpu(), k.cpu(), v.cpu(), out.cpu()
    worst = 0.0
    for b in range(w.B):
        ref = oracle.gqa_ref(qc[b:b + 1], kc[b:b + 1], vc[b:b + 1], causal=True)
        worst = max(worst, max_abs(oc[b:b + 1], ref))
        say(f"prefill headline b={b}: max|err| so far {worst:.3e}")
    assert worst <= TOL_BF16, worst


def _large_grid(B, h, g, T):
    """True when the launch takes the 12-wave, 32-key-tile configuration (at
    least 24 waves of 384-row work per CU)."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    return B * g * -(-(T * (h // g)) // 384) * 12 >= 24 * n_cu


@pytest.mark.parametrize("T,d,causal,out_dt", [
    (2000, 128, True, torch.bfloat16),   # the last key tile holds 16 keys
    (2001, 128, True, torch.float32),    # one key in the last tile; fp32 out (two staging passes)
    (1999, 64, False, torch.bfloat16),   # d = 64, no causal mask, only the tail
])
def test_bf16_large_grid_ragged(T, d, causal, out_dt):
    """B=8, h=32, g=8: enough row tiles for the large-grid configuration, with T
    not a multiple of its 32-key tile, so the last K/V tile is partial (its keys
    past T are clamped when staged and masked). The last tokens and sampled
    rows elsewhere, against the oracle."""
    B, h, g = 8, 32, 8
    assert _large_grid(B, h, g, T)
    say(f"bf16 large grid B={B} h={h} g={g} T={T} d={d} causal={causal} out={out_dt}")
    q, k, v = prefill_inputs(B, h, g, T, d, "bf16", seed=300 + T + d, device=dev())
    out = _run(q, k, v, causal=causal, out_dtype=out_dt)
    qc, kc, vc, oc = q.cpu(), k.cpu(), v.cpu(), out.cpu()
    worst = 0.0
    for t in sample_tokens(T, 24, seed=T, tile=32):
        for b in (0, B - 1):
            for i in (0, 13, h - 1):
                ref = oracle.gqa_ref_row(qc, kc, vc, b, i, t, causal=causal)
                worst = max(worst, float(np.abs(np64(oc[b, i, t]) - ref).max()))
    assert worst <= TOL_BF16, worst


def test_bf16_headline_shape_unit_values():
    """At the headline shape with V = 1 everywhere every output is 1 (the
    weights of a row sum to one), whatever q and k are."""
    w = WORKLOADS["prefill"]
    d = dev()
    say("prefill headline shape, V = 1")
    q, k, _ = prefill_inputs(w.B, w.h, w.g, w.T, w.d, "bf16", seed=w.seed, device=d)
    v = torch.ones_like(k)
    out = _run(q, k, v, causal=True, out_dtype=torch.float32)
    assert float((out - 1.0).abs().max()) <= TOL_BF16


def test_bf16_deterministic():
    say("bf16 determinism")
    q, k, v = prefill_inputs(2, 8, 2, 300, 128, "bf16", seed=9)
    a = _run(q, k, v, causal=True)
    b = _run(q, k, v, causal=True)
    assert torch.equal(a, b)


def test_empty_problem():
    import gqa_routed_query_amd as gq

    d = dev()
    say("empty T = 0")
    q = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device=d)
    k = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=d)
    out = gq.gqa_prefill(q, k, k, causal=True)
    assert out.shape == q.shape
