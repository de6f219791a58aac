"""GQA decode over a KV cache on the GPU against the float64 oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, dev, max_abs, np64, say
from workloads import WORKLOADS, decode_inputs

pytestmark = pytest.mark.gpu


def _run(q, kc, vc, lens, out_dtype=torch.float32):
    """The call into an output filled with NaN beforehand, so any element the
    launch leaves unwritten fails the comparison."""
    import gqa_routed_query_amd as gq

    d = dev()
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=d)
    out = gq.gqa_decode(q.to(d), kc.to(d), vc.to(d), lens.to(d), out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,h,g,T_max,d,out_dt", [
    (5, 8, 2, 1000, 128, torch.float32),
    (5, 8, 2, 1000, 128, torch.bfloat16),
    (3, 32, 1, 700, 128, torch.float32),     # MQA: 32 heads on one KV head
    (3, 16, 16, 300, 128, torch.float32),    # MHA
    (4, 16, 2, 400, 64, torch.float32),      # d = 64
    (2, 64, 1, 130, 128, torch.float32),     # 64 heads per group
    (3, 24, 1, 500, 128, torch.float32),     # 17-32 heads per group: the 32-column kernel, 8 idle columns
    (2, 32, 1, 400, 64, torch.bfloat16),     # 32 heads per group at d = 64
    (4, 16, 4, 600, 32, torch.float32),      # d = 32, 4 heads per group
    (3, 32, 1, 500, 32, torch.bfloat16),     # d = 32, 32 heads per group (the 32-column kernel)
    (2, 48, 1, 300, 32, torch.float32),      # d = 32, 48 heads per group
    (4, 16, 4, 600, 16, torch.float32),      # d = 16: half the score MFMA's reduction zeroed
    (3, 32, 1, 500, 16, torch.bfloat16),     # d = 16, 32 heads per group: two 16-head blocks
    (2, 48, 1, 300, 16, torch.float32),      # d = 16, 48 heads per group
])
def test_decode_shapes_poisoned_padding(B, h, g, T_max, d, out_dt):
    say(f"decode B={B} h={h} g={g} T_max={T_max} d={d} out={out_dt}")
    q, kc, vc, lens = decode_inputs(B, h, g, T_max, d, (1, T_max), seed=300 + h,
                                    poison_padding=True)
    lens[0] = T_max
    lens[-1] = 1
    kc[0] = kc[0].nan_to_num(0.0)  # row 0 is full: no padding there
    vc[0] = vc[0].nan_to_num(0.0)
    out = _run(q, kc, vc, lens, out_dt)
    assert torch.isfinite(out).all()
    err = max_abs(out, oracle.gqa_decode_ref(q, kc, vc, lens))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("B,h,g,T_max,d,out_dt", [
    (5, 8, 2, 1000, 128, torch.float32),     # 4 heads per group
    (5, 8, 2, 1000, 128, torch.bfloat16),
    (3, 32, 1, 700, 128, torch.float32),     # MQA: two 16-head blocks of the grid
    (2, 64, 1, 130, 128, torch.float32),     # 64 heads per group: four blocks
    (3, 16, 16, 300, 128, torch.float32),    # MHA
    (4, 16, 2, 400, 64, torch.float32),      # d = 64
    (3, 24, 1, 500, 32, torch.float32),      # d = 32, 24 heads: the second block half empty
    (4, 16, 4, 600, 16, torch.float32),      # d = 16
    (2, 48, 1, 300, 16, torch.bfloat16),     # d = 16, 48 heads per group
])
def test_decode_fp32_cache_poisoned_padding(B, h, g, T_max, d, out_dt):
    """fp32 q and caches: the fp32-operand kernel, at fp32 accuracy."""
    say(f"decode fp32 cache B={B} h={h} g={g} T_max={T_max} d={d} out={out_dt}")
    q, kc, vc, lens = decode_inputs(B, h, g, T_max, d, (1, T_max), dtype="f32", seed=310 + h,
                                    poison_padding=True)
    lens[0] = T_max
    lens[-1] = 1
    kc[0] = kc[0].nan_to_num(0.0)
    vc[0] = vc[0].nan_to_num(0.0)
    out = _run(q, kc, vc, lens, out_dt)
    assert torch.isfinite(out).all()
    err = max_abs(out, oracle.gqa_decode_ref(q, kc, vc, lens))
    assert err <= (TOL_F32 if out_dt == torch.float32 else TOL_BF16), err


def test_decode_fp32_cache_edge_lengths_and_shares(monkeypatch):
    """fp32 caches at lengths around the 16-key sub-block and 64-key step
    boundaries (and an empty sequence), on the default grid and on grids that
    cut the streams into pieces of different lengths."""
    lens_list = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 511, 512]
    B = len(lens_list)
    q, kc, vc, _ = decode_inputs(B, 8, 2, 512, 128, (1, 1), dtype="f32", seed=33)
    lens = torch.tensor(lens_list, dtype=torch.int32)
    for b, n in enumerate(lens_list):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    ref = oracle.gqa_decode_ref(q, kc, vc, lens)
    for units in (None, "1", "7", "300"):
        say(f"decode fp32 edge lengths, units={units}")
        if units:
            monkeypatch.setenv("GQA_DECODE_UNITS", units)
        else:
            monkeypatch.delenv("GQA_DECODE_UNITS", raising=False)
        out = _run(q, kc, vc, lens)
        assert torch.isfinite(out).all()
        assert float(out[0].abs().max()) == 0.0
        assert max_abs(out, ref) <= TOL_F32


def test_decode_edge_lengths():
    """Lengths around the 32-key sub-block and 128-key chunk boundaries, plus
    an empty sequence (zero row)."""
    lens_list = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 511, 512]
    B = len(lens_list)
    say("decode edge lengths")
    q, kc, vc, _ = decode_inputs(B, 8, 2, 512, 128, (1, 1), seed=31, poison_padding=False)
    lens = torch.tensor(lens_list, dtype=torch.int32)
    for b, n in enumerate(lens_list):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    out = _run(q, kc, vc, lens)
    ref = oracle.gqa_decode_ref(q, kc, vc, lens)
    assert torch.isfinite(out).all()
    assert float(out[0].abs().max()) == 0.0
    assert max_abs(out, ref) <= TOL_BF16


def test_decode_empty_cache():
    """T_max = 0: no cached positions at all, every output row is zero, with the
    workspace size the library reports for that shape."""
    import gqa_routed_query_amd as gq

    d = dev()
    say("decode T_max = 0")
    q = torch.randn(3, 8, 128, device=d).to(torch.bfloat16)
    kc = torch.empty(3, 2, 0, 128, dtype=torch.bfloat16, device=d)
    lens = torch.zeros(3, dtype=torch.int32, device=d)
    ws = torch.empty(gq.gqa_decode_workspace_bytes(3, 8, 2, 0, 128), dtype=torch.uint8, device=d)
    out = gq.gqa_decode(q, kc, kc, lens, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0


def test_decode_split_invariance(monkeypatch):
    """The result does not depend on how the key range is shared out over
    waves (up to fp32 rounding): one wave (every stream whole), a few waves
    (streams cut into long pieces), many waves (short pieces, several per
    stream) and the default grid."""
    q, kc, vc, lens = decode_inputs(6, 16, 4, 3000, 128, (1, 3000), seed=41)
    lens[2] = 0
    outs = []
    for units in ("1", "3", "64", "1000", None):
        say(f"decode units={units}")
        if units:
            monkeypatch.setenv("GQA_DECODE_UNITS", units)
        else:
            monkeypatch.delenv("GQA_DECODE_UNITS", raising=False)
        outs.append(_run(q, kc, vc, lens))
    ref = oracle.gqa_decode_ref(q, kc, vc, lens)
    for o in outs:
        assert float(o[2].abs().max()) == 0.0
        assert max_abs(o, outs[0]) <= 1e-3
        assert max_abs(o, ref) <= TOL_BF16


def test_decode_one_long_stream_many_pieces(monkeypatch):
    """One sequence of 40,000 keys on one KV head: with the default grid every
    share holds 256 keys, so the stream is cut into 157 pieces and the merge
    runs three rounds of 64 pieces; with 4 workgroups, 4 pieces."""
    q, kc, vc, lens = decode_inputs(1, 8, 1, 40000, 128, (40000, 40000), seed=45)
    ref = oracle.gqa_decode_ref(q, kc, vc, lens)
    for units in (None, "4"):
        if units:
            monkeypatch.setenv("GQA_DECODE_UNITS", units)
        else:
            monkeypatch.delenv("GQA_DECODE_UNITS", raising=False)
        say(f"decode one long stream, units={units}")
        out = _run(q, kc, vc, lens)
        assert max_abs(out, ref) <= TOL_BF16


def test_decode_repeated_calls_reuse_workspace():
    """Back-to-back calls with different lengths on one workspace give the
    same result as fresh calls: partial slots are rewritten each call and
    need no clearing."""
    import gqa_routed_query_amd as gq

    d = dev()
    q, kc, vc, lens = decode_inputs(8, 16, 4, 2048, 128, (1, 2048), seed=43)
    q, kc, vc = q.to(d), kc.to(d), vc.to(d)
    ws = torch.full((gq.gqa_decode_workspace_bytes(8, 16, 4, 2048, 128),), 0x7f, dtype=torch.uint8,
                    device=d)
    say("decode workspace reuse")
    for seed_lens in ([2048] * 8, [5, 2048, 0, 700, 33, 1500, 64, 1]):
        ln = torch.tensor(seed_lens, dtype=torch.int32)
        out = gq.gqa_decode(q, kc, vc, ln.to(d), out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert max_abs(out, oracle.gqa_decode_ref(q.cpu(), kc.cpu(), vc.cpu(), ln)) <= TOL_BF16


def test_decode_matches_prefill_last_row():
    """Decoding token t over a cache of t+1 positions equals row t of causal
    prefill (both on the GPU, both checked against the oracle)."""
    import gqa_routed_query_amd as gq
    from workloads import prefill_inputs

    d = dev()
    say("decode vs prefill row")
    q, k, v = prefill_inputs(1, 8, 2, 200, 128, "bf16", seed=51)
    pre = gq.gqa_prefill(q.to(d), k.to(d), v.to(d), causal=True, out_dtype=torch.float32)
    ts = [0, 63, 64, 199]
    qd = torch.stack([q[0, :, t] for t in ts])
    kc = k.expand(len(ts), -1, -1, -1).contiguous()
    vc = v.expand(len(ts), -1, -1, -1).contiguous()
    lens = torch.tensor([t + 1 for t in ts], dtype=torch.int32)
    out = _run(qd, kc, vc, lens)
    for j, t in enumerate(ts):
        assert max_abs(out[j], pre[0, :, t]) <= 5e-3


def test_decode_headline_shape():
    """B=64, h=32, g=8, d=128, cache lengths uniform in [1024, 8192], cache
    drawn on the GPU (seed 3), bf16 output as the benchmark launches it: every
    sequence against the oracle, one at a time (its valid cache positions only)."""
    w = WORKLOADS["decode"]
    d = dev()
    say("decode headline shape, all sequences")
    q, kc, vc, lens = decode_inputs(w.B, w.h, w.g, w.T, w.d, w.lens, seed=w.seed, device=d)
    out = _run(q, kc, vc, lens, out_dtype=torch.bfloat16)
    lens_c = lens.cpu()
    oc = out.cpu()
    worst = 0.0
    for b in range(w.B):
        n = int(lens_c[b])
        ref = oracle.gqa_decode_ref(q[b:b + 1].cpu(), kc[b:b + 1, :, :n].cpu(),
                                    vc[b:b + 1, :, :n].cpu(), np.array([n]))
        worst = max(worst, max_abs(oc[b:b + 1], ref))
    assert worst <= TOL_BF16, worst


@pytest.mark.parametrize("g", WORKLOADS["decode_sweep"].g_sweep)
def test_decode_group_sweep(g):
    """B=32, h=32, T=16384, d=128 at g in {1, 4, 8, 32}, bf16 output as the
    benchmark launches it: all 32 sequences against the oracle, streamed one
    sequence at a time."""
    w = WORKLOADS["decode_sweep"]
    d = dev()
    say(f"decode sweep g={g}, all sequences")
    q, kc, vc, lens = decode_inputs(w.B, w.h, g, w.T, w.d, w.lens, seed=w.seed + g, device=d)
    out = _run(q, kc, vc, lens, out_dtype=torch.bfloat16)
    oc = out.cpu()
    worst = 0.0
    for b in range(w.B):
        ref = oracle.gqa_decode_ref(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                    np.array([w.T]))
        worst = max(worst, max_abs(oc[b:b + 1], ref))
    say(f"decode sweep g={g}: max|err| {worst:.3e}")
    assert worst <= TOL_BF16, worst
    del q, kc, vc
    torch.cuda.empty_cache()
