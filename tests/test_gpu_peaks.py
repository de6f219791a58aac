"""The peak microbenchmarks on the GPU: each checks the work it counts.

The HBM read stream folds every 32-bit word of its buffer into one XOR, so
the result equals numpy's XOR over the same bytes only if every 16-byte word
was read exactly once (a skipped or doubled word changes it unless it is
zero; the buffers are random). The MFMA loop adds the sum of its
accumulators, which equals (waves x 4 chains x iters) x sum(A B) computed in
float64 from the operands' fragment layout; a wrong wave count or a dropped
chain changes it by a whole factor.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bytes,start", [(16, 0), (4096 * 16 + 48, 0x5a5a5a5a), (96 << 20, 7)])
def test_peak_hbm_read_reads_every_word_once(n_bytes, start):
    import gqa_routed_query_amd as gq

    d = dev()
    g = torch.Generator().manual_seed(n_bytes)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (n_bytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.to(d)
    xo = torch.tensor([start], dtype=torch.int32, device=d)
    say(f"peak_hbm_read {n_bytes} B")
    gq.peak_hbm_read(buf, xo)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32)) ^ np.uint32(start)
    assert int(xo.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_peak_mfma_counts_its_work():
    import gqa_routed_query_amd as gq

    d = dev()
    g = torch.Generator().manual_seed(11)
    ops = torch.rand(1024, generator=g).to(torch.bfloat16)  # positive: no cancellation in sum(A B)
    iters = 50
    say("peak_mfma_bf16")
    so, flops = gq.peak_mfma_bf16(ops.to(d), iters)
    torch.cuda.synchronize()
    x = ops.float().double().numpy().reshape(2, 64, 8)
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for lane in range(64):
        A[lane % 32, 8 * (lane // 32):8 * (lane // 32) + 8] = x[0, lane]
        Bm[8 * (lane // 32):8 * (lane // 32) + 8, lane % 32] = x[1, lane]
    n_mfma = flops / (2.0 * 32 * 32 * 16)
    n_cu = torch.cuda.get_device_properties(d).multi_processor_count
    assert n_mfma == n_cu * 2 * 4 * 4 * iters  # 2 workgroups of 4 waves per CU, 4 chains each
    want = n_mfma * (A @ Bm).sum()
    got = float(so.item())
    assert abs(got - want) <= 1e-3 * abs(want) + 1e-2


def test_peak_rates_are_plausible():
    """Measured peaks sit below the datasheet peaks and well above a stall."""
    import gqa_routed_query_amd as gq

    d = dev()
    buf = torch.empty(1 << 31, dtype=torch.uint8, device=d).fill_(3)
    ops = torch.randn(1024, device=d).to(torch.bfloat16)
    gq.peak_hbm_read(buf)
    gq.peak_mfma_bf16(ops, 20000)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    gq.peak_hbm_read(buf)
    e1.record()
    _, flops = gq.peak_mfma_bf16(ops, 20000)
    e2.record()
    torch.cuda.synchronize()
    gbps = buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    tflops = flops / (e1.elapsed_time(e2) * 1e-3) / 1e12
    say(f"peak rates: {gbps:.0f} GB/s, {tflops:.0f} TFLOP/s")
    assert 2000 < gbps < 8200
    assert 800 < tflops < 2600


@pytest.mark.parametrize("iters", [1, 7, 300])
def test_peak_attn_tile_computes_the_tile(iters):
    """The attention tile loop repeats one 32-key tile, so its normalised
    output is the attention of the 32 queries over the 32 keys: the oracle's
    GQA prefill of one head without a mask, within the bf16 tolerance (P is
    rounded to bf16). The flops are 16 MFMAs of 32x32x16 per wave (12 per CU)
    and iteration."""
    import gqa_routed_query_amd as gq
    import oracle
    from gpu_util import TOL_BF16, max_abs

    d = dev()
    g = torch.Generator().manual_seed(17 + iters)
    qkv = torch.randn(3, 32, 128, generator=g).to(torch.bfloat16)
    say(f"peak_attn_tile iters={iters}")
    out, flops = gq.peak_attn_tile(qkv.to(d), iters)
    torch.cuda.synchronize()
    q, k, v = (qkv[i].view(1, 1, 32, 128) for i in range(3))
    ref = oracle.gqa_ref(q, k, v, causal=False)[0, 0]
    assert max_abs(out, ref) <= TOL_BF16
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == n_cu * 12 * iters * 16 * (2 * 32 * 32 * 16)
