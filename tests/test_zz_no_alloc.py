"""gqa_decode_noalloc (split partials in the library's static device scratch,
no allocation in the call) against gqa_decode, its workspace twin: two calls in
a row, the second on a smaller input, each equal to gqa_decode bit for bit (the
same kernels on the same grid) and to the float64 oracle within the bf16
tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, dev, max_abs, say
from workloads import decode_inputs

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_decode_twice():
    import gqa_routed_query_amd as gq

    d = dev()
    cases = [  # (B, h, g, T_max, d, lens range, seed): the second call is smaller
        (16, 32, 8, 3000, 128, (1, 3000), 901),
        (3, 8, 2, 500, 64, (0, 500), 902),
    ]
    for B, h, g, T_max, hd, lr, seed in cases:
        say(f"decode noalloc B={B} h={h} g={g} T_max={T_max} d={hd}")
        q, kc, vc, lens = decode_inputs(B, h, g, T_max, hd, lr, seed=seed, device=d)
        out_na = torch.empty(B, h, hd, dtype=torch.float32, device=d)
        gq.gqa_decode_noalloc(q, kc, vc, lens, out_na)
        out_ws = gq.gqa_decode(q, kc, vc, lens, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws)
        ref = oracle.gqa_decode_ref(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu())
        assert max_abs(out_na, ref) <= TOL_BF16


def test_noalloc_bf16_out_and_empty_rows():
    import gqa_routed_query_amd as gq

    d = dev()
    say("decode noalloc bf16 out, empty sequences")
    q, kc, vc, lens = decode_inputs(5, 16, 4, 700, 128, (1, 700), seed=903, device=d)
    lens[1] = 0
    lens[3] = 0
    out_na = torch.empty(5, 16, 128, dtype=torch.bfloat16, device=d)
    gq.gqa_decode_noalloc(q, kc, vc, lens, out_na)
    out_ws = gq.gqa_decode(q, kc, vc, lens, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws)
    assert float(out_na[1].float().abs().max()) == 0.0 and float(out_na[3].float().abs().max()) == 0.0
    ref = oracle.gqa_decode_ref(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu())
    assert max_abs(out_na, ref) <= TOL_BF16


def test_noalloc_fp32_cache():
    """fp32 caches through the static scratch: bit for bit the workspace call,
    within the fp32 tolerance of the oracle, two calls in a row (the second
    smaller, 32 heads per group: two 16-head grid rows)."""
    import gqa_routed_query_amd as gq

    d = dev()
    for B, h, g, T_max, hd, lr, seed in [(8, 16, 4, 2000, 128, (1, 2000), 904),
                                         (3, 32, 1, 400, 32, (0, 400), 905)]:
        say(f"decode noalloc fp32 cache B={B} h={h} g={g} T_max={T_max} d={hd}")
        q, kc, vc, lens = decode_inputs(B, h, g, T_max, hd, lr, dtype="f32", seed=seed, device=d)
        out_na = torch.empty(B, h, hd, dtype=torch.float32, device=d)
        gq.gqa_decode_noalloc(q, kc, vc, lens, out_na)
        out_ws = gq.gqa_decode(q, kc, vc, lens, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws)
        ref = oracle.gqa_decode_ref(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu())
        assert max_abs(out_na, ref) <= TOL_F32
