"""The C-ABI library without a GPU: it loads, exports every function the
header declares, rejects bad arguments before touching HIP, and answers the
size queries. No kernel is launched here."""
import ctypes
import os
import re

import pytest
import torch

import gqa_routed_query_amd as gq
from gqa_routed_query_amd import _binding

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, NO_DEVICE = 0, 1, 2, 3, 4
F32, BF16 = gq.GQA_F32, gq.GQA_BF16
P = 0x100000  # an aligned, never dereferenced stand-in pointer
lib = _binding._lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gqa|gqe)_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared_functions()
    assert {"gqa_prefill", "gqa_decode", "gqe_routed_prefill", "gqe_workspace_bytes"} <= set(names)
    so = ctypes.CDLL(gq.lib_path)
    for n in names:
        assert hasattr(so, n), f"{n} declared in gqa.h but not exported"


def test_abi_version_and_status_strings():
    assert gq.abi_version() == 2
    for s in range(6):
        assert gq.status_string(s)
    assert gq.status_string(99) == "unknown status"


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, out=P, B=1, h=4, g=2, T=16, d=16, i=F32, o=F32, scale=0.25,
             causal=1, stream=None)
    a.update(kw)
    return lib.gqa_prefill(a["q"], a["k"], a["v"], a["out"], a["B"], a["h"], a["g"], a["T"],
                           a["d"], a["i"], a["o"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(h=6, g=4), INVALID),            # g does not divide h
    (dict(g=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(T=-3), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(causal=2), INVALID),
    (dict(q=None), INVALID),
    (dict(out=P + 4), INVALID),            # misaligned
    (dict(i=7), INVALID),                  # unknown dtype
    (dict(d=48), UNSUPPORTED),
    (dict(i=BF16, d=48), UNSUPPORTED),     # bf16: d in {16, 32, 64, 128}
    (dict(i=BF16, d=8), UNSUPPORTED),
    (dict(h=1 << 20, g=1, T=1 << 12), INVALID),  # h*T beyond the row limit
])
def test_prefill_rejects(kw, status):
    assert _prefill(**kw) == status
    assert gq.last_error()


def test_prefill_empty_is_ok():
    assert _prefill(B=0) == OK
    assert _prefill(T=0, q=None) == OK


def _decode(**kw):
    a = dict(q=P, kc=P, vc=P, lens=P, out=P, B=2, h=8, g=2, T=1024, d=128, i=BF16, o=BF16,
             scale=0.088, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.gqa_decode(a["q"], a["kc"], a["vc"], a["lens"], a["out"], a["B"], a["h"], a["g"],
                          a["T"], a["d"], a["i"], a["o"], a["scale"], a["ws"], a["wsb"],
                          a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(h=8, g=3), INVALID),
    (dict(lens=None), INVALID),
    (dict(i=7), INVALID),                  # not a dtype
    (dict(d=8), UNSUPPORTED),              # decode takes d in {16, 32, 64, 128}
    (dict(d=48), UNSUPPORTED),
    (dict(h=128, g=1), UNSUPPORTED),       # 128 heads per group
    (dict(wsb=0, T=1 << 16), WORKSPACE),
    (dict(scale=float("inf")), INVALID),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def _gqe(**kw):
    a = dict(q=P, k=P, v=P, lg=P, k_top=1, out=P, idx=P, gate=P, B=1, h=8, g=2, T=16, d=128,
             i=BF16, o=BF16, scale=0.088, causal=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.gqe_routed_prefill(a["q"], a["k"], a["v"], a["lg"], a["k_top"], a["out"],
                                  a["idx"], a["gate"], a["B"], a["h"], a["g"], a["T"], a["d"],
                                  a["i"], a["o"], a["scale"], a["causal"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k_top=0), INVALID),
    (dict(k_top=5), INVALID),              # more than h/g = 4
    (dict(lg=None), INVALID),
    (dict(idx=None), INVALID),
    (dict(h=130, g=1, k_top=1), UNSUPPORTED),
    (dict(ws=P + 8, wsb=1 << 20), INVALID),   # workspace not 16-byte aligned
])
def test_gqe_rejects(kw, status):
    assert _gqe(**kw) == status


def test_gqe_workspace_bytes():
    """Key splitting is planned only for causal grids of less than two blocks
    per CU, upper-half row tiles only: the GQE workload (B=2, T=4096, h=32, g=8,
    k=1) needs a workspace, large grids need none, invalid shapes return 0.
    Without a GPU the size is computed for 256 CUs (MI355X). At k=1 the split
    launch takes the 12-wave grid (384-row tiles: 11 per problem, at most 5 in
    the upper half with a split point)."""
    def per_split(BG, rows, d):
        # one split row tile of every problem: part 1's partial result (bf16 rows of d,
        # fp32 row max and row sum: rows * (d / 2 + 2) floats) and its 8-byte ready flag
        return BG * (rows * (d // 2 + 2) * 4 + 8)

    small = gq.gqe_workspace_bytes(2, 32, 8, 4096, 128, 1)
    assert small > 0 and small % 16 == 0
    assert small % per_split(16, 384, 128) == 0 and small // per_split(16, 384, 128) <= 6
    # at k=2 the grid takes two rounds of 12-wave blocks: the 8-wave grid (256-row tiles) is split
    k2 = gq.gqe_workspace_bytes(2, 32, 8, 4096, 128, 2)
    assert k2 == 0 or k2 % per_split(16, 256, 128) == 0
    # small split grids keep 12 waves too: B=2, g=2, T=300, k=2 is 600 rows per problem, two
    # 384-row tiles (one in the upper half); B=1, g=4, T=333, d=64, k=3 is 999 rows, three tiles
    assert gq.gqe_workspace_bytes(2, 8, 2, 300, 128, 2) == 1 * per_split(4, 384, 128)
    w = gq.gqe_workspace_bytes(1, 12, 4, 333, 64, 3)
    assert w > 0 and w % per_split(4, 384, 64) == 0
    # 170 problems of three 256-row tiles: two tiles have a split point, but the second parts
    # (which wait for the first) must stay fewer than the 256 CUs, so one split at most
    assert gq.gqe_workspace_bytes(17, 20, 10, 700, 128, 1) == 1 * per_split(170, 256, 128)
    assert gq.gqe_workspace_bytes(64, 32, 8, 4096, 128, 1) == 0   # 2048+ blocks: no split
    assert gq.gqe_workspace_bytes(2, 32, 8, 4096, 128, 5) == 0    # top_k > h/g
    assert gq.gqe_workspace_bytes(2, 32, 8, 4096, 96, 1) == 0     # d not run on the bf16 kernel
    assert gq.gqe_workspace_bytes(0, 32, 8, 4096, 128, 1) == 0


def _gqe_decode(**kw):
    a = dict(q=P, kc=P, vc=P, lens=P, lg=P, k_top=1, out=P, idx=P, gate=P, B=2, h=8, g=2, T=1024,
             d=128, i=BF16, o=BF16, scale=0.088, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.gqe_routed_decode(a["q"], a["kc"], a["vc"], a["lens"], a["lg"], a["k_top"], a["out"],
                                 a["idx"], a["gate"], a["B"], a["h"], a["g"], a["T"], a["d"], a["i"],
                                 a["o"], a["scale"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k_top=0), INVALID),
    (dict(k_top=5), INVALID),              # more than h/g = 4
    (dict(lg=None), INVALID),
    (dict(gate=None), INVALID),
    (dict(h=8, g=3), INVALID),
    (dict(i=7), INVALID),                  # not a dtype
    (dict(wsb=0), WORKSPACE),
])
def test_gqe_decode_rejects(kw, status):
    assert _gqe_decode(**kw) == status


def _router(**kw):
    a = dict(x=P, w=P, k_top=1, lg=P, idx=P, gate=P, n=64, dm=4096, h=32, g=8, i=BF16, stream=None)
    a.update(kw)
    return lib.gqe_router(a["x"], a["w"], a["k_top"], a["lg"], a["idx"], a["gate"], a["n"], a["dm"],
                          a["h"], a["g"], a["i"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k_top=0), INVALID),
    (dict(k_top=5), INVALID),              # more than h/g = 4
    (dict(h=32, g=5), INVALID),
    (dict(n=-1), INVALID),
    (dict(x=None), INVALID),
    (dict(idx=None), INVALID),
    (dict(w=P + 8), INVALID),              # misaligned
    (dict(i=F32), UNSUPPORTED),
    (dict(dm=200), UNSUPPORTED),           # not a multiple of 128
    (dict(h=128, g=2), UNSUPPORTED),       # more than 64 heads
])
def test_router_rejects(kw, status):
    assert _router(**kw) == status


def test_router_empty_and_optional_logits():
    assert _router(n=0, x=None) == OK
    if torch.cuda.device_count() == 0:
        assert _router(lg=None) == NO_DEVICE   # logits may be NULL


def _build(**kw):
    a = dict(q=P, qs=P, k=P, v=P, lg=P, k_top=1, skv=0, oc=P, ow=P, osh=P, idx=P, gate=P, B=1, h=16,
             g=8, T=64, d=128, i=BF16, o=BF16, scale=0.088, causal=1, stream=None)
    a.update(kw)
    return lib.gqe_prefill_build(a["q"], a["qs"], a["k"], a["v"], a["lg"], a["k_top"], a["skv"],
                                 a["oc"], a["ow"], a["osh"], a["idx"], a["gate"], a["B"], a["h"],
                                 a["g"], a["T"], a["d"], a["i"], a["o"], a["scale"], a["causal"],
                                 a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k_top=0), INVALID),
    (dict(k_top=3), INVALID),              # more than h/g = 2
    (dict(skv=8), INVALID),
    (dict(skv=-1), INVALID),
    (dict(qs=None), INVALID),
    (dict(osh=None), INVALID),
    (dict(ow=P + 4), INVALID),             # misaligned
    (dict(i=F32, d=16), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED),
])
def test_gqe_build_rejects(kw, status):
    assert _build(**kw) == status


def test_gqe_decode_empty_batch_is_ok():
    assert _gqe_decode(B=0, q=None, lg=None) == OK


def test_peak_probes_reject_bad_args():
    fl = ctypes.c_double(0.0)
    assert lib.gqa_peak_hbm_read(P, 15, P, None) == INVALID        # not a multiple of 16
    assert lib.gqa_peak_hbm_read(None, 16, P, None) == INVALID     # null buffer
    assert lib.gqa_peak_hbm_read(P, 16, None, None) == INVALID     # null result
    assert lib.gqa_peak_hbm_read(P + 8, 16, P, None) == INVALID    # misaligned buffer
    assert lib.gqa_peak_hbm_read(P, 16, P + 2, None) == INVALID    # misaligned result
    assert lib.gqa_peak_hbm_read(None, 0, None, None) == OK        # nothing to read
    assert lib.gqa_peak_mfma_bf16(P, 0, P, ctypes.byref(fl), None) == INVALID
    assert lib.gqa_peak_mfma_bf16(None, 1, P, ctypes.byref(fl), None) == INVALID
    assert lib.gqa_peak_mfma_bf16(P, 1, None, ctypes.byref(fl), None) == INVALID
    assert lib.gqa_peak_mfma_bf16(P, 1, P, None, None) == INVALID
    assert lib.gqa_peak_mfma_bf16(P + 4, 1, P, ctypes.byref(fl), None) == INVALID


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: would launch")
def test_valid_calls_report_no_device():
    assert _prefill() == NO_DEVICE
    assert _decode() == NO_DEVICE
    assert _decode(i=F32, o=F32) == NO_DEVICE      # fp32 caches pass validation
    assert _gqe() == NO_DEVICE
    assert _gqe_decode() == NO_DEVICE
    assert _gqe_decode(i=F32) == NO_DEVICE
    assert _build() == NO_DEVICE
    assert lib.gqa_peak_hbm_read(P, 16, P, None) == NO_DEVICE
    assert lib.gqa_peak_mfma_bf16(P, 1, P, ctypes.byref(ctypes.c_double(0.0)), None) == NO_DEVICE


def test_kv_cache_bytes_matches_oracle_law():
    for (B, n_kv, T, d) in [(1, 8, 4096, 128), (32, 1, 16384, 128), (64, 8, 4608, 128), (3, 5, 7, 16)]:
        assert gq.gqa_kv_cache_bytes(B, n_kv, T, d, torch.bfloat16) == \
            oracle.kv_cache_bytes(B, n_kv, T, d, 2)
        assert gq.gqa_kv_cache_bytes(B, n_kv, T, d, torch.float32) == \
            oracle.kv_cache_bytes(B, n_kv, T, d, 4)
    # the h/g reduction: 32 query heads over 8 KV groups -> 4x smaller cache
    assert gq.gqa_kv_cache_bytes(1, 32, 4096, 128) == 4 * gq.gqa_kv_cache_bytes(1, 8, 4096, 128)


def test_decode_workspace_bytes():
    assert gq.gqa_decode_workspace_bytes(-1, 8, 2, 100, 128) == 0
    assert gq.gqa_decode_workspace_bytes(2, 8, 2, -5, 128) == 0
    assert gq.gqa_decode_workspace_bytes(2, 8, 3, 100, 128) == 0   # g does not divide h
    # two partials of r heads per wave of the grid: independent of B and T_max,
    # empty batches and empty caches included
    small = gq.gqa_decode_workspace_bytes(1, 8, 2, 100, 128)
    assert small > 0
    assert small == gq.gqa_decode_workspace_bytes(64, 8, 2, 16384, 128)
    assert small == gq.gqa_decode_workspace_bytes(0, 8, 2, 100, 128)
    assert small == gq.gqa_decode_workspace_bytes(3, 8, 2, 0, 128)
    # and proportional to r*(d+2) (up to the 256-byte alignment of the first region)
    r4 = gq.gqa_decode_workspace_bytes(64, 32, 8, 8192, 128)
    r1 = gq.gqa_decode_workspace_bytes(64, 32, 32, 8192, 128)
    assert abs(r4 - 4 * r1) <= 1024
    # a small fraction of the decode workload's cache (64 x 8 groups x 8192 keys)
    assert r4 < 0.01 * gq.gqa_kv_cache_bytes(64, 8, 8192, 128)


def test_decode_workspace_units_override(monkeypatch):
    monkeypatch.setenv("GQA_DECODE_UNITS", "3")
    # 3 waves x 2 partials x 4 heads x 128 floats (rounded to 256 B) + 3 x 2 x 4 x 2 floats
    assert gq.gqa_decode_workspace_bytes(4, 16, 4, 1000, 128) == 12288 + 192


def test_decode_empty_cache_accepts_its_workspace():
    """T_max = 0 (every row zero): the size query's workspace passes the
    argument checks, so the call fails only for want of a device here. (With a
    device it would launch on the stand-in pointers; the GPU tests cover it.)"""
    if torch.cuda.is_available():
        pytest.skip("a device is visible: the call would launch")
    ws = gq.gqa_decode_workspace_bytes(2, 8, 2, 0, 128)
    st = lib.gqa_decode(P, None, None, P, P, 2, 8, 2, 0, 128, BF16, BF16, 0.1, P, ws, None)
    assert st == NO_DEVICE, gq.last_error()
    st = lib.gqa_decode(P, None, None, P, P, 2, 8, 2, 0, 128, BF16, BF16, 0.1, P, ws - 1, None)
    assert st == WORKSPACE


def _noalloc(B=4, h=32, g=8, T=8192, d=128, i=BF16):
    return lib.gqa_decode_noalloc(P, P, P, P, P, B, h, g, T, d, i, BF16, 0.1, None)


def test_decode_noalloc_checks(monkeypatch):
    """The allocation-free decode takes gqa_decode's argument checks and
    rejects, before any HIP call, shapes whose split partials exceed its
    16 MiB static scratch."""
    assert _noalloc(g=7) == INVALID
    assert _noalloc(i=7) == INVALID
    assert _noalloc(d=48) == UNSUPPORTED
    assert _noalloc(B=0) == OK
    monkeypatch.setenv("GQA_DECODE_UNITS", "100000")   # 100000 waves x 2 x 4 heads x 130 floats
    assert _noalloc() == WORKSPACE
    assert "16777216" in gq.last_error()
    if not torch.cuda.is_available():
        monkeypatch.setenv("GQA_DECODE_UNITS", "512")
        assert _noalloc() == NO_DEVICE
        assert _noalloc(i=F32) == NO_DEVICE
