"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each pin is a plain function that raises ``AssertionError`` when the oracle
disagrees with a library routine (torch's scaled_dot_product_attention in
float64, numpy's stable argsort, scipy's softmax), a closed form, an invariant,
brute force on tiny inputs, or a worked example printed on the pages (the
fixtures under ``tests/golden``). ``test_oracle.py`` runs every pin, and
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and
checks that some pin catches each one.

The pins call the oracle through its module attributes, so a patched step is
seen by every function that uses it.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import oracle.gqa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, causal, gqa=True, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal,
                                          enable_gqa=gqa, scale=scale).numpy()


# --------------------------------------------------------------------------
# GQA prefill
# --------------------------------------------------------------------------

def pin_sdpa_gqa():
    """Oracle = torch SDPA (float64, enable_gqa) on several head layouts,
    with and without the causal mask, default and explicit scale."""
    cases = [(1, 4, 2, 16, 16), (1, 4, 4, 16, 16), (1, 4, 1, 16, 16),
             (2, 8, 2, 13, 8), (1, 6, 3, 9, 5)]
    for n, (B, h, g, T, d) in enumerate(cases):
        q = _rand((B, h, T, d), 10 + n)
        k = _rand((B, g, T, d), 20 + n)
        v = _rand((B, g, T, d), 30 + n)
        for causal in (True, False):
            got = orc.gqa_ref(q, k, v, causal=causal)
            ref = _sdpa(q, k, v, causal)
            assert np.abs(got - ref).max() < 1e-12, (B, h, g, T, d, causal)
        got = orc.gqa_ref(q, k, v, causal=True, scale=0.3)
        ref = _sdpa(q, k, v, True, scale=0.3)
        assert np.abs(got - ref).max() < 1e-12


def pin_special_cases_mha_mqa():
    """g = h is plain multi-head attention (each head its own K/V); g = 1 is
    multi-query attention (all heads read KV head 0)."""
    cases = _golden("mha_mqa_special_cases.json")["cases"]
    for n, c in enumerate(cases):
        h, g = c["h"], c["g"]
        B, T, d = 2, 11, 8
        q = _rand((B, h, T, d), 40 + n)
        k = _rand((B, g, T, d), 50 + n)
        v = _rand((B, g, T, d), 60 + n)
        got = orc.gqa_ref(q, k, v, causal=True)
        if c["equals"] == "mha":
            ref = _sdpa(q, k, v, True, gqa=False)
        else:
            ke = np.broadcast_to(k, (B, h, T, d))
            ve = np.broadcast_to(v, (B, h, T, d))
            ref = _sdpa(q, ke, ve, True, gqa=False)
        assert np.abs(got - ref).max() < 1e-12, c


def pin_head_to_group_example():
    """Worked example: 8 query heads in 2 groups -> heads 0-3 use KV head 0,
    heads 4-7 use KV head 1. Checked on the index map and end to end: with
    V constant per KV head, each query head's output is its group's constant."""
    fx = _golden("head_to_group_map.json")
    h, g = fx["h"], fx["g"]
    assert [orc.kv_head_of(i, h, g) for i in range(h)] == fx["kv_head_of_query_head"]
    B, T, d = 1, 5, 4
    q = _rand((B, h, T, d), 70)
    k = _rand((B, g, T, d), 71)
    v = np.zeros((B, g, T, d))
    for gam in range(g):
        v[:, gam] = 10.0 * (gam + 1)
    out = orc.gqa_ref(q, k, v, causal=True)
    for i, kv in enumerate(fx["kv_head_of_query_head"]):
        assert np.abs(out[0, i] - 10.0 * (kv + 1)).max() < 1e-12, i


def pin_brute_force_tiny():
    """Scalar brute force with math.exp / math.fsum, no max shift, no matrix
    routines, on tiny inputs."""
    B, h, g, T, d = 1, 4, 2, 4, 3
    q = _rand((B, h, T, d), 80)
    k = _rand((B, g, T, d), 81)
    v = _rand((B, g, T, d), 82)
    r = h // g
    for causal in (True, False):
        got = orc.gqa_ref(q, k, v, causal=causal)
        for i in range(h):
            kv = i // r
            for t in range(T):
                keys = range(t + 1) if causal else range(T)
                w = [math.exp(math.fsum(q[0, i, t, c] * k[0, kv, j, c] for c in range(d))
                              / math.sqrt(d)) for j in keys]
                z = math.fsum(w)
                for c in range(d):
                    o = math.fsum(wj * v[0, kv, j, c] for wj, j in zip(w, keys)) / z
                    assert abs(got[0, i, t, c] - o) < 1e-12, (i, t, c, causal)


def pin_row_sums():
    """Attention weights of every row sum to one."""
    q = _rand((2, 8, 17, 16), 90, 3.0)
    k = _rand((2, 2, 17, 16), 91, 3.0)
    v = _rand((2, 2, 17, 16), 92)
    for causal in (True, False):
        _, sums = orc.gqa_ref(q, k, v, causal=causal, return_probs=True)
        assert np.abs(sums - 1.0).max() < 1e-12


def pin_closed_forms():
    """Q = 0 gives uniform weights: row t is the mean of V[0..t] (causal) or
    of all V (non-causal). T = 1 gives O = V. Row 0 under the mask is V[0].
    A constant V gives that constant. A key that matches far better than all
    others pulls the output onto its value row."""
    B, h, g, T, d = 2, 6, 3, 9, 8
    r = h // g
    q0 = np.zeros((B, h, T, d))
    k = _rand((B, g, T, d), 100)
    v = _rand((B, g, T, d), 101)
    oc = orc.gqa_ref(q0, k, v, causal=True)
    on = orc.gqa_ref(q0, k, v, causal=False)
    for i in range(h):
        pref = np.cumsum(v[:, i // r], axis=1) / np.arange(1, T + 1)[None, :, None]
        assert np.abs(oc[:, i] - pref).max() < 1e-12
        assert np.abs(on[:, i] - v[:, i // r].mean(axis=1, keepdims=True)).max() < 1e-12
    q = _rand((B, h, T, d), 102)
    o1 = orc.gqa_ref(q[:, :, :1], k[:, :, :1], v[:, :, :1], causal=False)
    assert np.abs(o1 - np.repeat(v[:, :, :1], r, axis=1)).max() < 1e-12
    oc = orc.gqa_ref(q, k, v, causal=True)
    assert np.abs(oc[:, :, 0] - np.repeat(v[:, :, 0], r, axis=1)).max() < 1e-12
    vc = np.full((B, g, T, d), 0.625)
    assert np.abs(orc.gqa_ref(q, k, vc, causal=True) - 0.625).max() < 1e-12
    # large-margin match: query equals 40 * (unit key j*), other keys orthogonal-ish
    d2 = 16
    keys = np.eye(d2)[None, None, :8]              # 8 orthonormal keys
    vals = _rand((1, 1, 8, d2), 103)
    qs = np.broadcast_to(40.0 * math.sqrt(d2) * np.eye(d2)[5], (1, 1, 8, d2))
    o = orc.gqa_ref(qs, keys, vals, causal=False)
    # weight on key 5 is 1/(1+7e^-40): every row equals vals[5] to ~1e-16
    assert np.abs(o[0, 0] - vals[0, 0, 5]).max() < 1e-12


def pin_causal_future_invariance():
    """Changing keys/values at positions after t leaves rows 0..t unchanged."""
    B, h, g, T, d = 1, 4, 2, 12, 8
    q = _rand((B, h, T, d), 110)
    k = _rand((B, g, T, d), 111)
    v = _rand((B, g, T, d), 112)
    base = orc.gqa_ref(q, k, v, causal=True)
    t0 = 6
    k2, v2 = k.copy(), v.copy()
    k2[:, :, t0 + 1:] = _rand(k2[:, :, t0 + 1:].shape, 113, 5.0)
    v2[:, :, t0 + 1:] = _rand(v2[:, :, t0 + 1:].shape, 114, 5.0)
    pert = orc.gqa_ref(q, k2, v2, causal=True)
    assert np.abs(pert[:, :, :t0 + 1] - base[:, :, :t0 + 1]).max() < 1e-14
    assert np.abs(pert[:, :, t0 + 1:] - base[:, :, t0 + 1:]).max() > 1e-3


def pin_single_row():
    """The one-row form agrees with the full prefill."""
    B, h, g, T, d = 2, 8, 2, 10, 8
    q = _rand((B, h, T, d), 120)
    k = _rand((B, g, T, d), 121)
    v = _rand((B, g, T, d), 122)
    for causal in (True, False):
        full = orc.gqa_ref(q, k, v, causal=causal)
        for (b, i, t) in [(0, 0, 0), (1, 7, 9), (0, 3, 4), (1, 4, 2)]:
            row = orc.gqa_ref_row(q, k, v, b, i, t, causal=causal)
            assert np.abs(row - full[b, i, t]).max() < 1e-12


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

def pin_decode_matches_prefill():
    """Decoding token t over a cache holding positions 0..t equals row t of
    causal prefill; lens = 0 gives zeros; NaN padding past lens is never read."""
    B, h, g, T, d = 3, 8, 2, 14, 8
    q = _rand((B, h, T, d), 130)
    k = _rand((B, g, T, d), 131)
    v = _rand((B, g, T, d), 132)
    pre = orc.gqa_ref(q, k, v, causal=True)
    ts = [0, 7, 13]
    lens = np.array([t + 1 for t in ts])
    qd = np.stack([q[b, :, t] for b, t in enumerate(ts)])
    kc, vc = k.copy(), v.copy()
    for b, n in enumerate(lens):
        kc[b, :, n:] = np.nan
        vc[b, :, n:] = np.nan
    out = orc.gqa_decode_ref(qd, kc, vc, lens)
    for b, t in enumerate(ts):
        assert np.abs(out[b] - pre[b, :, t]).max() < 1e-12, t
    out0 = orc.gqa_decode_ref(qd, kc, vc, np.array([0, 3, 0]))
    assert np.all(out0[0] == 0) and np.all(out0[2] == 0)
    assert np.isfinite(out0).all()


def pin_decode_sdpa():
    """Decode equals torch SDPA of one query against the valid cache prefix."""
    B, h, g, Tm, d = 4, 8, 4, 20, 16
    q = _rand((B, h, d), 140)
    kc = _rand((B, g, Tm, d), 141)
    vc = _rand((B, g, Tm, d), 142)
    lens = np.array([1, 20, 7, 13])
    out = orc.gqa_decode_ref(q, kc, vc, lens)
    for b in range(B):
        n = lens[b]
        ref = _sdpa(q[b:b + 1, :, None], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], False)
        assert np.abs(out[b] - ref[0, :, 0]).max() < 1e-12


# --------------------------------------------------------------------------
# GQE routing
# --------------------------------------------------------------------------

def _tied_logits(shape, seed):
    return np.round(_rand(shape, seed) * 2.0) / 2.0


def pin_topk_brute_force():
    """The kept set is a maximum-sum k-subset of the group's logits; among
    equal sums the lexicographically smallest head set wins (lower index on
    ties); the k indices come in rank order."""
    for r, g in [(2, 3), (3, 2), (4, 2), (8, 1)]:
        h = r * g
        lg = _tied_logits((2, 6, h), 150 + r).astype(np.float32)
        for k in range(1, r + 1):
            idx, gate = orc.gqe_topk_ref(lg, g, k)
            for b in range(2):
                for t in range(6):
                    for gam in range(g):
                        ell = lg[b, t, gam * r:(gam + 1) * r].astype(np.float64)
                        best = max(itertools.combinations(range(r), k),
                                   key=lambda s: (sum(ell[list(s)]), [-e for e in s]))
                        got = [int(x) - gam * r for x in idx[b, t, gam]]
                        assert sorted(got) == list(best), (r, k, ell, got, best)
                        for a, c in zip(got, got[1:]):
                            assert ell[a] > ell[c] or (ell[a] == ell[c] and a < c)


def pin_topk_stable_argsort():
    """Same selection and order as numpy's stable argsort of the negated
    float32 logits, including +0.0 / -0.0 ties."""
    g, r = 8, 4
    lg = _tied_logits((3, 40, g * r), 160).astype(np.float32)
    lg[0, 0, :4] = [0.0, -0.0, 0.0, -0.0]
    lg[0, 1, 4:8] = [-0.0, 0.0, 1.0, 1.0]
    for k in (1, 2, 3):
        idx, _ = orc.gqe_topk_ref(lg, g, k)
        for b in range(3):
            for t in range(40):
                for gam in range(g):
                    ell = lg[b, t, gam * r:(gam + 1) * r]
                    ref = np.argsort(-ell, kind="stable")[:k] + gam * r
                    assert list(idx[b, t, gam]) == list(ref)


def pin_gates():
    """k = 1 gives gate 1 exactly; the k gates sum to 1; k = h/g gives the
    full softmax of the group's logits (scipy) in rank order; all-equal
    logits keep the lowest heads with gates 1/k."""
    g, r = 4, 4
    lg = _rand((2, 10, g * r), 170).astype(np.float32)
    idx1, gate1 = orc.gqe_topk_ref(lg, g, 1)
    assert np.all(gate1 == 1.0)
    for k in (2, 3):
        _, gk = orc.gqe_topk_ref(lg, g, k)
        assert np.abs(gk.sum(-1) - 1.0).max() < 1e-14
    idx, gate = orc.gqe_topk_ref(lg, g, r)
    for b in range(2):
        for t in range(10):
            for gam in range(g):
                sm = scipy.special.softmax(lg[b, t, gam * r:(gam + 1) * r].astype(np.float64))
                ref = sm[idx[b, t, gam] - gam * r]
                assert np.abs(gate[b, t, gam] - ref).max() < 1e-14
    flat = np.zeros((1, 3, g * r), dtype=np.float32)
    for k in (1, 2, 4):
        idx, gate = orc.gqe_topk_ref(flat, g, k)
        for gam in range(g):
            assert list(idx[0, 0, gam]) == [gam * r + e for e in range(k)]
            assert np.abs(gate[0, 0, gam] - 1.0 / k).max() < 1e-15


def pin_gqe_structure():
    """Exactly B*T*g*k rows are nonzero; selected rows are gate times the
    dense GQA row (the KV path stays dense); with k = h/g and all gates
    compared, permuting experts inside a group together with their logits
    permutes the outputs."""
    B, h, g, T, d = 2, 8, 2, 9, 8
    r = h // g
    q = _rand((B, h, T, d), 180)
    k = _rand((B, g, T, d), 181)
    v = _rand((B, g, T, d), 182)
    lg = _rand((B, T, h), 183).astype(np.float32)
    dense = _sdpa(q, k, v, True)
    for kk in (1, 2, r):
        out, idx, gate = orc.gqe_ref(q, k, v, lg, kk, causal=True)
        nz = np.abs(out).sum(-1) > 0          # [B,h,T]
        assert nz.sum() == B * T * g * kk
        for b in range(B):
            for t in range(T):
                for gam in range(g):
                    for j in range(kk):
                        i = idx[b, t, gam, j]
                        assert nz[b, i, t]
                        assert np.abs(out[b, i, t] - gate[b, t, gam, j] * dense[b, i, t]).max() < 1e-12
        if kk == 1:
            assert np.all(gate == 1.0)
    perm = np.array([2, 0, 3, 1, 6, 7, 5, 4])  # within-group permutation
    out, _, _ = orc.gqe_ref(q, k, v, lg, 2, causal=True)
    outp, _, _ = orc.gqe_ref(q[:, perm], k, v, lg[:, :, perm], 2, causal=True)
    assert np.abs(outp - out[:, perm]).max() < 1e-12


def pin_gqe_decode():
    """Routed decode of token t over a cache of positions 0..t, with token t's
    router logits, equals row t of routed prefill (same kept heads, gates and
    rows); k = h/g keeps every head with gates equal to the group softmax
    (scipy); a sequence with no cached keys gives zero rows; NaN padding past
    lens is never read."""
    B, h, g, T, d = 3, 8, 2, 12, 8
    r = h // g
    q = _rand((B, h, T, d), 190)
    k = _rand((B, g, T, d), 191)
    v = _rand((B, g, T, d), 192)
    lg = _tied_logits((B, T, h), 193).astype(np.float32)
    ts = [0, 5, 11]
    lens = np.array([t + 1 for t in ts])
    qd = np.stack([q[b, :, t] for b, t in enumerate(ts)])
    lgd = np.stack([lg[b, t] for b, t in enumerate(ts)])
    kc, vc = k.copy(), v.copy()
    for b, n in enumerate(lens):
        kc[b, :, n:] = np.nan
        vc[b, :, n:] = np.nan
    for kk in (1, 2, r):
        pre, pidx, pgate = orc.gqe_ref(q, k, v, lg, kk, causal=True)
        out, idx, gate = orc.gqe_decode_ref(qd, kc, vc, lens, lgd, kk)
        assert np.isfinite(out).all()
        for b, t in enumerate(ts):
            assert np.array_equal(idx[b], pidx[b, t])
            assert np.abs(gate[b] - pgate[b, t]).max() < 1e-15
            assert np.abs(out[b] - pre[b, :, t]).max() < 1e-12, (kk, t)
        assert (np.abs(out).sum(-1) > 0).sum() == B * g * kk
    out, idx, gate = orc.gqe_decode_ref(qd, kc, vc, lens, lgd, r)
    for b in range(B):
        for gam in range(g):
            sm = scipy.special.softmax(lgd[b, gam * r:(gam + 1) * r].astype(np.float64))
            assert np.abs(gate[b, gam] - sm[idx[b, gam] - gam * r]).max() < 1e-14
    out0, _, _ = orc.gqe_decode_ref(qd, kc, vc, np.array([0, 4, 0]), lgd, 2)
    assert np.all(out0[0] == 0) and np.all(out0[2] == 0) and np.abs(out0[1]).sum() > 0


def pin_gqe_router():
    """Router logits equal torch's linear layer (x W^T, float64); the kept
    experts and gates equal gqe_topk_ref of those logits; the fp32 error bound
    covers a float32 evaluation of the same dot products (torch, float32)."""
    n, dm, h, g = 37, 96, 16, 4
    x = _rand((n, dm), 200)
    w = _rand((h, dm), 201) / math.sqrt(dm)
    logits, bound, idx, gate = orc.gqe_router_ref(x, w, g, 2)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    assert np.abs(logits - ref).max() < 1e-12
    ridx, rgate = orc.gqe_topk_ref(ref.reshape(1, n, h), g, 2)
    assert np.array_equal(idx, ridx[0]) and np.abs(gate - rgate[0]).max() < 1e-15
    f32 = torch.nn.functional.linear(torch.from_numpy(x).float(), torch.from_numpy(w).float())
    err = np.abs(f32.double().numpy() - ref)
    assert np.all(err <= bound) and bound.max() < 1e-3
    assert idx.shape == (n, g, 2) and gate.shape == (n, g, 2)


def pin_gqe_build():
    """The output build: each group's weighted-sum slot equals the sum over
    the group's heads of the routed output (gqe_ref: gate x row for kept heads,
    0 otherwise); with every expert kept the concatenation is the group's dense
    rows in rank order; the shared head equals torch SDPA of its query against
    its KV head; g*k routed + 1 shared computations are active (9 of 16 at
    16 heads, 8 groups, k = 1)."""
    B, h, g, T, d = 2, 8, 2, 11, 8
    r = h // g
    q = _rand((B, h, T, d), 210)
    qs = _rand((B, T, d), 211)
    k = _rand((B, g, T, d), 212)
    v = _rand((B, g, T, d), 213)
    lg = _tied_logits((B, T, h), 214).astype(np.float32)
    dense = _sdpa(q, k, v, True)
    for kk in (1, 2, r):
        concat, wsum, shared, idx, gate = orc.gqe_build_ref(q, qs, k, v, lg, kk, shared_kv=1)
        routed, _, _ = orc.gqe_ref(q, k, v, lg, kk, causal=True)
        for gam in range(g):
            grp = routed[:, gam * r:(gam + 1) * r].sum(axis=1)        # [B,T,d]
            assert np.abs(wsum[:, :, gam] - grp).max() < 1e-12
        if kk == r:
            for b in range(B):
                for t in range(T):
                    for gam in range(g):
                        ref = dense[b, idx[b, t, gam], t]
                        assert np.abs(concat[b, t, gam] - ref).max() < 1e-12
    sh = _sdpa(qs[:, None], k[:, 1:2], v[:, 1:2], True)[:, 0]
    assert np.abs(shared - sh).max() < 1e-12
    assert orc.gqe_active_query_heads(8, 1) == 9


# --------------------------------------------------------------------------
# Accounting printed on the pages
# --------------------------------------------------------------------------

def pin_kv_cache_law():
    """KV-cache bytes equal the bytes of the K and V cache arrays, grow as
    2 * L * n_kv * d_h * T, and shrink by h/g from MHA to GQA (32 over 8 is
    4x, the pages' example)."""
    fx = _golden("kv_cache_reduction.json")
    for (B, n_kv, T, d, L) in [(1, 8, 16, 128, 1), (3, 2, 5, 64, 4), (2, 32, 7, 16, 2)]:
        kc = np.zeros((L, B, n_kv, T, d), dtype=np.float16)
        vc = np.zeros_like(kc)
        assert orc.kv_cache_bytes(B, n_kv, T, d, kc.itemsize, layers=L) == kc.nbytes + vc.nbytes
    h, g = fx["h"], fx["g"]
    mha = orc.kv_cache_bytes(1, h, 4096, 128, 2)
    gqa = orc.kv_cache_bytes(1, g, 4096, 128, 2)
    mqa = orc.kv_cache_bytes(1, 1, 4096, 128, 2)
    assert mha == fx["reduction"] * gqa
    assert mha == h * mqa


def pin_gqe_active_count():
    """16 query heads, 8 KV groups, k = 1: 8 routed + 1 shared = 9 of 16."""
    fx = _golden("gqe_active_heads.json")
    n = orc.gqe_active_query_heads(fx["g"], fx["top_k"], fx["shared"])
    assert n == fx["active"]
    assert round(100 * n / fx["h"]) == fx["percent_rounded"]


PINS = [
    pin_sdpa_gqa,
    pin_special_cases_mha_mqa,
    pin_head_to_group_example,
    pin_brute_force_tiny,
    pin_row_sums,
    pin_closed_forms,
    pin_causal_future_invariance,
    pin_single_row,
    pin_decode_matches_prefill,
    pin_decode_sdpa,
    pin_topk_brute_force,
    pin_topk_stable_argsort,
    pin_gates,
    pin_gqe_structure,
    pin_gqe_decode,
    pin_gqe_router,
    pin_gqe_build,
    pin_kv_cache_law,
    pin_gqe_active_count,
]
