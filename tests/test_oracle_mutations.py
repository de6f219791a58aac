"""Plant plausible mistakes in the CPU oracle and check that the pins catch
each one (a dropped term, a wrong sign, index or axis, a transposed operand,
an off-by-one, a wrong tie rule). Every mutation runs on the CPU only and is
undone by monkeypatch after its test."""
import numpy as np
import pytest
import scipy.special

import oracle.gqa_oracle as orc
from oracle_pins import PINS

_orig = {name: getattr(orc, name) for name in orc.__all__}


def _tile_kv(x, h):                       # strided head map instead of contiguous
    return np.tile(x, (1, h // x.shape[1], 1, 1))


def _scores_unscaled(q, k_rep, scale):    # dropped 1/sqrt(d)
    return np.matmul(q, np.swapaxes(k_rep, -1, -2))


def _scores_transposed(q, k_rep, scale):  # S^T instead of S
    return np.swapaxes(np.matmul(q, np.swapaxes(k_rep, -1, -2)), -1, -2) * scale


def _mask_strict(Tq, Tk):                 # diagonal excluded
    return np.arange(Tk)[None, :] < np.arange(Tq)[:, None]


def _mask_future(Tq, Tk):                 # wrong direction
    return np.arange(Tk)[None, :] >= np.arange(Tq)[:, None]


def _softmax_axis(s, visible=None):       # normalised over queries
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    e = np.exp(s - np.max(s, axis=-2, keepdims=True))
    return e / e.sum(axis=-2, keepdims=True)


def _softmax_sign(s, visible=None):       # exp(-s)
    return _orig["softmax"](-s, visible)


def _softmax_unnormalised(s, visible=None):
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    return np.exp(s - m)


def _row_off_by_one(q, k, v, b, i, t, causal=True, scale=None):
    return _orig["gqa_ref_row"](q, k, v, b, i, max(t - 1, 0), causal, scale)


def _decode_short(q, kc, vc, lens, scale=None):   # one cached position too few
    lens = np.maximum(np.asarray(lens) - 1, 0)
    return _orig["gqa_decode_ref"](q, kc, vc, lens, scale)


def _topk_ties_high(logits, g, top_k):    # ties to the higher head index
    lg = np.asarray(logits)
    B, T, h = lg.shape
    r = h // g
    rev = np.concatenate([np.arange(gam * r, (gam + 1) * r)[::-1] for gam in range(g)])
    idx, gate = _orig["gqe_topk_ref"](lg[:, :, rev], g, top_k)
    return rev[idx].astype(np.int32), gate


def _topk_gate_unrenormalised(logits, g, top_k):
    idx, _ = _orig["gqe_topk_ref"](logits, g, top_k)
    lg = np.asarray(logits, dtype=np.float64)
    B, T, h = lg.shape
    r = h // g
    prob = scipy.special.softmax(lg.reshape(B, T, g, r), axis=-1).reshape(B, T, h)
    gate = np.take_along_axis(prob[:, :, None, :].repeat(g, 2), idx, axis=-1)
    return idx, gate


def _gqe_no_zero(q, k, v, logits, top_k, causal=True, scale=None):
    out, idx, gate = _orig["gqe_ref"](q, k, v, logits, top_k, causal, scale)
    dense = _orig["gqa_ref"](q, k, v, causal=causal, scale=scale)
    return np.where(out == 0, dense, out), idx, gate


def _gqe_no_gate(q, k, v, logits, top_k, causal=True, scale=None):
    out, idx, gate = _orig["gqe_ref"](q, k, v, logits, top_k, causal, scale)
    dense = _orig["gqa_ref"](q, k, v, causal=causal, scale=scale)
    return np.where(out != 0, dense, 0.0), idx, gate


def _kv_bytes_no_two(B, n_kv, T, d, elt_bytes, layers=1):
    return layers * n_kv * d * T * elt_bytes * B


def _kv_head_strided(i, h, g):
    return i % g


def _gqe_decode_no_gate(q, kc, vc, lens, logits, top_k, scale=None):
    out, idx, gate = _orig["gqe_decode_ref"](q, kc, vc, lens, logits, top_k, scale)
    dense = _orig["gqa_decode_ref"](q, kc, vc, lens, scale)
    return np.where(np.abs(out).sum(-1, keepdims=True) > 0, dense, 0.0), idx, gate


def _gqe_decode_no_zero(q, kc, vc, lens, logits, top_k, scale=None):
    out, idx, gate = _orig["gqe_decode_ref"](q, kc, vc, lens, logits, top_k, scale)
    dense = _orig["gqa_decode_ref"](q, kc, vc, lens, scale)
    return np.where(np.abs(out).sum(-1, keepdims=True) > 0, out, dense), idx, gate


def _router_dropped_feature(x, w_r, g, top_k):   # the last input feature ignored
    return _orig["gqe_router_ref"](np.asarray(x)[:, :-1], np.asarray(w_r)[:, :-1], g, top_k)


def _build_wrong_shared_kv(q, q_shared, k, v, logits, top_k, shared_kv=0, causal=True, scale=None):
    return _orig["gqe_build_ref"](q, q_shared, k, v, logits, top_k, (shared_kv + 1) % k.shape[1],
                                  causal, scale)


def _build_wsum_unrenormalised(q, q_shared, k, v, logits, top_k, shared_kv=0, causal=True, scale=None):
    concat, wsum, shared, idx, gate = _orig["gqe_build_ref"](q, q_shared, k, v, logits, top_k,
                                                             shared_kv, causal, scale)
    return concat, wsum * 0.5, shared, idx, gate


def _active_no_shared(g, top_k, shared=1):
    return g * top_k


MUTATIONS = {
    "replicate_kv/strided": ("replicate_kv", _tile_kv),
    "scores/unscaled": ("scores", _scores_unscaled),
    "scores/transposed": ("scores", _scores_transposed),
    "causal_mask/strict": ("causal_mask", _mask_strict),
    "causal_mask/future": ("causal_mask", _mask_future),
    "softmax/axis": ("softmax", _softmax_axis),
    "softmax/sign": ("softmax", _softmax_sign),
    "softmax/unnormalised": ("softmax", _softmax_unnormalised),
    "gqa_ref_row/off_by_one": ("gqa_ref_row", _row_off_by_one),
    "decode/short_by_one": ("gqa_decode_ref", _decode_short),
    "topk/ties_high": ("gqe_topk_ref", _topk_ties_high),
    "topk/gate_unrenormalised": ("gqe_topk_ref", _topk_gate_unrenormalised),
    "gqe/unselected_not_zero": ("gqe_ref", _gqe_no_zero),
    "gqe/gate_dropped": ("gqe_ref", _gqe_no_gate),
    "gqe_decode/gate_dropped": ("gqe_decode_ref", _gqe_decode_no_gate),
    "gqe_decode/unselected_not_zero": ("gqe_decode_ref", _gqe_decode_no_zero),
    "gqe_router/dropped_feature": ("gqe_router_ref", _router_dropped_feature),
    "gqe_build/wrong_shared_kv": ("gqe_build_ref", _build_wrong_shared_kv),
    "gqe_build/wsum_scaled": ("gqe_build_ref", _build_wsum_unrenormalised),
    "kv_cache_bytes/no_factor_two": ("kv_cache_bytes", _kv_bytes_no_two),
    "kv_head_of/strided": ("kv_head_of", _kv_head_strided),
    "active_heads/no_shared": ("gqe_active_query_heads", _active_no_shared),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as exc:  # an exception or a failed assertion counts
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
    assert caught, f"no pin caught mutation {name}"
