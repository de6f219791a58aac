"""CPU reference (oracle) for grouped-query attention and grouped query experts.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module. The HIP library never calls it and shares
no code with it; it exists to decide, element by element, whether the GPU path
computes the right thing.

Everything is plain NumPy in float64. Inputs (float32 or bfloat16 values that
were handed to the GPU) are upcast losslessly and no intermediate is rounded.
Each step is written as the pages define it, without blocking, fusion or
reordering:

* GQA (ml-canon "56 GQA / MQA", section on the PyTorch GQA function; IBM Think
  "What is grouped query attention (GQA)?", discussion of scaled dot-product
  attention): the g key/value heads are replicated explicitly so that each of
  the h query heads sees its group's head, then scores = q k^T / sqrt(d),
  a softmax over keys, and the probability-weighted sum of value rows.
* The causal (autoregressive) mask: a query at position t only sees key
  positions 0..t (IBM Think page, on autoregressive decoders attending to
  previous tokens).
* Decode over a KV cache (aiunderstanding.org "Attention aux requetes
  groupees", section "Plongee profonde"): one new query per sequence attends
  to every cached key of its sequence.
* GQE routing (gist.science explainer of "Grouped Query Experts: Mixture-of-
  Experts on GQA Self-Attention", section "Architecture et Routage"): for each
  token a router keeps k query-head experts inside every KV group, the KV path
  stays dense, and the selected outputs are weighted by the router
  probabilities renormalised over the k selected experts.
* The KV-cache size law (ml-canon page, section on where the KV-cache saving
  comes from): bytes grow as 2 * L * n_kv * d_h * T.

Readings where the pages are silent (all listed in the design notes):
contiguous head-to-group map (head i uses KV head i // (h/g)); causal mask
aligned at the top-left with the diagonal visible; stable softmax by row-max
subtraction; router ties go to the lower head index, and the k indices are
returned in rank order; unselected heads output zero.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "kv_head_of",
    "replicate_kv",
    "scores",
    "causal_mask",
    "softmax",
    "gqa_ref",
    "gqa_ref_row",
    "gqa_decode_ref",
    "gqe_topk_ref",
    "gqe_ref",
    "gqe_decode_ref",
    "gqe_router_ref",
    "gqe_build_ref",
    "kv_cache_bytes",
    "gqe_active_query_heads",
]


def _f64(x) -> np.ndarray:
    """Lossless upcast of a NumPy array or a torch tensor to float64."""
    if hasattr(x, "detach"):  # torch tensor, possibly bfloat16
        x = x.detach().to("cpu")
        import torch  # local: only needed when torch tensors are handed in

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(i: int, h: int, g: int) -> int:
    """KV head used by query head ``i``: contiguous blocks of h/g query heads.

    ml-canon page, PyTorch GQA function (repeat-interleave along the head
    axis); freenetmedia "Grouped-Query Attention", section "Jak dzialaja ...":
    with 8 query heads in 2 groups, heads 0-3 share the first K/V set and heads
    4-7 the second.
    """
    if h % g:
        raise ValueError(f"g={g} must divide h={h}")
    return i // (h // g)


def replicate_kv(x: np.ndarray, h: int) -> np.ndarray:
    """[B,g,T,d] -> [B,h,T,d], each KV head repeated h/g times in place
    (the explicit replication of the ml-canon GQA function)."""
    g = x.shape[1]
    if h % g:
        raise ValueError(f"g={g} must divide h={h}")
    return np.repeat(x, h // g, axis=1)


def scores(q: np.ndarray, k_rep: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot products q k^T * scale, [..., Tq, Tk] (IBM Think page,
    scaled dot-product attention with factor 1/sqrt(d_k))."""
    return np.matmul(q, np.swapaxes(k_rep, -1, -2)) * scale


def causal_mask(Tq: int, Tk: int) -> np.ndarray:
    """Boolean [Tq, Tk], True where key j is visible to query t (j <= t)."""
    t = np.arange(Tq)[:, None]
    j = np.arange(Tk)[None, :]
    return j <= t


def softmax(s: np.ndarray, visible: np.ndarray | None = None) -> np.ndarray:
    """Softmax over the last axis (IBM Think page: weights in [0, 1] that sum
    to one). Masked entries get weight 0; the row max is subtracted first,
    which changes no exact value."""
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    den = np.sum(e, axis=-1, keepdims=True)
    return np.divide(e, den, out=np.zeros_like(e), where=den > 0)


def gqa_ref(q, k, v, causal: bool = True, scale: float | None = None,
            return_probs: bool = False):
    """GQA prefill. q [B,h,T,d], k/v [B,g,T,d] -> out [B,h,T,d] (float64).

    Follows the ml-canon GQA function step by step (replicate KV, scores,
    softmax, weighted sum of V) and adds the causal mask. One batch element at
    a time bounds memory. With ``return_probs`` also returns the row sums of
    the attention weights, [B,h,T].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, h, T, d = q.shape
    if k.shape[0] != B or k.shape[2:] != (T, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = causal_mask(T, T) if causal else None
    out = np.empty((B, h, T, d))
    sums = np.empty((B, h, T)) if return_probs else None
    for b in range(B):
        kr = replicate_kv(k[b:b + 1], h)[0]
        vr = replicate_kv(v[b:b + 1], h)[0]
        p = softmax(scores(q[b], kr, scale), vis)
        out[b] = np.matmul(p, vr)
        if return_probs:
            sums[b] = p.sum(axis=-1)
    return (out, sums) if return_probs else out


def gqa_ref_row(q, k, v, b: int, i: int, t: int, causal: bool = True,
                scale: float | None = None) -> np.ndarray:
    """One output row out[b, i, t, :] of :func:`gqa_ref`, computed on its own
    (for sampled checks at sizes where the whole output is too costly)."""
    d = q.shape[-1]
    h, g = q.shape[1], k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kv = kv_head_of(i, h, g)
    n = t + 1 if causal else k.shape[2]
    qr = _f64(q[b, i, t])
    kr = _f64(k[b, kv, :n])
    vr = _f64(v[b, kv, :n])
    p = softmax(kr @ qr * scale)
    return p @ vr


def gqa_decode_ref(q, k_cache, v_cache, lens, scale: float | None = None):
    """Decode step. q [B,h,d], caches [B,g,T_max,d], lens [B] -> out [B,h,d].

    The new token's query attends to every cached position below lens[b]
    (the cache already holds the new token's key and value); positions at or
    beyond lens[b] are never read. lens[b] = 0 gives a zero row.
    """
    q = _f64(q)
    B, h, d = q.shape
    g = k_cache.shape[1]
    lens = np.asarray(lens.cpu() if hasattr(lens, "cpu") else lens).astype(np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, h, d))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        kr = replicate_kv(_f64(k_cache[b:b + 1, :, :n]), h)[0]   # [h,n,d]
        vr = replicate_kv(_f64(v_cache[b:b + 1, :, :n]), h)[0]
        s = scores(q[b][:, None, :], kr, scale)                   # [h,1,n]
        out[b] = np.matmul(softmax(s), vr)[:, 0, :]
    return out


def gqe_topk_ref(logits, g: int, top_k: int):
    """Router selection per (token, KV group).

    logits [B,T,h] (float32 values) -> idx [B,T,g,k] int32 global head indices
    in rank order and gate [B,T,g,k] float64.

    gist.science GQE explainer, section "Architecture et Routage": within each
    group of h/g query-head experts the router keeps k; the selected outputs
    are combined with the router probabilities renormalised over the k kept.
    Order: higher logit first, equal logits by lower head index. The raw
    float32 logits are compared (the upcast to float64 keeps order and ties).
    Router probabilities are the softmax over the group's logits; the gate is
    that probability divided by the sum over the selected experts.
    """
    lg = _f64(logits)
    B, T, h = lg.shape
    r = h // g
    if h % g or not 1 <= top_k <= r:
        raise ValueError("need g | h and 1 <= top_k <= h/g")
    ell = lg.reshape(B, T, g, r)                       # the group's r expert logits
    expert = np.broadcast_to(np.arange(r), ell.shape)
    # Rank order: sort by the key (-logit, expert); np.lexsort takes the primary
    # key last. -0.0 and +0.0 compare equal, so they tie and go by expert index.
    order = np.lexsort((expert, -ell), axis=-1)
    sel = order[..., :top_k]                           # [B,T,g,k] experts in rank order
    prob = np.exp(ell - ell.max(axis=-1, keepdims=True))
    prob /= prob.sum(axis=-1, keepdims=True)           # router probabilities in the group
    kept = np.take_along_axis(prob, sel, axis=-1)
    gate = kept / kept.sum(axis=-1, keepdims=True)     # renormalised over the kept
    idx = (sel + (np.arange(g) * r)[None, None, :, None]).astype(np.int32)
    return idx, gate


def gqe_ref(q, k, v, logits, top_k: int, causal: bool = True,
            scale: float | None = None):
    """GQE routed prefill -> (out [B,h,T,d] float64, idx, gate).

    The keys and values stay dense (every selected row attends to all visible
    keys of its group), so a selected head's row equals the dense GQA row,
    multiplied by its gate; the rows of heads the router did not select are 0.
    """
    g = k.shape[1]
    idx, gate = gqe_topk_ref(logits, g, top_k)
    dense = gqa_ref(q, k, v, causal=causal, scale=scale)
    out = np.zeros_like(dense)
    B, T = idx.shape[0], idx.shape[1]
    for b in range(B):
        for t in range(T):
            for gam in range(g):
                for j in range(top_k):
                    i = int(idx[b, t, gam, j])
                    out[b, i, t] = gate[b, t, gam, j] * dense[b, i, t]
    return out, idx, gate


def gqe_decode_ref(q, k_cache, v_cache, lens, logits, top_k: int,
                   scale: float | None = None):
    """GQE routed decode step -> (out [B,h,d] float64, idx [B,g,k], gate [B,g,k]).

    One new token per sequence. The router keeps top_k of the h/g query-head
    experts of every KV group for that token (gist.science GQE explainer,
    section "Architecture et Routage"); the K/V cache stays dense, so a kept
    head attends to every cached position below lens[b] of its group exactly
    as in plain decode, and its row is multiplied by its gate. Rows of heads
    the router did not keep are 0, and so is every row of a sequence with no
    cached keys. logits [B,h] holds the router's score of every head for the
    new token.
    """
    q = _f64(q)
    B, h, d = q.shape
    g = k_cache.shape[1]
    idx, gate = gqe_topk_ref(_f64(logits).reshape(B, 1, h), g, top_k)
    idx, gate = idx[:, 0], gate[:, 0]                  # [B,g,k]
    dense = gqa_decode_ref(q, k_cache, v_cache, lens, scale)
    out = np.zeros_like(dense)
    for b in range(B):
        for gam in range(g):
            for j in range(top_k):
                i = int(idx[b, gam, j])
                out[b, i] = gate[b, gam, j] * dense[b, i]
    return out, idx, gate


def gqe_router_ref(x, w_r, g: int, top_k: int):
    """GQE router: score every query-head expert for every token, then keep
    top_k per KV group -> (logits [N,h] float64, bound [N,h], idx, gate).

    x [N, d_model] holds the tokens' input vectors and w_r [h, d_model] one
    row of router weights per query head; logits = x @ w_r^T. The pages say
    the router examines each token and picks the experts of each group
    (gist.science GQE explainer, sections "Architecture et Routage" and the
    router analogy before it) without fixing its form; a linear map of the
    token, as for the Q/K/V projections of the attention layer (IBM Think
    page, the weight matrices W_Q, W_K, W_V), is the reading taken here.

    bound is the classical worst-case error of a float32 dot product of
    length n in any summation order: n * 2^-24 * sum_i |x_i w_i| (a GPU that
    accumulates in fp32 stays within it). idx and gate are gqe_topk_ref of
    the logits, laid out [N, g, k].
    """
    xf, wf = _f64(x), _f64(w_r)
    if xf.ndim != 2 or wf.ndim != 2 or xf.shape[1] != wf.shape[1]:
        raise ValueError("need x [N, d_model] and w_r [h, d_model]")
    n_tok, dm = xf.shape
    h = wf.shape[0]
    logits = xf @ wf.T
    bound = dm * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T)
    idx, gate = gqe_topk_ref(logits.reshape(1, n_tok, h), g, top_k)
    return logits, bound, idx[0], gate[0]


def gqe_build_ref(q, q_shared, k, v, logits, top_k: int, shared_kv: int = 0,
                  causal: bool = True, scale: float | None = None):
    """GQE layer output as the pages build it -> (concat, wsum, shared, idx, gate).

    gist.science GQE explainer, section "Architecture et Routage", output
    construction: (1) the outputs of the k experts the router kept in each
    group are concatenated (hard concatenation); (2) a weighted sum of those
    outputs with the router probabilities renormalised over the k kept forms
    an extra slot; (3) one more attention head, shared and always active, is
    computed for every token. With 16 query heads in 8 groups and k = 1 that
    is 8 routed + 1 shared = 9 query-attention computations out of 16, so the
    shared head is one attention over one KV head.

    Readings (the pages leave them open): the shared head reads KV head
    `shared_kv`; its query q_shared [B,T,d] is an input of its own; the slots
    are laid out token-major: concat [B,T,g,k,d] (kept experts in rank order,
    outputs not gated), wsum [B,T,g,d] (one slot per group), shared [B,T,d].
    """
    q, qs = _f64(q), _f64(q_shared)
    B, h, T, d = q.shape
    g = k.shape[1]
    idx, gate = gqe_topk_ref(logits, g, top_k)               # [B,T,g,k]
    dense = gqa_ref(q, k, v, causal=causal, scale=scale)      # [B,h,T,d]
    concat = np.empty((B, T, g, top_k, d))
    for b in range(B):
        for t in range(T):
            concat[b, t] = dense[b, idx[b, t], t]             # rows of the kept heads
    wsum = np.einsum("btgk,btgkd->btgd", gate, concat)
    kv = slice(shared_kv, shared_kv + 1)
    shared = gqa_ref(qs[:, None], _f64(k)[:, kv], _f64(v)[:, kv], causal=causal, scale=scale)[:, 0]
    return concat, wsum, shared, idx, gate


def kv_cache_bytes(B: int, n_kv: int, T: int, d: int, elt_bytes: int,
                   layers: int = 1) -> int:
    """KV-cache size: keys and values for each layer, KV head and token
    (ml-canon page, section on where the KV-cache saving comes from)."""
    return 2 * layers * n_kv * d * T * elt_bytes * B


def gqe_active_query_heads(g: int, top_k: int, shared: int = 1) -> int:
    """Query-attention computations per token in GQE: k routed experts in each
    of the g groups, plus the always-active shared head(s) (gist.science GQE
    explainer, section "Resultats Experimentaux")."""
    return g * top_k + shared
