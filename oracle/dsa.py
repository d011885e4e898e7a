"""Plain CPU oracle for DeepSeek Sparse Attention (DSA): index scores, top-k
token selection and sparse MLA attention in MQA mode.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
under ``oracle/``.  The product path (the HIP library and its Python binding)
never routes through this code, and this code imports nothing from it.

Everything is computed in float64, one query row at a time, straight from the
definitions on the pages:

* index score (page "Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture:
  DSA (§2.1)", the index-score formula):
      I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
  with one indexer key k[s] per token shared by all indexer heads j (the
  formula puts no head index on k);
* token selection (same section, the attention formula): query t attends to
  the latent entries c_s whose score is among the top-k of row I[t,:]; the
  candidates are the earlier tokens and t itself ("DeepSeek V3.2: Sparse
  Attention and Reinforcement Learning Updates", Summary: the selector keeps
  only high-scoring past tokens);
* sparse attention in MLA's MQA mode (page 1, "DSA under MLA (MQA Mode)"):
  one latent vector per selected token is shared by every query head; the key
  is the whole latent+rope vector, the value is its leading d_v latent part.

Readings of points the pages leave open:
inclusive causal boundary s <= q_offset + t; fewer than k candidates select
all of them and pad with -1; ties go to the lower index; indices come out
ascending; NaN ranks below every number; -0 equals +0.
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import dequantize


# --------------------------------------------------------------------------
# Lightning indexer


def _as_f64_tokens(x, scale):
    """Indexer operand as float64: FP8 codes times per-row scale, or raw floats."""
    x = np.asarray(x)
    if x.dtype == np.uint8:
        if scale is None:
            raise ValueError("FP8 codes need a scale")
        return dequantize(x, scale)
    return x.astype(np.float64)


def index_scores_row(q_row, w_row, K, n_cand):
    """One row of the index-score matrix.

    q_row : [H_I, d_I] float64 indexer queries of token t (one per head j)
    w_row : [H_I]      float64 head weights w[t,j]
    K     : [N, d_I]   float64 indexer keys k[s]
    n_cand: number of candidates, q_offset + t + 1 capped at N

    Returns I[t, 0:N] with -inf at s >= n_cand (outside the causal set).
    Follows the index-score formula of page 1, section 2 "Architecture: DSA
    (§2.1)": the sum over heads of w[t,j] * ReLU(q[t,j] . k[s]).
    """
    N = K.shape[0]
    out = np.full(N, -np.inf)
    if n_cand <= 0:
        return out
    D = q_row @ K[:n_cand].T  # [H_I, n_cand]; q[t,j] . k[s]
    out[:n_cand] = w_row @ np.maximum(D, 0.0)  # sum_j w[t,j] * ReLU(.)
    return out


def index_scores(q_idx, k_idx, w, q_offset, q_scale=None, k_scale=None, rows=None):
    """Index scores I[b,t,s] for the query rows ``rows`` (default: all).

    q_idx [B,T,H_I,d_I] (uint8 e4m3fn codes with q_scale [B,T,H_I], or floats),
    k_idx [B,N,d_I]     (uint8 codes with k_scale [B,N], or floats),
    w     [B,T,H_I]     float weights.
    Query t sits at absolute position q_offset + t and sees keys 0..q_offset+t.
    Returns float64 [len(rows), N] when ``rows`` is a list of (b, t), else
    [B, T, N].
    """
    q_idx = np.asarray(q_idx)
    B, T = q_idx.shape[:2]
    N = np.asarray(k_idx).shape[1]
    w = np.asarray(w, dtype=np.float64)
    full = rows is None
    if full:
        rows = [(b, t) for b in range(B) for t in range(T)]
    out = np.empty((len(rows), N))
    keys = {}
    for r, (b, t) in enumerate(rows):
        if b not in keys:
            keys = {b: _as_f64_tokens(np.asarray(k_idx)[b],
                                      None if k_scale is None else np.asarray(k_scale)[b])}
        qs = None if q_scale is None else np.asarray(q_scale)[b, t]
        q_row = _as_f64_tokens(q_idx[b, t], qs)
        n_cand = min(N, q_offset + t + 1)
        out[r] = index_scores_row(q_row, w[b, t], keys[b], n_cand)
    return out.reshape(B, T, N) if full else out


# --------------------------------------------------------------------------
# Token selector


def topk_select_row(scores_row, k, n_cand):
    """Top-k token selection over the candidates 0..n_cand-1 of one score row.

    Page 1, section 2 "Architecture: DSA (§2.1)": query t keeps the tokens s
    whose score I[t,s] is among the top-k of I[t,:].  With fewer than k
    candidates all of them are kept.  Among equal scores the lower index is
    kept; NaN scores rank below every number.  The kept indices are returned
    in ascending order and padded with -1 to length k.
    """
    v = np.asarray(scores_row, dtype=np.float64)[:n_cand]
    n = min(k, n_cand)
    out = np.full(k, -1, dtype=np.int64)
    if n <= 0:
        return out
    finite_or_inf = ~np.isnan(v)
    real = np.flatnonzero(finite_or_inf)
    if real.size <= n:
        # every non-NaN candidate is kept; the rest are the lowest-index NaNs
        nan_idx = np.flatnonzero(~finite_or_inf)[: n - real.size]
        keep = np.sort(np.concatenate([real, nan_idx]))
    else:
        vals = v[real]
        # threshold: the n-th largest value
        thr = np.partition(vals, vals.size - n)[vals.size - n]
        above = real[vals > thr]
        ties = real[vals == thr]  # ascending index order
        keep = np.sort(np.concatenate([above, ties[: n - above.size]]))
    out[: keep.size] = keep
    return out


def topk_select(scores, k, q_offset, rows=None):
    """Top-k selection for every row of a [B,T,N] score tensor (or ``rows``).

    ``scores`` may also be a [len(rows), N] array when ``rows`` is given; row
    r then belongs to query (b, t) = rows[r].
    """
    scores = np.asarray(scores)
    if rows is None:
        B, T, N = scores.shape
        out = np.empty((B, T, k), dtype=np.int64)
        for b in range(B):
            for t in range(T):
                out[b, t] = topk_select_row(scores[b, t], k, min(N, q_offset + t + 1))
        return out
    N = scores.shape[-1]
    out = np.empty((len(rows), k), dtype=np.int64)
    for r, (b, t) in enumerate(rows):
        row = scores[r] if scores.ndim == 2 else scores[b, t]
        out[r] = topk_select_row(row, k, min(N, q_offset + t + 1))
    return out


# --------------------------------------------------------------------------
# Sparse MLA attention, MQA mode


def sparse_mqa_attention_row(q_row, kv, idx_row, d_v, sm_scale):
    """Attention of one query token over its selected latent entries.

    q_row  : [H, d_qk] per-head queries in the latent(+rope) space
    kv     : [N, d_qk] latent entries c_s, shared by all H heads (MQA mode)
    idx_row: [k] selected token indices, -1 (or anything outside [0, N)) is an
             empty slot; duplicates count as often as they appear
    Returns (o [H, d_v], lse [H]).  With no valid index o = 0, lse = -inf.

    Page 1, section 2: u_t = Attn(h_t, {c_s : I[t,s] in Top-k(I[t,:])}), with
    "DSA under MLA (MQA Mode)": every head scores the same latent vector c_s;
    the value is the leading d_v (latent) part of c_s.
    """
    N = kv.shape[0]
    idx_row = np.asarray(idx_row)
    sel = idx_row[(idx_row >= 0) & (idx_row < N)]
    H = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    C = np.asarray(kv[sel], dtype=np.float64)    # [k', d_qk], exact widening
    z = sm_scale * (q_row @ C.T)                 # [H, k'] logits
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ C[:, :d_v]) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_mqa_attention(q, kv, idx, d_v, sm_scale, rows=None):
    """Sparse MQA attention for all query rows (or the (b, t) list ``rows``).

    q [B,T,H,d_qk], kv [B,N,d_qk], idx [B,T,k] (or [len(rows), k] with rows).
    Inputs are converted to float64 exactly (bf16 and fp32 both embed).
    Returns (out, lse): [B,T,H,d_v], [B,T,H] or [R,H,d_v], [R,H].
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    idx = np.asarray(idx)
    B, T, H, _ = q.shape
    full = rows is None
    if full:
        rows = [(b, t) for b in range(B) for t in range(T)]
    out = np.empty((len(rows), H, d_v))
    lse = np.empty((len(rows), H))
    for r, (b, t) in enumerate(rows):
        irow = idx[b, t] if (full or idx.ndim == 3) else idx[r]
        out[r], lse[r] = sparse_mqa_attention_row(
            q[b, t].astype(np.float64), kv[b], irow, d_v, sm_scale)
    if full:
        return out.reshape(B, T, H, d_v), lse.reshape(B, T, H)
    return out, lse


# --------------------------------------------------------------------------
# Sparse MLA attention, MHA mode
# --------------------------------------------------------------------------
# The DeepSeek-V3.2 paper's section list (page "aipaper.jasonlin.tech",
# "Sections", "Appendix A MHA and MQA Modes of MLA") names two modes of MLA;
# DSA runs in MQA mode ("Paper Breakdown: DeepSeek-V3.2", section 2 "DSA
# under MLA (MQA Mode)").  The appendix body is not on the pages, so MHA mode
# is read as plain multi-head attention over per-head keys and values
# up-projected from the same latent entries:
#     key of token s for head h   = [W_UK[h] c_s[:d_c] ; c_s[d_c:]]
#     value of token s for head h = W_UV[h] c_s[:d_c]
# (the rope part c_s[d_c:] is one key part shared by all heads), with per-head
# queries [q_nope ; q_rope].  W_UK is [H, d_n, d_c] and W_UV [H, d_vh, d_c].


def mha_keys_values(kv, w_uk, w_uv, d_c):
    """Per-head keys [N, H, d_n + d_r] and values [N, H, d_vh] of MHA mode
    from latent entries kv [N, d_c + d_r] (float64 results)."""
    C = np.asarray(kv, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    N = C.shape[0]
    H = w_uk.shape[0]
    d_n, d_vh = w_uk.shape[1], w_uv.shape[1]
    K = np.empty((N, H, d_n + C.shape[1] - d_c))
    V = np.empty((N, H, d_vh))
    for h in range(H):
        K[:, h, :d_n] = C[:, :d_c] @ w_uk[h].T   # W_UK[h] c_s[:d_c] for every s
        K[:, h, d_n:] = C[:, d_c:]               # the shared rope part
        V[:, h] = C[:, :d_c] @ w_uv[h].T         # W_UV[h] c_s[:d_c]
    return K, V


def sparse_mha_attention_row(q_row, K, V, idx_row, sm_scale):
    """One query token's attention in MHA mode: head h attends over its own
    keys K[s, h] and values V[s, h] of the selected tokens s.

    q_row [H, d_n + d_r], K [N, H, d_n + d_r], V [N, H, d_vh], idx_row [k]
    (-1 or anything outside [0, N) is an empty slot; duplicates count per
    slot).  Returns (o [H, d_vh], lse [H]); with no valid index o = 0 and
    lse = -inf.
    """
    N, H = K.shape[0], K.shape[1]
    idx_row = np.asarray(idx_row)
    sel = idx_row[(idx_row >= 0) & (idx_row < N)]
    if sel.size == 0:
        return np.zeros((H, V.shape[2])), np.full(H, -np.inf)
    o = np.empty((H, V.shape[2]))
    lse = np.empty(H)
    for h in range(H):
        z = sm_scale * (K[sel, h] @ np.asarray(q_row[h], dtype=np.float64))  # [k']
        m = z.max()
        p = np.exp(z - m)
        l = p.sum()
        o[h] = (p @ V[sel, h]) / l
        lse[h] = m + math.log(l)
    return o, lse


def sparse_mha_attention(q, kv, w_uk, w_uv, idx, sm_scale, d_c, rows=None):
    """Sparse MLA attention in MHA mode for all query rows (or ``rows``).

    q [B,T,H,d_n+d_r] per-head queries, kv [B,N,d_c+d_r] latent entries,
    w_uk [H,d_n,d_c], w_uv [H,d_vh,d_c], idx [B,T,k] (or [len(rows), k]).
    Returns (out, lse): [B,T,H,d_vh], [B,T,H] or [R,H,d_vh], [R,H].
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    idx = np.asarray(idx)
    B, T, H, _ = q.shape
    d_vh = np.asarray(w_uv).shape[1]
    full = rows is None
    if full:
        rows = [(b, t) for b in range(B) for t in range(T)]
    out = np.empty((len(rows), H, d_vh))
    lse = np.empty((len(rows), H))
    kvs = {}
    for r, (b, t) in enumerate(rows):
        if b not in kvs:
            kvs = {b: mha_keys_values(kv[b], w_uk, w_uv, d_c)}
        K, V = kvs[b]
        irow = idx[b, t] if (full or idx.ndim == 3) else idx[r]
        out[r], lse[r] = sparse_mha_attention_row(q[b, t], K, V, irow, sm_scale)
    if full:
        return out.reshape(B, T, H, d_vh), lse.reshape(B, T, H)
    return out, lse


# --------------------------------------------------------------------------
# Sparse attention backward (the sparse training stage)
# --------------------------------------------------------------------------
# "Paper Breakdown: DeepSeek-V3.2", section 2, "Continued Pre-Training
# (§2.1.1)": in the sparse training stage the main model is trained through
# the sparse attention (only the selected entries c_s take part), so the
# gradients of u_t = Attn(h_t, {c_s : selected}) with respect to the query
# heads and to the selected latent entries are needed.  They follow from the
# chain rule through the forward above; with z[h,i] = scale * q[h] . c_i,
# P = softmax_i(z[h,:]) over the valid slots and o[h] = sum_i P[h,i] c_i[:d_v]:
#     dP[h,i] = do[h] . c_i[:d_v]
#     dz[h,i] = P[h,i] * (dP[h,i] - sum_j P[h,j] dP[h,j])
#     dq[h]   = scale * sum_i dz[h,i] c_i
#     dc_i    = scale * sum_h dz[h,i] q[h]  (+ sum_h P[h,i] do[h] on [:d_v])
# A slot outside [0, N) contributes nothing; a token selected in several
# slots receives the sum of their contributions.

def sparse_mqa_attention_bwd_row(q_row, kv, idx_row, do_row, d_v, sm_scale):
    """Gradients of one query token's sparse MQA attention.

    q_row [H, d_qk], kv [N, d_qk], idx_row [k], do_row [H, d_v] (the
    gradient of the loss with respect to the row's output o).  Returns
    (dq [H, d_qk], dkv [N, d_qk]) in float64; dkv is zero outside the
    selected rows.
    """
    N = kv.shape[0]
    q_row = np.asarray(q_row, dtype=np.float64)
    do_row = np.asarray(do_row, dtype=np.float64)
    idx_row = np.asarray(idx_row)
    sel = idx_row[(idx_row >= 0) & (idx_row < N)]
    H, d_qk = q_row.shape
    dkv = np.zeros((N, d_qk))
    if sel.size == 0:
        return np.zeros((H, d_qk)), dkv
    C = np.asarray(kv[sel], dtype=np.float64)         # [k', d_qk]
    z = sm_scale * (q_row @ C.T)                      # [H, k']
    P = np.exp(z - z.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = do_row @ C[:, :d_v].T                        # [H, k']
    dz = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    dq = sm_scale * (dz @ C)
    dC = sm_scale * (dz.T @ q_row)                    # [k', d_qk]
    dC[:, :d_v] += P.T @ do_row
    np.add.at(dkv, sel, dC)
    return dq, dkv


def sparse_mqa_attention_bwd(q, kv, idx, do, d_v, sm_scale):
    """Gradients of sparse MQA attention for a whole batch.

    q [B,T,H,d_qk], kv [B,N,d_qk], idx [B,T,k], do [B,T,H,d_v].  Returns
    (dq [B,T,H,d_qk], dkv [B,N,d_qk]) in float64; dkv sums the contributions
    of every query row of the sequence.
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    idx = np.asarray(idx)
    do = np.asarray(do)
    B, T, H, d_qk = q.shape
    dq = np.zeros((B, T, H, d_qk))
    dkv = np.zeros((B, kv.shape[1], d_qk))
    for b in range(B):
        for t in range(T):
            dq[b, t], g = sparse_mqa_attention_bwd_row(q[b, t], kv[b], idx[b, t], do[b, t],
                                                       d_v, sm_scale)
            dkv[b] += g
    return dq, dkv


# --------------------------------------------------------------------------
# The whole path


def dsa_forward(q_idx, k_idx, w, q, kv, *, k, q_offset, d_v, sm_scale,
                q_scale=None, k_scale=None, rows=None):
    """Index scores -> top-k selection -> sparse MQA attention.

    Page 1, section 2 "Architecture: DSA (§2.1)": the indexer scores every
    earlier token, the selector keeps the top-k per query, and attention runs
    over the kept latent entries only.  Returns a dict with ``scores``,
    ``idx``, ``out`` and ``lse`` (restricted to ``rows`` when given).
    """
    B, T = np.asarray(q_idx).shape[:2]
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(T)]
    scores = index_scores(q_idx, k_idx, w, q_offset, q_scale=q_scale,
                          k_scale=k_scale, rows=rows)
    idx = topk_select(scores, k, q_offset, rows=rows)
    out, lse = sparse_mqa_attention(q, kv, idx, d_v, sm_scale, rows=rows)
    return {"scores": scores, "idx": idx, "out": out, "lse": lse, "rows": rows}


# --------------------------------------------------------------------------
# Cache append (the step before the path at decode)
# --------------------------------------------------------------------------
def cache_append(k_new, kv_new, k_cache, k_cache_scale, kv_cache, pos):
    """Append new tokens to a sequence batch's caches; returns updated copies.

    The indexer keys are kept per token in FP8 and the latent entries c_s in
    the attention dtype ("Paper Breakdown: DeepSeek-V3.2", section 2
    "Architecture: DSA (§2.1)": FP8 indexer, and the latent entry c_s each
    selected token contributes).  New token t of sequence b goes to row
    pos[b] + t: its indexer key row k_new[b,t] (float32) is quantised with
    quantize_rows into k_cache / k_cache_scale, and its latent row
    kv_new[b,t] is copied into kv_cache unchanged.  Rows whose position falls
    outside [0, N) are dropped; every other cache row keeps its contents.
    """
    from .fp8 import quantize_rows

    k_new = np.asarray(k_new, dtype=np.float32)
    kc = np.array(k_cache, copy=True)
    ks = np.array(k_cache_scale, copy=True)
    kvc = np.array(kv_cache, copy=True)
    B, T, _ = k_new.shape
    N = kc.shape[1]
    for b in range(B):
        for t in range(T):
            p = int(pos[b]) + t
            if p < 0 or p >= N:
                continue
            codes, scale = quantize_rows(k_new[b, t])
            kc[b, p] = codes
            ks[b, p] = scale
            kvc[b, p] = kv_new[b, t]
    return kc, ks, kvc


# --------------------------------------------------------------------------
# Indexer alignment loss (continued pre-training)
# --------------------------------------------------------------------------
# "Paper Breakdown: DeepSeek-V3.2", section 2, "Continued Pre-Training
# (§2.1.1)": the dense warm-up trains the indexer with
#     L^I = sum_t KL(p_{t,:} || Softmax(I_{t,:})),
# and sparse training keeps the KL objective on the selected set S_t only.
# Readings: the softmax runs over the row's causal candidates (dense) or over
# S_t (sparse); the target p is taken as given (no renormalisation), so the
# loss of a row is sum_s p_s (log p_s - log q_s) over the entries with
# p_s > 0 (0 log 0 = 0) and its gradient with respect to I_s is
# P q_s - p_s with P = sum_s p_s (q_s - p_s for a distribution).

def _kl_terms(I, p):
    I = np.asarray(I, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    if I.size == 0:
        return 0.0, np.zeros(0)
    m = np.max(I)
    lse = m + math.log(np.sum(np.exp(I - m)))
    logq = I - lse
    q = np.exp(logq)
    pos = p > 0
    loss = float(np.sum(p[pos] * (np.log(p[pos]) - logq[pos])))
    grad = np.sum(p) * q - p
    return loss, grad


def indexer_kl_dense_row(I_row, p_row, n_cand):
    """Loss and gradient (w.r.t. the row's scores) of KL(p || softmax(I))
    over the causal candidates s < n_cand; the gradient is 0 elsewhere."""
    loss, g = _kl_terms(np.asarray(I_row)[:n_cand], np.asarray(p_row)[:n_cand])
    grad = np.zeros(len(I_row))
    grad[:n_cand] = g
    return loss, grad


def indexer_kl_sparse_row(I_row, idx_row, p_sel):
    """Loss and per-slot gradient of the KL restricted to the selected set:
    slot i holds token idx_row[i] with target p_sel[i]; slots whose index is
    outside [0, N) are skipped (gradient 0); duplicates count once per slot."""
    I_row = np.asarray(I_row, dtype=np.float64)
    idx_row = np.asarray(idx_row)
    ok = (idx_row >= 0) & (idx_row < I_row.size)
    loss, g = _kl_terms(I_row[idx_row[ok]], np.asarray(p_sel, dtype=np.float64)[ok])
    grad = np.zeros(idx_row.size)
    grad[ok] = g
    return loss, grad


def indexer_kl(scores, p, q_offset, idx=None):
    """Per-row losses [B,T] and gradients of the indexer KL objective.

    Dense (idx None): scores and p are [B,T,N]; row t's candidates are
    s <= q_offset + t; gradients [B,T,N].  Sparse: idx [B,T,k] and p [B,T,k]
    (the target of each selected slot); gradients [B,T,k]."""
    scores = np.asarray(scores, dtype=np.float64)
    B, T, N = scores.shape
    loss = np.zeros((B, T))
    if idx is None:
        grad = np.zeros((B, T, N))
        for b in range(B):
            for t in range(T):
                n_cand = min(N, q_offset + t + 1)
                loss[b, t], grad[b, t] = indexer_kl_dense_row(scores[b, t], p[b, t], n_cand)
    else:
        idx = np.asarray(idx)
        grad = np.zeros(idx.shape)
        for b in range(B):
            for t in range(T):
                loss[b, t], grad[b, t] = indexer_kl_sparse_row(scores[b, t], idx[b, t], p[b, t])
    return loss, grad
