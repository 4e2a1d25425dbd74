"""Phase-1 encoding, Phase-2 query attention and the exact LSE merge
(test infrastructure only).

Sources:
  * "Dropping the Anchor ..." Section 2 Method and Section 2.1: host i encodes
    [sink || summaries of earlier blocks || own block] with original position
    IDs and keeps only its own block's KV;
  * the same page, Section 2.2 Query phase: the query is broadcast, each host
    attends locally over its shard, and an online-softmax merge of the
    gathered partials gives exact attention over the retained shards;
  * the Star Attention review (arXiv 2411.17116): each host returns one
    partial output vector and one softmax statistic per token to the query
    host; the corrected merge weight is exp(s_h - s_global) applied to A_h.

Every output here is a definition written out: softmax attention over an
explicitly listed set of keys, in float64.  Scores are (q . k) / sqrt(d) on
the bf16 rotated operands; softmax subtracts the row maximum before exp.
Query head h reads KV head floor(h * Hkv / Hq) (groups of Hq / Hkv
consecutive query heads share a KV head).
"""
import numpy as np

from .bf16 import round_bf16
from .rope import rope


def rotate_bf16(x, pos, base):
    """bf16(RoPE(x, pos)): the rotated attention operand the bf16 model uses."""
    return round_bf16(rope(x, pos, base))


def attend(q_hat, k_hat, v):
    """Softmax attention of one query token over an explicit key list.

    q_hat [Hq][d], k_hat [n][Hkv][d], v [n][Hkv][d] -> (O [Hq][d], lse [Hq]),
    lse = natural-log sum of exp(score) over the n keys.
    """
    q_hat = np.asarray(q_hat, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v = np.asarray(v, np.float64)
    hq, d = q_hat.shape
    hkv = k_hat.shape[1]
    group = hq // hkv
    out = np.empty((hq, d), np.float64)
    lse = np.empty(hq, np.float64)
    for h in range(hq):
        g = h // group
        s = k_hat[:, g, :] @ q_hat[h] / np.sqrt(d)
        m = s.max()
        w = np.exp(s - m)
        out[h] = (w @ v[:, g, :]) / w.sum()
        lse[h] = m + np.log(w.sum())
    return out, lse


# ----------------------------------------------------------------- Phase 1
def phase1_key_positions(prefix_i, i, r, block_size):
    """Keys visible to row r of block i: the whole prefix (every prefix entry
    precedes the block in the concatenated input, so the causal mask keeps all
    of it) followed by the block's own rows 0..r."""
    own = np.arange(i * block_size, i * block_size + r + 1, dtype=np.int64)
    return np.concatenate([np.asarray(prefix_i, np.int64), own])


def phase1_rows(q, k_hat, v, prefixes, rows, block_size, base):
    """Phase-1 attention output of selected block rows.

    q      : indexable [L][Hq][d] pre-RoPE query values
    k_hat  : indexable [L][Hkv][d] rotated bf16 keys (see rotate_bf16)
    v      : indexable [L][Hkv][d] values
    prefixes: per-block prefix position lists (selection.prefix_positions)
    rows   : iterable of (block i, row r)
    returns O [len(rows)][Hq][d] float64
    """
    outs = []
    for (i, r) in rows:
        p = i * block_size + r
        keys = phase1_key_positions(prefixes[i], i, r, block_size)
        q_hat = rotate_bf16(np.asarray(q[np.array([p])], np.float64), np.array([p]), base)[0]
        o, _ = attend(q_hat, k_hat[keys], v[keys])
        outs.append(o)
    return np.stack(outs)


def phase1_rows_in_block(q, k_hat, v, prefix_i, i, rows, block_size, base):
    """Phase-1 output of several rows of one block: the definition of
    phase1_rows (row r sees every entry of prefix_i, then the block's own rows
    0..r), written as one masked softmax per head over the explicit key list
    [prefix_i || own rows 0..max(rows)], own row j hidden from row r when j > r.

    q, k_hat, v : indexable [L][H][d] as for phase1_rows
    rows        : row indices within block i
    returns O [len(rows)][Hq][d] float64
    """
    rows = np.asarray(rows, np.int64)
    lo = i * block_size
    r_max = int(rows.max())
    prefix_i = np.asarray(prefix_i, np.int64)
    keys = np.concatenate([prefix_i, np.arange(lo, lo + r_max + 1, dtype=np.int64)])
    kh = np.asarray(k_hat[keys], np.float64)
    vv = np.asarray(v[keys], np.float64)
    pos = lo + rows
    q_hat = rotate_bf16(np.asarray(q[pos], np.float64), pos, base)
    hq, d = q_hat.shape[1], q_hat.shape[2]
    group = hq // kh.shape[1]
    visible = np.ones((len(rows), len(keys)), bool)
    visible[:, len(prefix_i):] = np.arange(r_max + 1)[None, :] <= rows[:, None]
    out = np.empty((len(rows), hq, d))
    for h in range(hq):
        g = h // group
        s = np.where(visible, q_hat[:, h, :] @ kh[:, g, :].T / np.sqrt(d), -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ vv[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def phase1_block_dense(q, k_hat, v, prefix_i, i, block_size, base):
    """Twin formulation of Phase 1 for all rows of block i: one softmax over the
    whole preceding context with an additive bias, ln(multiplicity of the
    position in the prefix) on prefix positions, 0 on the block's own rows up
    to the diagonal and -inf everywhere else.  A key listed twice contributes
    exp(s + ln 2) = 2 exp(s), the same as two copies."""
    q = np.asarray(q, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v = np.asarray(v, np.float64)
    lo = i * block_size
    n_ctx = lo + block_size
    hq, d = q.shape[1], q.shape[2]
    hkv = k_hat.shape[1]
    group = hq // hkv
    counts = np.bincount(np.asarray(prefix_i, np.int64), minlength=n_ctx)[:n_ctx].astype(np.float64)
    bias = np.full((block_size, n_ctx), -np.inf)
    with np.errstate(divide="ignore"):
        bias[:, :lo] = np.log(counts[:lo])[None, :]
    own = np.tril(np.ones((block_size, block_size), bool))
    bias[:, lo:] = np.where(own, 0.0, -np.inf)
    pos = np.arange(lo, lo + block_size)
    q_hat = rotate_bf16(q[lo:lo + block_size], pos, base)
    out = np.empty((block_size, hq, d))
    for h in range(hq):
        g = h // group
        s = q_hat[:, h, :] @ k_hat[:n_ctx, g, :].T / np.sqrt(d) + bias
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ v[:n_ctx, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def prefix_rows(q, k_hat, v, prefix_last, rows, base):
    """Attention output of prefix rows, the states a next layer would need.
    Host i runs one forward pass over [prefix_i || B_i]; its prefix rows are
    queries too, each attending causally (by list index) to the prefix entries up
    to itself ("Dropping the Anchor ..." Section 2 and the Dutch technical
    summary's per-host input [S_sink || Sigma_0 || ... || Sigma_{i-1} || B_i]).
    Every prefix_i is a leading part of the last block's prefix, so one pass
    over prefix_last gives every host's prefix rows.

    q, k_hat, v : indexable [L][H][d] (q pre-RoPE, k_hat rotated bf16)
    prefix_last : positions of the last block's prefix (duplicates kept)
    rows        : list indices e; row e attends to prefix_last[0 .. e]
    returns O [len(rows)][Hq][d]
    """
    prefix_last = np.asarray(prefix_last, np.int64)
    outs = []
    for e in rows:
        keys = prefix_last[:e + 1]
        p = prefix_last[e]
        q_hat = rotate_bf16(np.asarray(q[np.array([p])], np.float64), np.array([p]), base)[0]
        o, _ = attend(q_hat, k_hat[keys], v[keys])
        outs.append(o)
    return np.stack(outs)


def prefix_rows_dense(q, k_hat, v, prefix_last, base):
    """Twin of prefix_rows for every row: one softmax per row over all context
    positions with bias ln(multiplicity of the position among entries 0..e) and
    -inf where the position does not occur."""
    q = np.asarray(q, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v = np.asarray(v, np.float64)
    prefix_last = np.asarray(prefix_last, np.int64)
    n_ctx = int(prefix_last.max()) + 1
    hq, d = q.shape[1], q.shape[2]
    group = hq // k_hat.shape[1]
    out = np.empty((len(prefix_last), hq, d))
    counts = np.zeros(n_ctx)
    for e, p in enumerate(prefix_last):
        counts[p] += 1
        with np.errstate(divide="ignore"):
            bias = np.log(counts)
        q_hat = rotate_bf16(q[np.array([p])], np.array([p]), base)[0]
        for h in range(hq):
            g = h // group
            s = k_hat[:n_ctx, g, :] @ q_hat[h] / np.sqrt(d) + bias
            m = s.max()
            w = np.exp(s - m)
            out[e, h] = w @ v[:n_ctx, g, :] / w.sum()
    return out


def retained_cache(k, v, n_blocks, block_size, base):
    """What each host keeps after Phase 1: its own block's rotated keys and its
    values, [N][Hkv][b][d] each.  Sink and summary entries are discarded."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    pos = np.arange(n_blocks * block_size)
    k_hat = rotate_bf16(k, pos, base)
    kc = k_hat.reshape(n_blocks, block_size, k.shape[1], k.shape[2]).transpose(0, 2, 1, 3)
    vc = v.reshape(n_blocks, block_size, v.shape[1], v.shape[2]).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(kc), np.ascontiguousarray(vc)


# ----------------------------------------------------------------- Phase 2
def _shard_attend(q_hat, k_hat, v, causal, offset=0):
    """All query tokens against one shard.  q_hat [Lq][Hq][d], k_hat/v
    [Hkv][n][d].  causal: query t sees shard keys 0..t+offset.
    -> O [Lq][Hq][d], lse [Lq][Hq]."""
    lq, hq, d = q_hat.shape
    hkv, n, _ = k_hat.shape
    group = hq // hkv
    out = np.empty((lq, hq, d))
    lse = np.empty((lq, hq))
    for h in range(hq):
        g = h // group
        s = q_hat[:, h, :] @ k_hat[g].T / np.sqrt(d)            # [Lq][n]
        if causal:
            s = np.where(np.arange(n)[None, :] <= np.arange(lq)[:, None] + offset, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        ws = w.sum(axis=1)
        out[:, h, :] = (w @ v[g]) / ws[:, None]
        lse[:, h] = m[:, 0] + np.log(ws)
    return out, lse


def phase2_partials(qq, q_pos0, k_cache, v_cache, k_self, v_self, base):
    """Per-shard partial results for one sequence.

    qq      [Lq][Hq][d] pre-RoPE query values at positions q_pos0 .. q_pos0+Lq-1
    k_cache [S][Hkv][n][d] rotated bf16 keys of the retained shards, v_cache alike
    k_self, v_self [Lq][Hkv][d] pre-RoPE keys / values of the query tokens
            themselves (or None): the query host's own shard, attended causally
    returns a list of (O_s [Lq][Hq][d], lse_s [Lq][Hq]), one per shard, the
    self shard last.
    """
    qq = np.asarray(qq, np.float64)
    lq = qq.shape[0]
    pos = q_pos0 + np.arange(lq)
    q_hat = rotate_bf16(qq, pos, base)
    parts = []
    for s in range(k_cache.shape[0]):
        parts.append(_shard_attend(q_hat, np.asarray(k_cache[s], np.float64),
                                   np.asarray(v_cache[s], np.float64), causal=False))
    if k_self is not None:
        ks = rotate_bf16(np.asarray(k_self, np.float64), pos, base).transpose(1, 0, 2)
        vs = np.asarray(v_self, np.float64).transpose(1, 0, 2)
        parts.append(_shard_attend(q_hat, ks, vs, causal=True))
    return parts


def decode_partials(qq, k_cache, v_cache, k_self, v_self, self_pos0, base):
    """Phase 2 of a generation step.  The query host's own shard holds n_self
    tokens at positions self_pos0 .. self_pos0 + n_self - 1: the query, then
    every token generated so far ("Dropping the Anchor ..." Section 2.2; Section
    5 runs the method with --tokens_to_generate 128).  The Lq query tokens are
    the last Lq of them; query t attends to every retained shard and, causally,
    to self tokens 0 .. n_self - Lq + t.

    qq             [Lq][Hq][d] pre-RoPE
    k_self, v_self [n_self][Hkv][d] pre-RoPE keys / values of the self tokens
    returns per-part (O, lse) like phase2_partials, the self shard last.
    With n_self == Lq this is phase2_partials with the self shard.
    """
    qq = np.asarray(qq, np.float64)
    lq = qq.shape[0]
    n_self = np.asarray(k_self).shape[0]
    off = n_self - lq
    q_hat = rotate_bf16(qq, self_pos0 + off + np.arange(lq), base)
    parts = []
    for s in range(k_cache.shape[0]):
        parts.append(_shard_attend(q_hat, np.asarray(k_cache[s], np.float64),
                                   np.asarray(v_cache[s], np.float64), causal=False))
    ks = rotate_bf16(np.asarray(k_self, np.float64), self_pos0 + np.arange(n_self), base)
    vs = np.asarray(v_self, np.float64)
    parts.append(_shard_attend(q_hat, ks.transpose(1, 0, 2), vs.transpose(1, 0, 2), causal=True,
                               offset=off))
    return parts


def dense_decode_attention(qq, k_cache, v_cache, k_self, v_self, self_pos0, base):
    """Twin of decode_partials + lse_merge, written as one masked softmax per
    query row over an explicit visible-key list."""
    qq = np.asarray(qq, np.float64)
    lq, hq, d = qq.shape
    n_self = np.asarray(k_self).shape[0]
    keys, vals = [], []
    for s in range(k_cache.shape[0]):
        keys.append(np.asarray(k_cache[s], np.float64))
        vals.append(np.asarray(v_cache[s], np.float64))
    ks = rotate_bf16(np.asarray(k_self, np.float64), self_pos0 + np.arange(n_self), base)
    keys.append(ks.transpose(1, 0, 2))
    vals.append(np.asarray(v_self, np.float64).transpose(1, 0, 2))
    kc = np.concatenate(keys, axis=1)
    vc = np.concatenate(vals, axis=1)
    n_ret = kc.shape[1] - n_self
    group = hq // kc.shape[0]
    out = np.empty((lq, hq, d))
    lse = np.empty((lq, hq))
    for t in range(lq):
        q_hat = rotate_bf16(qq[t:t + 1], np.array([self_pos0 + n_self - lq + t]), base)[0]
        n_vis = n_ret + (n_self - lq + t + 1)      # retained keys, then self keys up to itself
        for h in range(hq):
            g = h // group
            sc = kc[g, :n_vis] @ q_hat[h] / np.sqrt(d)
            m = sc.max()
            w = np.exp(sc - m)
            out[t, h] = w @ vc[g, :n_vis] / w.sum()
            lse[t, h] = m + np.log(w.sum())
    return out, lse


def lse_merge(o_parts, lse_parts):
    """Exact merge of normalised partials: lse = ln sum_s exp(lse_s),
    O = sum_s exp(lse_s - lse) O_s.  o_parts [S][...][d], lse_parts [S][...]."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    m = lse_parts.max(axis=0)
    lse = m + np.log(np.exp(lse_parts - m).sum(axis=0))
    w = np.exp(lse_parts - lse[None])
    return (w[..., None] * o_parts).sum(axis=0), lse


def dense_query_attention(qq, q_pos0, k_cache, v_cache, k_self, v_self, base):
    """Twin of phase2_partials + lse_merge: one softmax over the concatenation
    of every retained key and the causal self keys."""
    qq = np.asarray(qq, np.float64)
    lq = qq.shape[0]
    pos = q_pos0 + np.arange(lq)
    q_hat = rotate_bf16(qq, pos, base)
    kc = np.concatenate([np.asarray(k_cache[s], np.float64) for s in range(k_cache.shape[0])], axis=1)
    vc = np.concatenate([np.asarray(v_cache[s], np.float64) for s in range(v_cache.shape[0])], axis=1)
    n_ret = kc.shape[1]
    if k_self is not None:
        ks = rotate_bf16(np.asarray(k_self, np.float64), pos, base).transpose(1, 0, 2)
        vs = np.asarray(v_self, np.float64).transpose(1, 0, 2)
        kc = np.concatenate([kc, ks], axis=1)
        vc = np.concatenate([vc, vs], axis=1)
    hq, d = q_hat.shape[1], q_hat.shape[2]
    hkv = kc.shape[0]
    group = hq // hkv
    n = kc.shape[1]
    visible = np.ones((lq, n), bool)
    if k_self is not None:
        visible[:, n_ret:] = np.arange(lq)[None, :] <= np.arange(lq)[:, None]
    out = np.empty((lq, hq, d))
    lse = np.empty((lq, hq))
    for h in range(hq):
        g = h // group
        s = np.where(visible, q_hat[:, h, :] @ kc[g].T / np.sqrt(d), -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ vc[g]) / w.sum(axis=1, keepdims=True)
        lse[:, h] = m[:, 0] + np.log(w.sum(axis=1))
    return out, lse
