"""Dense float64 attention over an explicit visibility mask (test infrastructure only).

Definitions followed:

* Two mask regimes, chosen per layer.  A full-attention layer is purely causal:
  key position j is visible to query position p iff j <= p.  A sliding layer is
  causal and also requires p - j < W, a strict comparison (unsloth commit
  ca9dbce, the change that builds one block mask per attention regime).
* The window counts the query's own position, so a query sees at most W keys
  including itself; an API that measures an inclusive distance would be given
  W - 1 (pegainfer issue #807, Description).
* Grouped-query heads: query head h reads KV head h // (Hq / Hkv).  The pages
  only say that several query heads share one KV head; contiguous groups are
  this oracle's reading.
* Softmax scale: passed in by the caller (the tiny workload fixes 1/sqrt(D)).
* No softcap on attention logits: the only softcap the pages describe is on the
  final logits (unsloth commit ca9dbce, Gemma-4 port, last bullet).

Nothing is blocked, fused or reordered: every (query, head) row is a masked
softmax over all stored rows, then a weighted sum of the value rows.
"""

import numpy as np


def visibility_mask(q_pos, kv_pos, window):
    """Boolean matrix M[i, r]: is the key stored at position kv_pos[r] visible to
    the query at position q_pos[i]?

    ``window == 0`` means a full-attention (pure causal) layer.
    """
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(kv_pos, dtype=np.int64)[None, :]
    m = j <= p
    if window > 0:
        m = m & ((p - j) < window)
    return m


def decode_positions(kv_len):
    """A decode query sits at the last stored position: the new token's K/V is
    written before attention and is visible to itself."""
    return np.array([kv_len - 1], dtype=np.int64)


def extend_positions(prefix_len, n_new):
    """An extend chunk of n_new queries follows a cached prefix of prefix_len."""
    return np.arange(prefix_len, prefix_len + n_new, dtype=np.int64)


def attend(q, q_pos, k, v, kv_pos, window, sm_scale):
    """Attention output in float64.

    q      : [nq, Hq, D]   query rows (any real dtype; taken as float64)
    q_pos  : [nq]          their positions
    k, v   : [n_kv, Hkv, D] stored key / value rows, in any order
    kv_pos : [n_kv]        the position each stored row holds
    window : 0 for full attention, else W
    returns: [nq, Hq, D] float64

    Every query must see at least one stored row (its own position is always
    visible once stored); a query that sees none is an input error.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, hq, d = q.shape
    n_kv, hkv, dk = k.shape
    if dk != d or v.shape != k.shape:
        raise ValueError("q, k, v head dims or k/v shapes disagree")
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    mask = visibility_mask(q_pos, kv_pos, window)
    if not mask.any(axis=1).all():
        raise ValueError("a query sees no stored key")
    # Rows no query can see never enter the arithmetic (they may be absent or
    # hold any bits in a real cache).
    used = mask.any(axis=0)
    mask = mask[:, used]
    k = k[used]
    v = v[used]
    out = np.empty((nq, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = sm_scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        s_max = s.max(axis=1, keepdims=True)
        w = np.exp(s - s_max)
        w = np.where(mask, w, 0.0)
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
