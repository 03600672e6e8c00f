"""Plain forward pass of the scoring transformer (oracle; test infrastructure).

Model, read from the pages (see the package docstring for titles):
  * Encoder workloads (compact BERT / BERT-base shapes): post-LN layers with an
    embedding LayerNorm, bidirectional attention inside each sequence.
  * Decoder reward model ("Learning to summarize from human feedback",
    Compute setup and Method adaptation): pre-LN layers, causal attention, a final LayerNorm, and a scalar
    head read at the last token of the complete sequence.
  * Every workload: token + learned absolute position embeddings (positions
    restart at 0 in each sequence), GELU in its exact erf form, LayerNorm with
    biased variance and the workload's epsilon, attention scores scaled by
    1/sqrt(head_dim) with masked keys excluded, and a reward
    r = w . h_last + b + offset, where the offset makes the reference
    sequences average zero.

Everything is computed per sequence ("one at a time") in ``dtype``; the packed
and padded batch forms exist only so the tests can show that all three agree.
"""
import math

import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------- primitives

def layer_norm(x, g, b, eps):
    """Row-wise LayerNorm: (x - mean) / sqrt(var + eps) * g + b, biased var.

    TurboTransformers review, Proposed method: LayerNorm is a per-row reduction.
    """
    mu = x.mean(axis=-1, keepdims=True)
    c = x - mu
    var = (c * c).mean(axis=-1, keepdims=True)
    return c / np.sqrt(var + x.dtype.type(eps)) * g + b


def softmax_rows(s):
    """Row-wise softmax: exp(s - max) / sum; -inf entries get weight 0.

    TurboTransformers review, Proposed method: Softmax is a per-row reduction.
    """
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def gelu(z):
    """GELU(z) = z * Phi(z) = z/2 * (1 + erf(z / sqrt(2))), erf in float64."""
    z64 = np.asarray(z, dtype=np.float64)
    return (0.5 * z64 * (1.0 + erf(z64 / math.sqrt(2.0)))).astype(np.asarray(z).dtype)


def linear(x, w, b):
    """x W^T + b with W stored [out, in] (one library matmul)."""
    return x @ w.T + b


def attention(x, w_qkv, b_qkv, n_heads, causal, key_mask=None):
    """Multi-head self-attention context (before the output projection).

    ``x`` is [n, H]; W_qkv rows are Q | K | V, head h owning rows h*d..h*d+d-1
    of each block.  ``key_mask`` [n, n] (True = visible) replaces the default
    mask (all keys, or keys j <= i when causal); used by the packed form.
    """
    H = x.shape[1]
    qkv = linear(x, w_qkv, b_qkv)
    return masked_attention(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], n_heads, causal, key_mask)


def masked_attention(q, k, v, n_heads, causal, key_mask=None):
    """Per head h: softmax(Q_h K_h^T / sqrt(d)) V_h over the visible keys,
    heads concatenated; q, k, v are [n, H] with head h at columns
    h*d..h*d+d-1.  Mask as in ``attention``."""
    n, H = q.shape
    d = H // n_heads
    if key_mask is None:
        key_mask = np.ones((n, n), dtype=bool)
        if causal:
            key_mask = np.tril(key_mask)
    scale = q.dtype.type(1.0 / math.sqrt(d))
    ctx = np.empty_like(q)
    for h in range(n_heads):
        sl = slice(h * d, (h + 1) * d)
        s = (q[:, sl] @ k[:, sl].T) * scale
        s = np.where(key_mask, s, -np.inf)
        ctx[:, sl] = softmax_rows(s) @ v[:, sl]
    return ctx


def _widen(a, dtype):
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)
    return a.astype(dtype)


# ---------------------------------------------------------------- model

class OracleModel:
    """Reference forward of one scoring model in ``dtype`` (float64 default)."""

    def __init__(self, cfg, weights, dtype=np.float64, cache=True):
        self.cfg = cfg
        self.w = weights
        self.dtype = np.dtype(dtype)
        self.cache = cache
        self._c = {}

    def W(self, name):
        if name in self._c:
            return self._c[name]
        a = _widen(self.w[name], self.dtype)
        if self.cache:
            self._c[name] = a
        return a

    def _rows(self, name, idx):
        a = self.w[name][idx]
        return _widen(a, self.dtype)

    # -- embeddings (positions restart at 0 in every sequence)
    def embed(self, ids, positions):
        cfg = self.cfg
        x = self._rows("tok_emb", ids) + self._rows("pos_emb", positions)
        if not cfg.pre_ln:
            x = layer_norm(x, self.W("norm_g"), self.W("norm_b"), cfg.eps)
        return x

    def layer(self, l, x, key_mask=None):
        cfg, p = self.cfg, f"l{l}."
        W = self.W
        if not cfg.pre_ln:
            ctx = attention(x, W(p + "w_qkv"), W(p + "b_qkv"), cfg.n_heads, cfg.causal, key_mask)
            y = layer_norm(x + linear(ctx, W(p + "w_o"), W(p + "b_o")),
                           W(p + "ln1_g"), W(p + "ln1_b"), cfg.eps)
            f = linear(gelu(linear(y, W(p + "w_1"), W(p + "b_1"))), W(p + "w_2"), W(p + "b_2"))
            return layer_norm(y + f, W(p + "ln2_g"), W(p + "ln2_b"), cfg.eps)
        u = layer_norm(x, W(p + "ln1_g"), W(p + "ln1_b"), cfg.eps)
        ctx = attention(u, W(p + "w_qkv"), W(p + "b_qkv"), cfg.n_heads, cfg.causal, key_mask)
        x = x + linear(ctx, W(p + "w_o"), W(p + "b_o"))
        m = layer_norm(x, W(p + "ln2_g"), W(p + "ln2_b"), cfg.eps)
        return x + linear(gelu(linear(m, W(p + "w_1"), W(p + "b_1"))), W(p + "w_2"), W(p + "b_2"))

    def hidden(self, ids, n_layers=None):
        """Residual stream [n, H] after ``n_layers`` layers (default: all)."""
        ids = np.asarray(ids)
        L = self.cfg.n_layers if n_layers is None else n_layers
        x = self.embed(ids, np.arange(ids.size))
        for l in range(L):
            x = self.layer(l, x)
        return x

    def head(self, h_last, offset=0.0):
        """Scalar head on final-token rows [b, H] (pre-LN: final LayerNorm first)."""
        if self.cfg.pre_ln:
            h_last = layer_norm(h_last, self.W("norm_g"), self.W("norm_b"), self.cfg.eps)
        r = h_last @ self.W("head_w") + self.W("head_b")[0]
        return r + self.dtype.type(offset)

    # -- one at a time: the definition
    def score(self, ids, offset=0.0):
        return float(self.head(self.hidden(ids)[-1:], offset)[0])

    def score_many(self, seqs, offset=0.0):
        return np.array([self.score(s, offset) for s in seqs], dtype=np.float64)

    # -- packed form: all sequences in one [T, H] array, block-diagonal mask
    def score_packed(self, ids, lengths, offset=0.0):
        lengths = np.asarray(lengths)
        offs = np.concatenate([[0], np.cumsum(lengths)])
        T = int(offs[-1])
        seq_of = np.repeat(np.arange(lengths.size), lengths)
        pos = np.arange(T) - offs[seq_of]
        mask = seq_of[:, None] == seq_of[None, :]
        if self.cfg.causal:
            mask &= pos[None, :] <= pos[:, None]
        x = self.embed(np.asarray(ids), pos)
        for l in range(self.cfg.n_layers):
            x = self.layer(l, x, key_mask=mask)
        return self.head(x[offs[1:] - 1], offset).astype(np.float64)

    # -- padded form: [b, max_n] with padding keys masked, padded rows dropped
    def score_padded(self, seqs, offset=0.0, pad_id=0):
        b = len(seqs)
        nmax = max(len(s) for s in seqs)
        n = np.array([len(s) for s in seqs])
        ids = np.full((b, nmax), pad_id, dtype=np.int64)
        for i, s in enumerate(seqs):
            ids[i, :n[i]] = s
        blk = np.repeat(np.arange(b), nmax)          # row -> sequence
        pos = np.tile(np.arange(nmax), b)            # row -> position
        mask = (blk[:, None] == blk[None, :]) & (pos < n[blk])[None, :]
        if self.cfg.causal:
            mask &= pos[None, :] <= pos[:, None]
        x = self.embed(ids.reshape(-1), pos)
        for l in range(self.cfg.n_layers):
            x = self.layer(l, x, key_mask=mask)
        last = np.arange(b) * nmax + n - 1
        return self.head(x[last], offset).astype(np.float64)

    def calibrate_offset(self, ref_seqs):
        """offset = -mean of the raw reference rewards (mean taken in float64).

        "Learning to summarize from human feedback", Method adaptation: reward outputs are
        normalised so that reference summaries score zero on average.
        """
        raw = self.score_many(ref_seqs, 0.0)
        return float(np.float32(-raw.mean()))
