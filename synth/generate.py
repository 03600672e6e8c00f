"""Seeded draws of weights and request streams (numpy PCG64).

Weights: every matrix, embedding, bias and the head are N(0, 0.02); LayerNorm
gains are 1 + N(0, 0.02) and shifts N(0, 0.02), so the affine paths are
exercised.  For bf16 workloads every value is rounded once to the nearest bf16
(ties to even) at generation time, so the oracle and the GPU read identical
numbers; matrices and embeddings are then kept as raw bf16 bit patterns
(uint16) to halve host memory, vectors as float32 holding bf16-exact values.

Requests: lengths follow the workload's law (inclusive integer ranges) and
token ids are uniform on [0, vocab).  Nothing here computes any part of the
scoring method.
"""
import numpy as np

from .configs import ModelConfig

STD = 0.02


def WEIGHT_ORDER(cfg: ModelConfig):
    """(name, shape, kind) of every tensor in draw order.

    kind: "mat" (matrix / embedding), "vec" (bias, shift, head), "gain" (LN gain).
    The slot "norm_*" is the embedding LayerNorm of a post-LN encoder and the
    final LayerNorm of a pre-LN decoder.
    """
    H, F, V, P = cfg.hidden, cfg.ffn, cfg.vocab, cfg.max_pos
    out = [("tok_emb", (V, H), "mat"), ("pos_emb", (P, H), "mat"),
           ("norm_g", (H,), "gain"), ("norm_b", (H,), "vec")]
    for l in range(cfg.n_layers):
        p = f"l{l}."
        out += [(p + "w_qkv", (3 * H, H), "mat"), (p + "b_qkv", (3 * H,), "vec"),
                (p + "w_o", (H, H), "mat"), (p + "b_o", (H,), "vec"),
                (p + "ln1_g", (H,), "gain"), (p + "ln1_b", (H,), "vec"),
                (p + "w_1", (F, H), "mat"), (p + "b_1", (F,), "vec"),
                (p + "w_2", (H, F), "mat"), (p + "b_2", (H,), "vec"),
                (p + "ln2_g", (H,), "gain"), (p + "ln2_b", (H,), "vec")]
    out += [("head_w", (H,), "vec"), ("head_b", (1,), "vec")]
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_float32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_float(arr: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Widen a stored weight (float32, or bf16 bits as uint16) to ``dtype``."""
    if arr.dtype == np.uint16:
        return bf16_to_float32(arr).astype(dtype, copy=False)
    return arr.astype(dtype, copy=False)


def make_weights(cfg: ModelConfig, seed=None) -> dict:
    """Draw all parameters in WEIGHT_ORDER from one PCG64 stream."""
    rng = np.random.default_rng(cfg.seeds["weights"] if seed is None else seed)
    w = {}
    for name, shape, kind in WEIGHT_ORDER(cfg):
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(STD)
        if kind == "gain":
            x = x + np.float32(1.0)
        if cfg.bf16:
            b = round_to_bf16(x)
            w[name] = b if kind == "mat" else bf16_to_float32(b)
        else:
            w[name] = np.ascontiguousarray(x, dtype=np.float32)
    return w


def _draw(rng, lengths, vocab):
    lengths = np.asarray(lengths, dtype=np.int32)
    ids = rng.integers(0, vocab, size=int(lengths.sum()), dtype=np.int64).astype(np.int32)
    return ids, lengths


def split(ids: np.ndarray, lengths: np.ndarray):
    """Packed ids + lengths -> list of per-sequence id arrays."""
    cuts = np.cumsum(lengths)[:-1]
    return np.split(ids, cuts)


def make_requests(cfg: ModelConfig, seed=None):
    """The workload's request stream, in arrival order.

    Returns (ids int32[sum n], lengths int32[n], group int32[n]); ``group`` is
    the prompt index for the best-of-N decoder workload and -1 elsewhere.
    """
    rng = np.random.default_rng(cfg.seeds["requests"] if seed is None else seed)
    name = cfg.name
    if name == "tiny_fp32":
        lengths = rng.integers(2, 33, size=8)
    elif name == "tinybert":
        lengths = np.full(64, 128)
    elif name == "bert_base_short":
        lengths = rng.integers(2, 101, size=2000)
    elif name == "bert_base_longtail":
        lengths = np.concatenate([rng.integers(5, 501, size=1800),
                                  rng.integers(400, 501, size=200)])
        lengths = lengths[rng.permutation(lengths.size)]
    elif name == "decoder_rm":
        n_prompts, n_cand, plen = 64, 16, 512
        prompts = rng.integers(0, cfg.vocab, size=(n_prompts, plen), dtype=np.int64)
        slen = rng.integers(8, 49, size=(n_prompts, n_cand))
        seqs, group = [], []
        for p in range(n_prompts):
            for c in range(n_cand):
                summ = rng.integers(0, cfg.vocab, size=int(slen[p, c]), dtype=np.int64)
                seqs.append(np.concatenate([prompts[p], summ]))
                group.append(p)
        lengths = np.array([s.size for s in seqs], dtype=np.int32)
        ids = np.concatenate(seqs).astype(np.int32)
        return ids, lengths, np.array(group, dtype=np.int32)
    else:
        raise KeyError(name)
    ids, lengths = _draw(rng, lengths, cfg.vocab)
    return ids, lengths, np.full(lengths.size, -1, dtype=np.int32)


def make_reference_set(cfg: ModelConfig, seed=None):
    """Reference sequences whose mean reward the offset sets to zero.

    Decoder workload: one reference summary (U{8..48}) after each of the 64
    prompts.  tiny: 8 x U{2..32}.  tinybert: 64 x 128.  BERT-base streams: 64
    lengths from U{2..100} or U{5..500}.  Returns (ids, lengths).
    """
    rng = np.random.default_rng(cfg.seeds["reference"] if seed is None else seed)
    name = cfg.name
    if name == "tiny_fp32":
        lengths = rng.integers(2, 33, size=8)
    elif name == "tinybert":
        lengths = np.full(64, 128)
    elif name == "bert_base_short":
        lengths = rng.integers(2, 101, size=64)
    elif name == "bert_base_longtail":
        lengths = rng.integers(5, 501, size=64)
    elif name == "decoder_rm":
        ids_r, lengths_r, group = make_requests(cfg)
        starts = np.concatenate([[0], np.cumsum(lengths_r)[:-1]])
        seqs = []
        for p in range(64):
            first = int(np.flatnonzero(group == p)[0])
            prompt = ids_r[starts[first]:starts[first] + 512]
            summ = rng.integers(0, cfg.vocab, size=int(rng.integers(8, 49)), dtype=np.int64)
            seqs.append(np.concatenate([prompt, summ.astype(np.int32)]))
        lengths = np.array([s.size for s in seqs], dtype=np.int32)
        return np.concatenate(seqs).astype(np.int32), lengths
    else:
        raise KeyError(name)
    return _draw(rng, lengths, cfg.vocab)


def make_fixed_batch(cfg: ModelConfig, seq_len: int, batch: int, seed=None):
    """``batch`` sequences of exactly ``seq_len`` uniform ids (fixed-length runs)."""
    s = cfg.seeds["requests"] * 100003 + seq_len * 1009 + batch if seed is None else seed
    rng = np.random.default_rng(s)
    return _draw(rng, np.full(batch, seq_len), cfg.vocab)


def random_stream(seed: int, n: int, lo: int, hi: int, vocab: int):
    """Generic seeded stream: n sequences with lengths U{lo..hi}; (ids, lengths)."""
    rng = np.random.default_rng(seed)
    return _draw(rng, rng.integers(lo, hi + 1, size=n), vocab)


def best_of_n_form(ids, lengths, group, prompt_len):
    """Split a best-of-N request stream into its prompt / candidate form.

    Every request is prompt + candidate, requests of one prompt are adjacent
    and share their first ``prompt_len`` ids (the decoder workload's law).
    Pure slicing.  Returns (prompt_ids, prompt_lengths, cand_ids, cand_lengths,
    cand_counts), all int32; candidates keep request order.
    """
    ids = np.asarray(ids)
    lengths = np.asarray(lengths)
    group = np.asarray(group)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    p_ids, p_len, c_ids, c_len, counts = [], [], [], [], []
    i = 0
    while i < lengths.size:
        j = i
        while j < lengths.size and group[j] == group[i]:
            j += 1
        p_ids.append(ids[starts[i]:starts[i] + prompt_len])
        p_len.append(prompt_len)
        for k in range(i, j):
            assert np.array_equal(ids[starts[k]:starts[k] + prompt_len], p_ids[-1])
            c_ids.append(ids[starts[k] + prompt_len:starts[k + 1]])
            c_len.append(int(lengths[k]) - prompt_len)
        counts.append(j - i)
        i = j
    as32 = lambda a: np.asarray(a, dtype=np.int32)
    return (as32(np.concatenate(p_ids)), as32(p_len), as32(np.concatenate(c_ids)), as32(c_len),
            as32(counts))
