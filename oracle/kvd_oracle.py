"""CPU oracle for the KV-cached decoder step.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path
and never calls it. It is plain and slow on purpose: every step follows the
definitions on the pages, in float64, from the exact values of the stored
elements.

Sources (page title, section):
  [W]  "Whisper のデコーダー内部：Beam Search、Logit フィルター、KV キャッシュ"
       (readoss.com, openai/whisper): section "Inference 抽象と KV キャッシュ"
       (the cache hook, then the greedy and beam-search decoder paragraphs),
       section "言語検出" (-inf masking before argmax).
  [S]  "추측 디코딩으로 Whisper 추론 속도 2배 향상" (agentlenshq.com):
       section "추측 디코딩이란?".
  [N]  "nanoVLM における KV キャッシュ実装" (agentlenshq.com): sections
       "自己回帰生成における計算の冗長性", "KV キャッシュが推論を最適化する方法",
       "nanoVLM における技術的実装" (1. attention block, 2. per-layer cache
       tracking with start_pos, 3. prefill / decode split).
  [G]  Georgian translation of the Hugging Face speculative-decoding post
       (aitime.ge): the algorithm and its worked example.

Readings taken where the pages are silent (each pinned by a test unless
marked): scale 1/sqrt(D) on the score; max-subtracted softmax; a new token's
K/V is appended before attention, so the N queries sit at positions
L-N .. L-1 and query i sees keys j <= L-N+i; grouped heads are contiguous
(kv head = q head // (Hq/Hkv)); rotary embedding pairs (i, i+D/2) with
theta_i = base^(-2i/D) and is applied to keys before they are cached and to
queries at attention time; argmax ties go to the lowest index; verify row i
is compared with draft i. The rotary variant itself is a reading (the pages
name only the start_pos argument): parity for it is pinned to the RoFormer
identities, not to the pages. Logit filters set suppressed tokens to -inf
before the argmax: one token set on every row, and one more on the first
sampled row only. Beam-search candidate scoring follows the
decoder's update steps on [W]; the readings there: natural-log softmax, each
beam's K + 1 best tokens with equal values in index order, candidates with
equal scores in the order beam then rank, and end-of-text candidates met
before the K-th next beam recorded as finished.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Storage dtypes: exact widening to float64, correct rounding back.
# ---------------------------------------------------------------------------


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (f32, f16 or bf16 bit patterns)."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        with np.errstate(invalid="ignore"):     # NaN patterns stay NaN
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 the spacing is fixed at 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)                     # x = mant * 2^exp, 0.5 <= |mant| < 1
    quantum_exp = np.maximum(exp - 8, -133)     # spacing of bf16 values near x
    q = np.ldexp(1.0, quantum_exp)
    r = np.rint(x / q) * q                      # np.rint rounds half to even
    big = np.abs(r) > 3.3895313892515355e38     # above the largest finite bf16
    return np.where(big, np.copysign(np.inf, x), r)


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype (nearest, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        f = _round_bf16(x).astype(np.float32)   # exact: the value fits bf16
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Rotary position embedding at absolute positions ([N] "nanoVLM における技術的
# 実装", item 2: start_pos keeps rotary positions equal to the absolute
# generation index). The variant below (pairs (i, i+D/2), base^(-2i/D)) is the
# RoFormer one, a reading: the pages name no variant.
# ---------------------------------------------------------------------------


def rope_theta(base: float, D: int) -> np.ndarray:
    """theta_i = base^(-2i/D) for i < D/2, each the C library's float64 pow
    of the exact exponent -2i/D (math.pow; a vectorised numpy power may
    round differently from one CPU to the next)."""
    return np.array([math.pow(float(base), -(2.0 * i) / D) for i in range(D // 2)],
                    dtype=np.float64)


def rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate float64 rows x[..., t, :] by position positions[t].

    Pairs (i, i + D/2) turn by angle p * theta_i, one float64 product, with
    theta_i = base^(-2i/D); then (lo, hi) -> (lo c - hi s, hi c + lo s) with
    every product and sum rounded in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = rope_theta(base, D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# The KV cache: grown by concatenation along the sequence axis.
# [W] "Inference 抽象と KV キャッシュ", the save_to_cache hook: self attention
# the new key/value projection onto the cached sequence; the cross-attention
# entry is stored once from the encoder output and reused.
# [N] "KV キャッシュが推論を最適化する方法": a per-layer dict holding key and
# value tensors of shape (batch, heads, seq_cached, head_dim).
# ---------------------------------------------------------------------------


class ConcatCache:
    """One layer's K/V cache, stored in the storage dtype, [B, H, len, D]."""

    def __init__(self, B: int, H: int, D: int, dtype: str):
        self.dtype = dtype
        self.k = np.zeros((B, H, 0, D), dtype=_np_storage(dtype))
        self.v = np.zeros((B, H, 0, D), dtype=_np_storage(dtype))

    @property
    def length(self) -> int:
        return self.k.shape[2]

    def append(self, k_new: np.ndarray, v_new: np.ndarray, rope_base: float = 0.0):
        """Concatenate T new rows ([B, H, T, D], storage dtype).

        With rope_base > 0 the keys are rotated at positions len .. len+T-1
        first and the rotated keys are stored, rounded to the storage dtype.
        """
        if rope_base > 0.0:
            pos = np.arange(self.length, self.length + k_new.shape[2])
            k_new = narrow(rope(widen(k_new, self.dtype), pos, rope_base), self.dtype)
        self.k = np.concatenate([self.k, k_new], axis=2)
        self.v = np.concatenate([self.v, v_new], axis=2)

    def set_once(self, k: np.ndarray, v: np.ndarray):
        """Cross-attention cache: written once from the encoder-derived K/V."""
        self.k = np.array(k, copy=True)
        self.v = np.array(v, copy=True)

    def truncate(self, length: int):
        """Drop rows from position ``length`` on (speculative rollback)."""
        self.k = self.k[:, :, :length].copy()
        self.v = self.v[:, :, :length].copy()

    def reorder(self, parent):
        """Beam reorder ([W] beam search, step 4): row b takes the cache of
        beam parent[b], gathered from a snapshot taken before any row moves."""
        self.k = reorder(self.k, parent)
        self.v = reorder(self.v, parent)


def _np_storage(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def reorder(x: np.ndarray, parent) -> np.ndarray:
    snapshot = np.array(x, copy=True)
    out = np.empty_like(snapshot)
    for b, p in enumerate(parent):
        out[b] = snapshot[int(p)]
    return out


# ---------------------------------------------------------------------------
# Attention of the current queries over the cached keys and values.
# [N] workflow step 4: the current token's query is combined with the cached
# K and V. [W]: the hook hands attention the whole concatenated sequence even
# when only one token is new.
# ---------------------------------------------------------------------------


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           causal_offset: int | None) -> np.ndarray:
    """softmax(q K^T * scale) V for every (batch row, query head, query).

    q: [B, Hq, N, D]; k, v: [Bkv, Hkv, L, D] (float64 values; Bkv is B, or 1
    for a cache shared by every row). causal_offset=None lets every query see
    all L keys (cross attention); otherwise query i sees keys
    0 .. causal_offset + i.
    """
    B, Hq, N, D = q.shape
    Bkv, Hkv, L, _ = k.shape
    group = Hq // Hkv
    out = np.empty((B, Hq, N, D), dtype=np.float64)
    for b in range(B):
        bk = b if Bkv == B else 0
        for h in range(Hq):
            hk = h // group
            for i in range(N):
                seen = L if causal_offset is None else causal_offset + i + 1
                keys = k[bk, hk, :seen]
                vals = v[bk, hk, :seen]
                s = (keys @ q[b, h, i]) * scale
                w = np.exp(s - s.max())
                out[b, h, i] = (w @ vals) / w.sum()
    return out


def attend_self(q_store: np.ndarray, cache: ConcatCache, scale: float,
                rope_base: float = 0.0) -> np.ndarray:
    """Self attention after the N newest rows were appended: the queries sit
    at positions len-N .. len-1 and see keys up to their own position."""
    N = q_store.shape[2]
    L = cache.length
    q = widen(q_store, cache.dtype)
    if rope_base > 0.0:
        q = rope(q, np.arange(L - N, L), rope_base)
    return attend(q, widen(cache.k, cache.dtype), widen(cache.v, cache.dtype),
                  scale, causal_offset=L - N)


def attend_self_ragged(q_store: np.ndarray, caches, scale: float,
                       rope_base: float = 0.0) -> np.ndarray:
    """A ragged batch ([S] over a batch of sequences): batch row b has its own
    cache caches[b] (B = 1) with its own length, and its N queries sit at the
    last N positions of its own sequence. Rows are independent."""
    return np.concatenate([attend_self(q_store[b:b + 1], caches[b], scale, rope_base)
                           for b in range(len(caches))], axis=0)


def attend_cross(q_store: np.ndarray, cache: ConcatCache, scale: float) -> np.ndarray:
    """Cross attention: every query sees every encoder frame, no mask."""
    return attend(widen(q_store, cache.dtype), widen(cache.k, cache.dtype),
                  widen(cache.v, cache.dtype), scale, causal_offset=None)


# ---------------------------------------------------------------------------
# No-cache full recomputation ([N] "自己回帰生成における計算の冗長性"):
# without a cache every step projects K and V again for all tokens so far and
# attends over them with a causal mask. Written with whole-matrix products so
# that it shares no loop with ``attend``.
# ---------------------------------------------------------------------------


def full_causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                          scale: float) -> np.ndarray:
    """Q, K, V: [H, T, D] float64 (same head count). Row t attends keys 0..t."""
    T = Q.shape[1]
    scores = np.einsum("htd,hsd->hts", Q, K) * scale
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    scores = np.where(future[None], -np.inf, scores)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("hts,hsd->htd", w, V)


# ---------------------------------------------------------------------------
# Speculative verification.
# [W] "Inference 抽象と KV キャッシュ", greedy decoder paragraph: at
# temperature 0 the next token is the argmax; "言語検出": -inf entries are
# masked out and the argmax is taken over what remains.
# [S] / [G]: the main model scores all draft tokens in one pass; drafts are
# kept up to the first one that differs from the main model's token, that
# token replaces it, and everything after it is dropped.
# ---------------------------------------------------------------------------


def argmax_rows(logits: np.ndarray) -> np.ndarray:
    """Lowest index of the largest value in each row of [..., V] logits.

    -inf is an ordinary value (a row of only -inf gives 0). NaN is outside
    the contract.
    """
    flat = np.asarray(logits).reshape(-1, logits.shape[-1])
    out = np.empty(flat.shape[0], dtype=np.int32)
    for r in range(flat.shape[0]):
        row = flat[r].astype(np.float64)
        top = row.max()
        out[r] = np.flatnonzero(row == top)[0]
    return out.reshape(logits.shape[:-1])


def accept(argmax_row: np.ndarray, draft_row: np.ndarray):
    """Accepted length and corrected token for one batch row.

    argmax_row has R entries (R = N, or N + 1 with a bonus row); draft_row N.
    n = the first i with draft[i] != argmax[i] (N if none). The next token is
    argmax[n] when row n exists, else -1 (all drafts kept and no bonus row).
    """
    N = len(draft_row)
    R = len(argmax_row)
    n = 0
    while n < N and int(draft_row[n]) == int(argmax_row[n]):
        n += 1
    nxt = int(argmax_row[n]) if n < R else -1
    return n, nxt


def verify_accept(logits: np.ndarray, draft: np.ndarray):
    """logits [B, R, V], draft [B, N] -> (argmax [B, R], accept_len [B],
    next_token [B])."""
    am = argmax_rows(logits)
    B = draft.shape[0]
    acc = np.empty(B, dtype=np.int32)
    nxt = np.empty(B, dtype=np.int32)
    for b in range(B):
        acc[b], nxt[b] = accept(am[b], draft[b])
    return am, acc, nxt


# ---------------------------------------------------------------------------
# Logit filters before the argmax ([W] section "LogitFilter チェーン":
# SuppressBlank sets the blank and end-of-text logits to -inf at the first
# sampled position only, SuppressTokens sets a fixed token list to -inf on
# every step; section "言語検出": every token but the language tokens at -inf,
# then argmax).
# ---------------------------------------------------------------------------


def apply_suppression(logits: np.ndarray, suppress=None, suppress_first=None) -> np.ndarray:
    """Float64 copy of logits [B, R, V] with suppressed tokens at -inf:
    `suppress` (boolean [V]) on every row, `suppress_first` (boolean [V]) on
    row 0 of each batch row as well (the first sampled position)."""
    x = np.array(logits, dtype=np.float64, copy=True)
    if suppress is not None:
        x[:, :, np.asarray(suppress, dtype=bool)] = -np.inf
    if suppress_first is not None:
        x[:, 0, np.asarray(suppress_first, dtype=bool)] = -np.inf
    return x


def verify_accept_masked(logits: np.ndarray, draft: np.ndarray, suppress=None,
                         suppress_first=None):
    """verify_accept on the filtered logits. With no drafts (N = 0, R = 1) it
    is the masked argmax of one row per batch row: a greedy step, or language
    detection with every non-language token suppressed."""
    return verify_accept(apply_suppression(logits, suppress, suppress_first), draft)


# ---------------------------------------------------------------------------
# Beam-search candidate scoring ([W] beam-search decoder, update steps 1-3;
# step 4 is reorder() above).
# ---------------------------------------------------------------------------


def log_softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Natural-log softmax over the last axis, in float64, max-subtracted."""
    x = np.asarray(logits, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    return x - (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))


def beam_select(logits: np.ndarray, sum_logprobs: np.ndarray, eot: int):
    """One beam-search update for each audio row b of logits [B, K, V] (K
    beams) with running scores sum_logprobs [B, K]:

      1. log-probabilities of each beam's row, and its K + 1 best tokens
         (larger first, equal values: lower token first);
      2. every candidate (beam j, token t) scores sum_logprobs[b, j] + logp;
      3. candidates in order of score (larger first; equal scores keep the
         order beam, then rank) are taken one by one: an end-of-text token is
         recorded as finished (its beam and score), any other token becomes
         the next beam, until K next beams are chosen.

    Returns (parent [B, K], token [B, K], score [B, K], finished_count [B],
    finished_parent [B, K] (-1 past the count), finished_score [B, K]
    (nan past the count)).
    """
    B, K, V = logits.shape
    lp = log_softmax_rows(logits)
    parent = np.empty((B, K), dtype=np.int32)
    token = np.empty((B, K), dtype=np.int32)
    score = np.empty((B, K), dtype=np.float64)
    fin_count = np.zeros(B, dtype=np.int32)
    fin_parent = np.full((B, K), -1, dtype=np.int32)
    fin_score = np.full((B, K), np.nan)
    idx = np.arange(V)
    for b in range(B):
        cands = []
        for j in range(K):
            order = np.lexsort((idx, -lp[b, j]))[:K + 1]   # by -logp, then index
            for r, t in enumerate(order):
                cands.append((float(sum_logprobs[b, j]) + lp[b, j, t], j, r, int(t)))
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        kept = 0
        for sc, j, _, t in cands:
            if t == eot:
                fin_parent[b, fin_count[b]] = j
                fin_score[b, fin_count[b]] = sc
                fin_count[b] += 1
            else:
                parent[b, kept], token[b, kept], score[b, kept] = j, t, sc
                kept += 1
                if kept == K:
                    break
    return parent, token, score, fin_count, fin_parent, fin_score


# ---------------------------------------------------------------------------
# One decoder step over all layers, as the engine runs it.
# ---------------------------------------------------------------------------


def decode_step(q_self, q_cross, k_new, v_new, self_caches, cross_caches,
                scale: float, rope_base: float = 0.0, layers=None):
    """Append each layer's new K/V, then self attention and (if the layer has
    a cross cache) cross attention. Lists are indexed by layer; returns
    (self_out, cross_out) lists of float64 [B, Hq, N, D]."""
    layers = range(len(self_caches)) if layers is None else layers
    so, co = [], []
    for l in layers:
        self_caches[l].append(k_new[l], v_new[l], rope_base)
        so.append(attend_self(q_self[l], self_caches[l], scale, rope_base))
        if cross_caches is not None and cross_caches[l] is not None:
            co.append(attend_cross(q_cross[l], cross_caches[l], scale))
    return so, co
