"""Plain fp64 CPU oracle of the MISA indexer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The HIP library never
calls it and shares no code with it; its inputs come from the seeded
generator, which holds none of the indexer's arithmetic.

Every step is written out in float64 with numpy, one query at a time, in the
order the method's description gives.  A matrix product per query (a library
primitive) is the only aggregation; there is no blocking, fusion or reordering
beyond that.

What the method computes (sources: the gist.science technical summary of
"MISA: Mixture of Indexer Sparse Attention for Long-Context LLM Inference",
sections "Metodologia: MISA" and "Variante Hierárquica (MISA†)"; the
agents-report summary, sections "設計觀察與方法概述" and "階層化擴展：MISA†";
the abstract in the fugumt listing of arXiv 2605.07363):

  * the prefix of query t (length L = t+1) is cut into ceil(L/B) blocks and
    each block gets one mean-pooled indexer key;
  * a router scores every indexer head against the pooled keys, aggregates
    along the blocks into one importance per head, and keeps the top h heads;
  * only those heads score every prefix token; the top-k tokens are selected;
  * MISA-dagger keeps k' candidates from the routed pass and re-ranks them
    with the original all-head DSA indexer before taking the final top-k.

The token score is the DSA indexer score (DeepSeek-V3.2 lightning indexer),
which the pages name but do not print:
      I[t, s] = sum_j w[t, j] * ReLU(q[t, j] . k[s]).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of this repository):
  * block m covers absolute positions [mB, mB+B); the partial last block of a
    query's prefix is pooled over its visible keys (ceil counts it);
  * head importance r_j = w_j * sum_m ReLU(q_j . pooled_m) (signed weight, sum
    over the query's own causal blocks including the partial one);
  * ties: larger value first, then the lower head / token id; -0.0 == +0.0;
  * a query sees its own key (s <= t);
  * rows shorter than k are padded with id -1 (value -inf);
  * fp8 keys are OCP e4m3fn codes times a per-token fp32 scale.

Parity unpinned: the router's definition (how the partial block enters and
how the per-block affinities and the head weight combine into one head
importance) is a reading; the pages fix no formula or worked example for it.
Its arithmetic is pinned (brute force, the B = 1 closed form, relabelling and
scaling invariants), its agreement with the pages is not.  The other readings
(partial block dropped; |w| or no weight; max instead of sum over blocks) are
available here (head_importance_reading) so that the tests can measure how
many routed heads change between readings; the HIP path implements only the
first.
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# Input formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (bf16 is the top half of an IEEE float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities) -> float64.

    Layout s.eeee.mmm, exponent bias 7.  e > 0: (-1)^s * 2^(e-7) * (1 + m/8);
    e == 0: (-1)^s * 2^-6 * (m/8) (subnormal); s.1111.111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out


def f32_to_e4m3fn_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn code, round to nearest, ties to the even code.

    Written from the format: below 2^-6 the step is 2^-9 (subnormals, codes
    0..8, code 8 being the first normal 2^-6); in binade [2^E, 2^(E+1)) the
    step is 2^(E-3) and the code is ((E+7) << 3) | (mantissa steps - 8).
    Magnitudes past 448 (the largest finite value) saturate to it.  Every
    operation here is exact in float64 (power-of-two scaling of a float32)
    except the half-even rounding itself.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code = np.where(sub, np.rint(a / 2.0 ** -9).astype(np.int64), code)      # 0..8
    _, e2 = np.frexp(np.where(sub, 1.0, a))                                 # a = f * 2^e2, f in [0.5, 1)
    E = e2 - 1                                                              # a in [2^E, 2^(E+1))
    steps = np.rint(np.where(sub, 8.0, a) / np.ldexp(1.0, E - 3)).astype(np.int64)   # 8..16
    E = np.where(steps == 16, E + 1, E)
    steps = np.where(steps == 16, 8, steps)
    normal = ((E + 7) << 3) | (steps - 8)
    code = np.where(sub, code, normal)
    code = np.minimum(code, 0x7E)                                           # saturate at 448
    return (code | sign).astype(np.uint8)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def quantize_q_e4m3(q_bits: np.ndarray):
    """Per-row fp8 quantisation of bf16 indexer queries (rows = the last axis).

    Scale s = fp32(amax / 448), amax = max |q| over the row (s = 1 for an
    all-zero row); code = e4m3fn round-to-nearest-even of fp32(q / s), both
    divisions correctly rounded float32 operations.  The dequantised query is
    code * s.  Returns (codes uint8, same shape; scales float32, shape[:-1]).
    """
    q = bf16_bits_to_f32(q_bits)
    amax = np.abs(q).max(axis=-1)
    s = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    x = (q / s[..., None]).astype(np.float32)
    return f32_to_e4m3fn_rne(x), s


def dequantize_q_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3fn_to_f64(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def seq_keys(inp, b: int) -> np.ndarray:
    """Keys of sequence b as float64 [N, d]: bf16 widened, or fp8 decoded times scale."""
    if inp.k_scale is None:
        return bf16_bits_to_f64(inp.k[b])
    return e4m3fn_to_f64(inp.k[b]) * inp.k_scale[b].astype(np.float64)[:, None]


def seq_queries(inp, b: int) -> np.ndarray:
    return bf16_bits_to_f64(inp.q[b])          # [M, H, d]


def seq_weights(inp, b: int) -> np.ndarray:
    return inp.w[b].astype(np.float64)          # [M, H]


# --------------------------------------------------------------------------
# Step 1: block pooling of the shared indexer keys
# --------------------------------------------------------------------------

def pool_full_blocks(keys: np.ndarray, B: int) -> np.ndarray:
    """Mean-pooled key of every complete block m: mean of keys[mB : mB+B]."""
    n_full = keys.shape[0] // B
    out = np.empty((n_full, keys.shape[1]))
    for m in range(n_full):
        out[m] = keys[m * B:(m + 1) * B].sum(axis=0) / B
    return out


def tail_of(keys: np.ndarray, t: int, B: int):
    """Mean of the partial block of query t's prefix, or None when it is empty.

    The prefix [0, t] has floor((t+1)/B) complete blocks; the remaining
    t+1 - floor((t+1)/B)*B keys form the partial last block.
    """
    start = ((t + 1) // B) * B
    if start > t:
        return None
    return keys[start:t + 1].sum(axis=0) / (t + 1 - start)


# --------------------------------------------------------------------------
# Step 2: head router
# --------------------------------------------------------------------------

def head_importance(qt: np.ndarray, wt: np.ndarray, pooled: np.ndarray, tail, t: int, B: int):
    """S_j = sum over the query's complete blocks of ReLU(q_j . pooled_m), plus
    ReLU(q_j . tail) for the partial block; r_j = w_j * S_j.  qt [H, d], wt [H]."""
    n_full = (t + 1) // B
    S = np.zeros(qt.shape[0])
    if n_full > 0:
        S += np.maximum(qt @ pooled[:n_full].T, 0.0).sum(axis=1)
    if tail is not None:
        S += np.maximum(qt @ tail, 0.0)
    return S, wt * S


# Other readings of the router, for measuring how much the routed heads depend
# on the reading (the pages say the per-head affinities against the pooled
# block keys are aggregated along the blocks, but print no formula):
#   tail:   "pool" (the partial last block is pooled over its visible keys:
#           the block count ceil(L/B) includes it) | "drop" (floor(L/B)
#           complete blocks only);
#   weight: "signed" (r = w S) | "abs" (r = |w| S) | "none" (r = S);
#   agg:    "sum" (S = sum over blocks of ReLU(q . pooled)) | "max" (S = the
#           largest of those terms, 0 without any block).
# The first of each is the reading every other function here takes.
ROUTER_READINGS = dict(tail=("pool", "drop"), weight=("signed", "abs", "none"), agg=("sum", "max"))


def head_importance_reading(qt, wt, pooled, tail, t, B, tail_mode="pool", weight="signed", agg="sum"):
    """head_importance under the reading (tail_mode, weight, agg); returns (S, r)."""
    assert tail_mode in ROUTER_READINGS["tail"] and weight in ROUTER_READINGS["weight"]
    assert agg in ROUTER_READINGS["agg"]
    n_full = (t + 1) // B
    cols = [pooled[:n_full]]
    if tail is not None and tail_mode == "pool":
        cols.append(tail[None, :])
    blocks = np.concatenate(cols, axis=0)                    # [n_blocks, d]
    terms = np.maximum(qt @ blocks.T, 0.0)                   # [H, n_blocks]
    if terms.shape[1] == 0:
        S = np.zeros(qt.shape[0])
    elif agg == "sum":
        S = terms.sum(axis=1)
    else:
        S = terms.max(axis=1)
    f = {"signed": wt, "abs": np.abs(wt), "none": np.ones_like(wt)}[weight]
    return S, f * S


def top_positions(values: np.ndarray, ids: np.ndarray, count: int) -> np.ndarray:
    """Positions of the `count` entries with the largest values; equal values ->
    lower id first.  Returned in selection order (value descending, id ascending).

    -0.0 and +0.0 compare equal.  Entries are first put in ascending id order,
    then a stable sort on -value keeps equal values in that order.
    """
    order = np.argsort(ids, kind="stable")
    v = values[order] + 0.0                   # -0.0 -> +0.0
    sel = np.argsort(-v, kind="stable")[:count]
    return order[sel]


def top_ids(values: np.ndarray, ids: np.ndarray, count: int) -> np.ndarray:
    return ids[top_positions(values, ids, count)]


def route_query(qt, wt, pooled, keys, t, B, h, reading=None):
    """reading: None (this repository's reading), or a dict of the keywords of
    head_importance_reading (tail_mode, weight, agg)."""
    tail = tail_of(keys, t, B)
    if reading is None:
        S, r = head_importance(qt, wt, pooled, tail, t, B)
    else:
        S, r = head_importance_reading(qt, wt, pooled, tail, t, B, **reading)
    heads = np.sort(top_ids(r, np.arange(qt.shape[0]), h))   # stored ascending
    return S, r, heads


# --------------------------------------------------------------------------
# Step 3: token scoring with given heads (routed heads, or all heads = dense DSA)
# --------------------------------------------------------------------------

def score_query(qt, wt, keys, t, heads, n_cols=None):
    """I[s] = sum_{j in heads, ascending} w_j ReLU(q_j . k_s) for s <= t; -inf after."""
    n_cols = keys.shape[0] if n_cols is None else n_cols
    out = np.full(n_cols, NEG_INF)
    heads = np.sort(np.asarray(heads))
    dots = qt[heads] @ keys[:t + 1].T                  # [h, t+1]
    out[:t + 1] = (wt[heads][:, None] * np.maximum(dots, 0.0)).sum(axis=0)
    return out


def dense_query(qt, wt, keys, t, n_cols=None):
    return score_query(qt, wt, keys, t, np.arange(qt.shape[0]), n_cols)


def score_candidates(qt, wt, keys, cand):
    """All-head DSA score of the candidate tokens cand (entries < 0 -> -inf)."""
    out = np.full(len(cand), NEG_INF)
    ok = cand >= 0
    dots = qt @ keys[cand[ok]].T                       # [H, n_ok]
    out[ok] = (wt[:, None] * np.maximum(dots, 0.0)).sum(axis=0)
    return out


# --------------------------------------------------------------------------
# Step 4: top-k token selection
# --------------------------------------------------------------------------

def topk_row(values: np.ndarray, ids: np.ndarray, k: int):
    """Top-k of (values, ids): value descending, ties -> lower id; pad id -1 / -inf.
    Entries whose id is negative are not candidates."""
    keep = ids >= 0
    values, ids = values[keep], ids[keep]
    pos = top_positions(values, ids, k)
    out_i = np.full(k, -1, np.int64)
    out_v = np.full(k, NEG_INF)
    out_i[:len(pos)] = ids[pos]
    out_v[:len(pos)] = values[pos]
    return out_i, out_v


def topk_prefix(I_row: np.ndarray, t: int, k: int):
    """Top-k over the causal prefix s in [0, t] of a logit row."""
    return topk_row(I_row[:t + 1], np.arange(t + 1), k)


# --------------------------------------------------------------------------
# Whole indexer, per query
# --------------------------------------------------------------------------

class SeqContext:
    """Widened inputs of one sequence plus its pooled keys."""

    def __init__(self, inp, b: int, q8: bool = False):
        """q8: the queries as the fp8 path sees them (quantize_q_e4m3, then
        dequantised): every step below then follows that path."""
        cfg = inp.cfg
        self.B = cfg.block
        self.q_pos0 = inp.q_pos0
        self.keys = seq_keys(inp, b)
        self.q = dequantize_q_e4m3(*quantize_q_e4m3(inp.q[b])) if q8 else seq_queries(inp, b)
        self.w = seq_weights(inp, b)
        self.pooled = pool_full_blocks(self.keys, self.B)

    def t(self, i):
        return self.q_pos0 + i

    def tail(self, i):
        return tail_of(self.keys, self.t(i), self.B)

    def route(self, i, h, reading=None):
        return route_query(self.q[i], self.w[i], self.pooled, self.keys, self.t(i), self.B, h, reading)

    def score(self, i, heads):
        return score_query(self.q[i], self.w[i], self.keys, self.t(i), heads)

    def dense(self, i):
        return dense_query(self.q[i], self.w[i], self.keys, self.t(i))

    def misa(self, i, h, k):
        """MISA: route -> sparse scoring -> top-k.  Returns a dict of every stage."""
        S, r, heads = self.route(i, h)
        I = self.score(i, heads)
        idx, vals = topk_prefix(I, self.t(i), k)
        return dict(S=S, r=r, heads=heads, I=I, idx=idx, vals=vals)

    def misa_dagger(self, i, h, k_prime, k):
        """MISA-dagger: top-k' of the routed scores, all-head re-rank, top-k."""
        out = self.misa(i, h, k_prime)
        cand = out["idx"]                               # selection order, -1 padded
        D = score_candidates(self.q[i], self.w[i], self.keys, cand)
        fidx, fvals = topk_row(D, cand, k)
        out.update(cand=cand, cand_vals=out.pop("vals"), D=D, idx=fidx, vals=fvals)
        return out

    def dense_topk(self, i, k):
        I = self.dense(i)
        idx, vals = topk_prefix(I, self.t(i), k)
        return dict(I=I, idx=idx, vals=vals)
