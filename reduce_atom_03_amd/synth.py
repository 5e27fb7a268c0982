"""Seeded synthetic inputs for the Atom collectives.

This module draws numbers and lays them out; it performs none of the
collectives' arithmetic (no sums, no rounding of results, no offset
derivation). Both the CPU oracle and the GPU library are fed from it, so
that every comparison runs on the same bytes.

Every rank's stream is ``numpy.random.default_rng([seed, rank])``; draws are
made in float32. bfloat16 inputs are produced by torch's CPU float32 ->
bfloat16 conversion (round to nearest even), and are returned as raw
``uint16`` bit patterns. Values never depend on how many threads generate
them.

Workloads (P virtual ranks held in one GPU's HBM):

* ``c1``: ReduceScatter, P=4, each input 4 partitions x 65536 fp32, U[-1,1], seed 1.
* ``c2``: composed AllReduce, P=8, 2**27 bf16 per input (256 MiB), N(0,1), seed 2.
* ``c3``: AllToAllV MoE dispatch, P=8 sources x 4096 tokens x 7168 bf16, N(0,1),
  seed 3; per-source counts C[r,:] ~ Multinomial(4096, Dirichlet(1^8)) drawn
  from ``default_rng([3, 1000])``.
* ``c4``: AllGather, P=8 partitions of S bytes bf16, U[-1,1], seed 4.
* ``c5``: decode AllReduce, P=8, b x 7168 bf16, N(0, 0.02) (0.02 = std), seed 5.
* ``moe``: expert-parallel dispatch and combine, P=8 ranks x 512 tokens x
  7168 bf16, N(0,1), seed 6; E=256 experts (32 per rank), top-8 routing ids
  and float32 gate weights from ``moe_routing`` (seed 6, stream 1002).
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

BF16 = "bf16"
F32 = "f32"

HIDDEN = 7168            # token width of the MoE / decode workloads
C3_TOKENS = 4096         # tokens per source in the AllToAllV workload
COUNTS_STREAM = 1000     # rank slot of the count-matrix stream
ROUTING_STREAM = 1002    # rank slot of the MoE routing stream
MOE_TOKENS = 512         # tokens per rank in the MoE workload (x top-8 = 4096 rows)
MOE_EXPERTS = 256
MOE_TOPK = 8


def rank_rng(seed: int, rank: int) -> np.random.Generator:
    """The generator of one virtual rank."""
    return np.random.default_rng([int(seed), int(rank)])


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch  # local import: torch is only needed for bf16 draws
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def draw(seed: int, rank: int, count: int, dist: str, dtype: str,
         scale: float = 1.0) -> np.ndarray:
    """``count`` values for ``rank``: dist 'uniform' = U[-scale, scale],
    'normal' = N(0, scale). Returns float32 for f32, uint16 bits for bf16."""
    g = rank_rng(seed, rank)
    if dist == "uniform":
        x = g.random(count, dtype=np.float32)
        x *= np.float32(2.0 * scale)
        x -= np.float32(scale)
    elif dist == "normal":
        x = g.standard_normal(count, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if dtype == F32:
        return x
    if dtype == BF16:
        return _bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def ranks(seed: int, P: int, count: int, dist: str, dtype: str,
          scale: float = 1.0, threads: int = 8) -> list[np.ndarray]:
    """One array per virtual rank, drawn in parallel (numpy releases the GIL)."""
    if threads <= 1 or P == 1 or count < (1 << 20):
        return [draw(seed, r, count, dist, dtype, scale) for r in range(P)]
    with ThreadPoolExecutor(min(threads, P)) as ex:
        return list(ex.map(lambda r: draw(seed, r, count, dist, dtype, scale),
                           range(P)))


def dirichlet_multinomial_counts(seed: int, P: int, tokens: int,
                                 alpha: float = 1.0) -> np.ndarray:
    """P x P int64 count matrix: row r ~ Multinomial(tokens, Dirichlet(alpha^P)).
    Zero entries are legal. Row r is source r's per-destination token counts."""
    g = rank_rng(seed, COUNTS_STREAM)
    C = np.empty((P, P), dtype=np.int64)
    for r in range(P):
        p = g.dirichlet(np.full(P, alpha))
        C[r] = g.multinomial(tokens, p)
    return C


def random_counts(seed: int, P: int, max_rows: int,
                  zero_frac: float = 0.25) -> np.ndarray:
    """Small ragged count matrices for edge tests: uniform in [0, max_rows]
    with about ``zero_frac`` of the entries forced to zero."""
    g = rank_rng(seed, COUNTS_STREAM + 1)
    C = g.integers(0, max_rows + 1, size=(P, P), dtype=np.int64)
    C[g.random((P, P)) < zero_frac] = 0
    return C


def tagged_rows(P: int, rows_per_rank: list[int], row_elems: int,
                seed: int = 7) -> list[np.ndarray]:
    """uint16 payloads whose rows are self-identifying: element 0 of row t of
    rank r holds r, element 1 holds t (mod 2**16); the rest are random bits,
    NaN and subnormal patterns included. Copies must move them bit-exactly."""
    out = []
    for r in range(P):
        g = rank_rng(seed, r)
        a = g.integers(0, 1 << 16, size=(rows_per_rank[r], row_elems),
                       dtype=np.uint16)
        if row_elems >= 1:
            a[:, 0] = r
        if row_elems >= 2:
            a[:, 1] = np.arange(rows_per_rank[r], dtype=np.int64) & 0xFFFF
        if row_elems >= 4 and rows_per_rank[r] > 0:
            a[0, 2] = 0x7FC1   # a quiet NaN with payload
            a[0, 3] = 0x0001   # the smallest bf16 subnormal
        out.append(a.reshape(-1))
    return out


# ---------------------------------------------------------------- workloads

def c1_inputs(P: int = 4, n: int = 65536) -> list[np.ndarray]:
    """ReduceScatter workload: P inputs of P*n fp32, U[-1,1], seed 1."""
    return ranks(1, P, P * n, "uniform", F32)


def c2_inputs(P: int = 8, elems: int = 1 << 27) -> list[np.ndarray]:
    """Composed AllReduce workload: P inputs of ``elems`` bf16, N(0,1), seed 2."""
    return ranks(2, P, elems, "normal", BF16)


def c3_counts(P: int = 8, tokens: int = C3_TOKENS) -> np.ndarray:
    return dirichlet_multinomial_counts(3, P, tokens)


def c3_inputs(P: int = 8, tokens: int = C3_TOKENS,
              hidden: int = HIDDEN) -> list[np.ndarray]:
    """AllToAllV workload: P sources of tokens x hidden bf16, N(0,1), seed 3."""
    return ranks(3, P, tokens * hidden, "normal", BF16)


def c4_inputs(S_bytes: int, P: int = 8) -> list[np.ndarray]:
    """AllGather workload: P partitions of S bytes of bf16, U[-1,1], seed 4."""
    return ranks(4, P, S_bytes // 2, "uniform", BF16)


def c5_inputs(b: int, P: int = 8, hidden: int = HIDDEN) -> list[np.ndarray]:
    """Decode AllReduce workload: P inputs of b x hidden bf16, N(0, 0.02), seed 5."""
    return ranks(5, P, b * hidden, "normal", BF16, scale=0.02)


def mixed_bits(seed: int, rank: int, count: int, dtype: str,
               specials: bool = True) -> np.ndarray:
    """Bit patterns spread over every binade, with signed zeros, subnormals,
    values near overflow and (when ``specials``) infinities and NaNs mixed
    in. uint16 for bf16, float32 (bit-cast) for f32."""
    g = rank_rng(seed, rank)
    if dtype == BF16:
        bits = g.integers(0, 1 << 16, size=count, dtype=np.uint32)
        pool = [0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80]
        if specials:
            pool += [0x7F80, 0xFF80, 0x7FC0, 0x7F81]
        exp_mask, frac_mask, shift = 0xFF, 0x7F, 7
    else:
        bits = g.integers(0, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)
        pool = [0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F7FFFFF,
                0xFF7FFFFF, 0x3F800000, 0xBF800000]
        if specials:
            pool += [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001]
        exp_mask, frac_mask, shift = 0xFF, 0x7FFFFF, 23
    if not specials:
        # keep random patterns finite: clamp an all-ones exponent down by one
        e = (bits >> shift) & exp_mask
        bits = np.where(e == exp_mask, bits - (1 << shift), bits).astype(np.uint32)
    # Narrow the exponent range of half the values so that sums interact.
    mid = g.random(count) < 0.5
    sign = bits >> (shift + 8)
    near = (np.uint32(127 - 4) + g.integers(0, 9, size=count).astype(np.uint32))
    bits = np.where(mid, (sign << (shift + 8)) | (near << shift) | (bits & frac_mask),
                    bits).astype(np.uint32)
    pick = g.random(count) < 0.1
    bits = np.where(pick, np.asarray(pool, dtype=np.uint32)[
        g.integers(0, len(pool), size=count)], bits).astype(np.uint32)
    if dtype == BF16:
        return bits.astype(np.uint16)
    return bits.view(np.float32)


def zipf_partition(total: int, P: int, s: float = 0.125, unit: int = 1) -> np.ndarray:
    """Sizes of P partitions in Zipf proportion: partition k gets a share
    proportional to (k + 1) ** -s of `total` elements, in whole multiples of
    `unit` (total must be a multiple of unit). Shares are floored and the
    remainder goes to the largest fractional parts, so the sizes sum to
    `total` exactly. s = 0 gives equal partitions."""
    if total % unit:
        raise ValueError("total must be a multiple of unit")
    units = total // unit
    w = (np.arange(1, P + 1, dtype=np.float64)) ** (-float(s))
    share = units * w / w.sum()
    base = np.floor(share).astype(np.int64)
    rest = int(units - base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rest]] += 1
    return base * unit


def moe_routing(seed: int, P: int, tokens: int, experts: int, topk: int,
                alpha: float = 1.0):
    """Synthetic router output for P ranks of ``tokens`` tokens.

    Expert popularity p ~ Dirichlet(alpha^E) (one draw shared by all ranks,
    so some experts are hot and some receive nothing); every token then picks
    ``topk`` distinct experts by Gumbel-top-k sampling from p (a draw without
    replacement in proportion to p), listed in descending key order. Gate
    weights are a softmax over ``topk`` N(0,1) logits, in float32. Returns
    (ids, weights): P int32 arrays and P float32 arrays of tokens*topk,
    token-major."""
    g = rank_rng(seed, ROUTING_STREAM)
    p = g.dirichlet(np.full(experts, alpha))
    logp = np.log(np.maximum(p, 1e-300))
    ids, weights = [], []
    for r in range(P):
        gr = rank_rng(seed, ROUTING_STREAM + 1 + r)
        key = logp[None, :] + gr.gumbel(size=(tokens, experts))
        top = np.argsort(-key, axis=1, kind="stable")[:, :topk]
        ids.append(np.ascontiguousarray(top, dtype=np.int32).reshape(-1))
        z = gr.standard_normal((tokens, topk)).astype(np.float32)
        z = np.exp(z - z.max(axis=1, keepdims=True))
        weights.append(np.ascontiguousarray(z / z.sum(axis=1, keepdims=True),
                                            dtype=np.float32).reshape(-1))
    return ids, weights


def moe_inputs(P: int = 8, tokens: int = MOE_TOKENS, hidden: int = HIDDEN):
    """Token rows of the MoE workload: P ranks of tokens x hidden bf16, N(0,1), seed 6."""
    return ranks(6, P, tokens * hidden, "normal", BF16)
