"""Byte and launch ledgers of the three fused chains, walked stage by stage.

TEST INFRASTRUCTURE (part of the oracle): the library's own accounting uses
closed forms; this module re-derives the same integers from the pages'
per-stage read/write descriptions so the two can be compared.

Sources:
  * "K4 讲解：fusion 的三笔账", section 1: each operator of the GEMM epilogue
    chain is described by the elements it writes and the elements it reads
    from outside the chain (weights, bias, residual).  A split plan is a list of
    segment lengths; every segment is one kernel, every cut writes one [M,N]
    intermediate back to DRAM and the next kernel reads it again.
  * "AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.2: one pass over an
    N-element tensor reads N*b and writes N*b bytes; an unfused K-stage chain
    makes K passes, the fused chain one.
  * same page, appendix ledger [A3]: the five softmax steps read/write the
    score tensor 1 + 2 + 2 + 1 + 2 = 8 times unfused and 2 times fused, plus
    one materialised mask of the score's size.
  * same page, section 3.5: causal block skipping, query block q computes key
    blocks 0..q only.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import List, Sequence


@dataclass(frozen=True)
class Stage:
    """One operator of a chain: elements it writes, elements it reads from
    outside the chain, and the elements of the chain value it reads (0 for the
    chain's first operator, whose operands are all external)."""
    name: str
    writes: int
    external_reads: int
    chain_reads: int


def gemm_epilogue_stages(M: int, N: int, K: int) -> List[Stage]:
    """mm -> bias -> gelu -> res on an [M,N] output (K4 section 1)."""
    MN = M * N
    return [
        Stage("mm", MN, M * K + K * N, 0),
        Stage("bias", MN, N, MN),
        Stage("gelu", MN, 0, MN),
        Stage("res", MN, MN, MN),
    ]


def check_plan(plan: Sequence[int], n_stages: int) -> None:
    if len(plan) == 0 or any(int(p) <= 0 for p in plan) or sum(plan) != n_stages:
        raise ValueError(f"plan {list(plan)} is not a composition of {n_stages}")


def traffic(stages: Sequence[Stage], plan: Sequence[int], elem_bytes: int):
    """DRAM bytes and kernel launches of one split plan.

    Walk the segments: inside a segment the chain value stays on chip, so only
    the segment's first operator reads the chain value from DRAM (unless it
    starts the chain) and only its last operator writes to DRAM; every operator
    reads its external operands once.
    """
    check_plan(plan, len(stages))
    elems = 0
    pos = 0
    for seg_len in plan:
        seg = stages[pos:pos + seg_len]
        elems += seg[0].chain_reads           # re-read the previous cut (0 at chain start)
        for st in seg:
            elems += st.external_reads
        elems += seg[-1].writes               # one write-back per segment
        pos += seg_len
    return elems * elem_bytes, len(plan)


def plan_bytes(M: int, N: int, K: int, plan: Sequence[int], elem_bytes: int = 2) -> int:
    return traffic(gemm_epilogue_stages(M, N, K), plan, elem_bytes)[0]


def plan_launches(plan: Sequence[int]) -> int:
    check_plan(plan, 4)
    return len(plan)


def compositions(n: int) -> List[List[int]]:
    """All 2**(n-1) ways to cut an n-stage chain into contiguous segments,
    enumerated by which of the n-1 gaps carry a cut."""
    out = []
    for mask in range(1 << (n - 1)):
        plan, run = [], 1
        for gap in range(n - 1):
            if mask >> gap & 1:
                plan.append(run)
                run = 1
            else:
                run += 1
        plan.append(run)
        out.append(plan)
    return out


# ---------------------------------------------------------------- pointwise chain

def chain_stages(n: int, K: int) -> List[Stage]:
    """K pointwise stages on n elements; the first reads x from outside."""
    return [Stage(f"s{s}", n, n if s == 0 else 0, 0 if s == 0 else n) for s in range(K)]


def chain_bytes(n: int, K: int, fused: bool, elem_bytes: int = 4) -> int:
    plan = [K] if fused else [1] * K
    return traffic(chain_stages(n, K), plan, elem_bytes)[0]


# ---------------------------------------------------------------- causal softmax

def causal_kept_fraction(S: int) -> Fraction:
    """Exact kept fraction S(S+1)/2 / S^2 (section 3.5), counted element by element."""
    kept = sum(i + 1 for i in range(S))
    return Fraction(kept, S * S)


def causal_block_fraction(S: int, tile: int) -> Fraction:
    """Block-level kept fraction: query block q computes key blocks 0..q."""
    nb = -(-S // tile)
    done = sum(1 for q in range(nb) for kb in range(nb) if kb <= q)
    return Fraction(done, nb * nb)


def softmax_elements_read(S: int, tile: int) -> int:
    """Score elements one [S,S] head reads when each query row i loads the key
    tiles 0..floor(i/tile) (the last tile may be partial)."""
    total = 0
    for i in range(S):
        total += min(S, (i // tile + 1) * tile)
    return total


def softmax_bytes(BH: int, S: int, tile: int, fused: bool, elem_bytes: int = 2,
                  stat_bytes: int = 4) -> int:
    """Fused: read the kept tiles once, write the whole [S,S] output once.
    Unfused: the five steps touch the score-sized tensor 1+2+2+1+2 = 8 times,
    step three also reads the materialised mask (one more score-sized read),
    and the row max and row sum are each written once and read once."""
    score = BH * S * S
    if fused:
        return (BH * softmax_elements_read(S, tile) + score) * elem_bytes
    steps = [("max", 1, 0), ("sub", 1, 1), ("exp_mask", 1, 1), ("sum", 1, 0), ("div", 1, 1)]
    touches = sum(r + w for _, r, w in steps)            # 8
    mask_reads = 1
    stats = 4 * BH * S * stat_bytes                      # m: write+read, l: write+read
    return (touches + mask_reads) * score * elem_bytes + stats


def softmax_launches(fused: bool) -> int:
    return 1 if fused else 5


# ---------------------------------------------------------------- RMSNorm

RMSNORM_PASSES = ("square", "mean", "scale by 1/rms", "gain")


def rmsnorm_bytes(n: int, fused: bool, elem_bytes: int = 4) -> int:
    """The appendix ledger's RMSNorm count ("AIGC 基本功", section 3.2): the
    unfused form is four passes (square, mean, multiply by the reciprocal
    root, multiply by the gain), each counted as one read and one write of the
    n-element tensor; fused, one pass reads x and writes y."""
    passes = 1 if fused else len(RMSNORM_PASSES)
    return passes * 2 * n * elem_bytes
