"""Host-side RoundPipe algorithms, stated plainly -- TEST INFRASTRUCTURE ONLY.

* bubble formula and a brute-force schedule simulator (RoundPipe paper,
  section 3.2 "Round-robin dispatch" and section 3.3 "Bubble Analysis");
* partition objective, the O(L^3) candidate + greedy partitioner and an
  exhaustive search (section 4.4.1 "Problem Formulation", 4.4.2 "Algorithm");
* longest-processing-time-first packing of parameter/gradient transfers into
  data-transfer windows, with splitting of oversized tensors (section 4.2.2),
  and a brute-force optimum for checking Graham's bound;
* the per-layer activation-memory model (appendix B.1 of the paperlayer.ai
  summary).

Readings where the pages are silent:

* simulator: stage slot k (counted across rounds, forward slots then backward
  slots) runs on GPU k mod N; inside a slot the round's micro-batches run in
  order; micro-batch j of slot i waits for micro-batch j of slot i-1 of the
  same round and for its GPU; no dependency between rounds (gradient
  accumulation / staleness-1 optimizer); transfer time zero;
* partitioner: the units are the L layers plus the LM head, which always sits
  in the fused first backward stage B_1. A forward stage costs the sum of its
  layers' forward times, a backward stage the sum of their backward times
  (recompute included), the fused stage h + sum of its layers' backward times
  (its forward doubles as the recompute). Memory is additive per stage and
  capped. B_1 >= 1;
* LPT: windows = micro-batches of the stage; a tensor larger than
  ceil(total / windows) (or than an optional absolute cap) is cut into chunks
  of that threshold rounded up to the alignment, the last chunk taking the
  remainder; chunks are sorted by size descending (stable) and each goes to
  the least-loaded window (ties: lowest window index).
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from typing import List, Sequence, Tuple

# ---------------------------------------------------------------------------
# bubble ratio (section 3.3)
# ---------------------------------------------------------------------------


def bubble_formula(n_gpus: int, n_micro: int, n_stages: int) -> Fraction:
    """N(N-1) / (M S + N(N-1)), exact rational."""
    N, M, S = n_gpus, n_micro, n_stages
    return Fraction(N * (N - 1), M * S + N * (N - 1))


def simulate_roundpipe(n_gpus: int, n_micro: int, per_round: int, n_stages: int,
                       stage_times: Sequence[Fraction] | None = None):
    """Event simulation of the round-robin dispatch; returns (makespan, busy, bubble).

    stage_times[i] is the per-micro-batch time of stage slot i (default 1).
    """
    N, M, MR, S = n_gpus, n_micro, per_round, n_stages
    if M % MR:
        raise ValueError("micro-batches must be a whole number of rounds")
    t = [Fraction(1)] * S if stage_times is None else [Fraction(x) for x in stage_times]
    R = M // MR
    gpu_free = [Fraction(0)] * N
    finish_prev_slot = None
    busy = Fraction(0)
    makespan = Fraction(0)
    for r in range(R):
        for i in range(S):
            g = (r * S + i) % N
            fin = []
            for j in range(MR):
                ready = finish_prev_slot[j] if i > 0 else Fraction(0)
                start = max(ready, gpu_free[g])
                end = start + t[i]
                gpu_free[g] = end
                fin.append(end)
                busy += t[i]
            finish_prev_slot = fin
            makespan = max(makespan, fin[-1])
    bubble = (N * makespan - busy) / (N * makespan)
    return makespan, busy, bubble


# ---------------------------------------------------------------------------
# partitioner (section 4.4)
# ---------------------------------------------------------------------------


def objective(n_micro: int, n_gpus: int, n_stages: int, t_max) -> float:
    """(M S + N (N-1)) t_max -- total GPU time under the slowest stage."""
    return (n_micro * n_stages + n_gpus * (n_gpus - 1)) * t_max


def _stage_times(f, b, h, fwd: Sequence[int], b1: int, bwd: Sequence[int]):
    L = len(f)
    times, lo = [], 0
    for n in fwd:
        times.append(sum(f[lo:lo + n]))
        lo += n
    times.append(h + sum(b[L - b1:L]))
    hi = L - b1
    for n in bwd:
        times.append(sum(b[hi - n:hi]))
        hi -= n
    return times


def _stage_mems(mf, mb, mh, fwd, b1, bwd):
    return _stage_times(mf, mb, mh, fwd, b1, bwd)


def _compositions(n: int):
    """All ordered ways to cut n consecutive layers into non-empty groups."""
    if n == 0:
        yield ()
        return
    for cuts in itertools.product([0, 1], repeat=n - 1):
        parts, run = [], 1
        for c in cuts:
            if c:
                parts.append(run)
                run = 1
            else:
                run += 1
        parts.append(run)
        yield tuple(parts)


def partition_exhaustive(f, b, h, mf, mb, mh, cap, n_micro, n_gpus):
    """Minimum objective over every (F_1..F_Sf, B_1) x (B_1..B_Sb) partition."""
    L = len(f)
    best = None
    for b1 in range(1, L + 1):
        rest = L - b1
        for fwd in _compositions(rest):
            for bwd in _compositions(rest):
                mems = _stage_mems(mf, mb, mh, fwd, b1, bwd)
                if max(mems) > cap:
                    continue
                times = _stage_times(f, b, h, fwd, b1, bwd)
                S = len(fwd) + 1 + len(bwd)
                val = objective(n_micro, n_gpus, S, max(times))
                if best is None or val < best[0]:
                    best = (val, fwd, b1, bwd)
    return best


def _greedy_count(vals, mems, t_max, cap):
    """Minimum number of contiguous groups with sum(vals) <= t_max and
    sum(mems) <= cap, packing front to back; None if a single item fails."""
    groups, cur_t, cur_m, cur_n = [], 0, 0, 0
    for v, m in zip(vals, mems):
        if v > t_max or m > cap:
            return None
        if cur_n and (cur_t + v > t_max or cur_m + m > cap):
            groups.append(cur_n)
            cur_t, cur_m, cur_n = 0, 0, 0
        cur_t += v
        cur_m += m
        cur_n += 1
    if cur_n:
        groups.append(cur_n)
    return tuple(groups)


def partition_greedy(f, b, h, mf, mb, mh, cap, n_micro, n_gpus):
    """Candidate t_max values: every contiguous sum of f, every contiguous sum
    of b, and h + every suffix sum of b (O(L^2)). Per candidate: the largest
    feasible fused stage B_1, then min-count greedy packing of the remaining
    layers forward (front to back) and backward (back to front), O(L).
    Returns (objective, fwd groups, B_1, bwd groups)."""
    L = len(f)
    cands = set()
    for i in range(L):
        sf = sb = 0
        for j in range(i, L):
            sf += f[j]
            sb += b[j]
            cands.add(sf)
            cands.add(sb)
    suf = 0
    for j in reversed(range(L)):
        suf += b[j]
        cands.add(h + suf)
    best = None
    for t0 in sorted(cands):
        # a stage fits when its time is at most t0 up to summation order: a
        # group summed in another order than the candidate can exceed it by a
        # few ulps, and exactly equal times fit
        t = t0 * (1 + 1e-12)
        b1, tt, mm = 0, h, mh
        for j in reversed(range(L)):
            if tt + b[j] <= t and mm + mb[j] <= cap:
                tt += b[j]
                mm += mb[j]
                b1 += 1
            else:
                break
        if b1 == 0 or h > t or mh > cap:
            continue
        rest = L - b1
        fwd = _greedy_count(f[:rest], mf[:rest], t, cap)
        bwd = _greedy_count(list(reversed(b[:rest])), list(reversed(mb[:rest])), t, cap)
        if fwd is None or bwd is None:
            continue
        times = _stage_times(f, b, h, fwd, b1, bwd)
        S = len(fwd) + 1 + len(bwd)
        val = objective(n_micro, n_gpus, S, max(times))
        if best is None or val < best[0]:
            best = (val, fwd, b1, bwd)
    return best


# ---------------------------------------------------------------------------
# LPT window packing (section 4.2.2)
# ---------------------------------------------------------------------------


def split_items(sizes: Sequence[int], n_windows: int, align: int = 1,
                max_chunk: int = 0) -> List[Tuple[int, int, int]]:
    """Cut oversized tensors into chunks: returns (item, offset, bytes) in item order."""
    total = sum(sizes)
    thresh = -(-total // max(n_windows, 1))
    if max_chunk > 0:
        thresh = min(thresh, max_chunk)
    thresh = max(thresh, 1)
    out = []
    for i, s in enumerate(sizes):
        if s <= thresh:
            out.append((i, 0, s))
            continue
        n = -(-s // thresh)
        c = -(-s // n)
        c = -(-c // align) * align
        off = 0
        while off < s:
            n_b = min(c, s - off)
            out.append((i, off, n_b))
            off += n_b
    return out


def lpt_assign(sizes: Sequence[int], n_windows: int) -> List[int]:
    """Window index per item: sort by size descending (stable), each item to
    the window with the least assigned bytes (ties: lowest index)."""
    order = sorted(range(len(sizes)), key=lambda i: -sizes[i])
    load = [0] * n_windows
    win = [0] * len(sizes)
    for i in order:
        w = min(range(n_windows), key=lambda k: (load[k], k))
        win[i] = w
        load[w] += sizes[i]
    return win


def makespan(sizes: Sequence[int], win: Sequence[int], n_windows: int) -> int:
    load = [0] * n_windows
    for s, w in zip(sizes, win):
        load[w] += s
    return max(load)


def optimal_makespan(sizes: Sequence[int], n_windows: int) -> int:
    """Brute force over all n_windows ** len(sizes) assignments."""
    best = None
    for win in itertools.product(range(n_windows), repeat=len(sizes)):
        v = makespan(sizes, win, n_windows)
        if best is None or v < best:
            best = v
    return best


# ---------------------------------------------------------------------------
# activation memory (appendix B.1)
# ---------------------------------------------------------------------------


def activation_bytes_per_layer(s: int, b: int, h: int, h_kv: int, m: int, e_act: int = 1) -> int:
    """16-bit activations a layer stores for backward without recomputation:
    two norms 4sbh; attention 6sbh + 4sbh_kv (shared QKV input, Q, K, V and
    output for flash attention); MLP 2sbh + 6sbm*E_act (inputs of its linears
    and of SwiGLU)."""
    norms = 4 * s * b * h
    attn = 6 * s * b * h + 4 * s * b * h_kv
    mlp = 2 * s * b * h + 6 * s * b * m * e_act
    return norms + attn + mlp


def checkpoint_bytes_per_layer(s: int, b: int, h: int) -> int:
    """With full recomputation only the layer input is kept: 2sbh bytes."""
    return 2 * s * b * h
