"""Plain CPU oracle of expert-parallel load balancing (EPLB): replicas of hot
experts, their placement on ranks, and the routing of token slots to replicas.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
library (whose planner is C++ and whose remap is a HIP kernel); both sides
receive the same inputs and nothing else.

What the pages fix
------------------
* "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
  "Routing imbalance": measure per-expert token counts; the busiest GPU's
  token count over the mean is the imbalance factor (worth acting on above
  about 1.3); replicate hot experts, putting the redundant copies on
  less-loaded GPUs; without replication, co-locating hot and cold experts
  already evens out the per-GPU load.
* "Serve MoE models with expert parallelism" (aiengineeringfromscratch),
  list of serving features: the load balancer moves busy experts so that the
  load spreads.
* flatkey.ai vLLM expert-parallel deployment page, section on EPLB: the
  balancer gathers load statistics over a window and periodically remaps
  experts to ranks; its knobs include the number of redundant experts.

The pages give no algorithm.  The reading taken here, in the order the pages
name the steps:

1. Replication.  ``P = E + R`` physical expert slots on ``G`` ranks, ``S = P/G``
   per rank (``P`` divisible by ``G``).  Every expert has one copy; each of the
   ``R`` redundant copies in turn goes to the expert whose load per copy,
   ``load[e] / replicas[e]``, is largest (exact rational comparison; ties to
   the lower expert id), among experts with fewer than ``G`` copies.
2. Placement.  A copy of expert e carries ``load[e] / replicas[e]`` (float64).
   Copies are taken heaviest first (ties: lower expert id, then lower copy
   index) and each goes to the least-loaded rank (float64 sum of the copies
   placed on it so far, in placement order; ties to the lower rank) among
   the ranks that still have a free slot and hold no copy of the same
   expert; if every rank with a free slot already holds one, the least-loaded
   rank with a free slot takes it.  Heaviest-first onto the least-loaded rank
   is what puts hot and cold experts together.
3. Numbering.  Rank g's slots are physical ids ``g*S .. g*S + S - 1``, holding
   its experts in increasing expert id (copies of one expert on one rank in
   increasing copy index).  ``log_to_phys[e, j]`` is the physical id of copy j
   of expert e, copies numbered in increasing physical id; unused entries -1.
4. Routing to copies.  The slot (t, i) routed to expert e goes to copy
   ``t mod replicas[e]`` (a fixed rule, so that a token's slots and hence the
   layer output do not depend on the plan).

The contiguous placement without copies (rank g holds experts
``g*E/G .. (g+1)*E/G - 1``) is the baseline the pages measure against.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = ["plan", "contiguous_rank_of_expert", "remap", "rank_slot_counts",
           "imbalance_factor", "predicted_rank_loads"]


def _check(load, G: int, R: int):
    E = len(load)
    if E < 1 or G < 1 or R < 0 or (E + R) % G != 0 or R > E * (G - 1):
        raise ValueError("need E >= 1, G >= 1, 0 <= R <= E (G - 1), (E + R) divisible by G")
    if any(int(c) < 0 for c in load):
        raise ValueError("loads are counts (>= 0)")
    return E


def plan(load, G: int, R: int):
    """Steps 1-3 of the module docstring.

    Returns ``(replicas [E] int32, phys_to_log [E+R] int32,
    log_to_phys [E, G] int32 (-1 padded), rank_load [G] float64)``.
    """
    E = _check(load, G, R)
    load = [int(c) for c in load]
    P = E + R
    S = P // G
    # 1. replication: R times, the largest exact load per copy gets a copy
    rep = [1] * E
    for _ in range(R):
        best = -1
        for e in range(E):
            if rep[e] >= G:
                continue
            if best < 0 or Fraction(load[e], rep[e]) > Fraction(load[best], rep[best]):
                best = e
        rep[best] += 1
    # 2. placement: heaviest copy first onto the least-loaded eligible rank
    copies = [(load[e] / rep[e], e, j) for e in range(E) for j in range(rep[e])]
    copies.sort(key=lambda c: (-c[0], c[1], c[2]))
    rank_load = [0.0] * G
    held = [[] for _ in range(G)]  # (expert, copy) per rank, in placement order
    for w, e, j in copies:
        free = [g for g in range(G) if len(held[g]) < S]
        fresh = [g for g in free if all(e2 != e for e2, _ in held[g])]
        cand = fresh if fresh else free
        g_best = cand[0]
        for g in cand[1:]:
            if rank_load[g] < rank_load[g_best]:
                g_best = g
        held[g_best].append((e, j))
        rank_load[g_best] += w
    # 3. numbering
    phys_to_log = np.empty(P, dtype=np.int32)
    phys_copy = []
    for g in range(G):
        for slot, (e, j) in enumerate(sorted(held[g])):
            phys_to_log[g * S + slot] = e
            phys_copy.append((e, g * S + slot))
    log_to_phys = np.full((E, G), -1, dtype=np.int32)
    for e in range(E):
        ps = sorted(p for e2, p in phys_copy if e2 == e)
        log_to_phys[e, :len(ps)] = ps
    return (np.asarray(rep, dtype=np.int32), phys_to_log, log_to_phys,
            np.asarray(rank_load, dtype=np.float64))


def contiguous_rank_of_expert(E: int, G: int) -> np.ndarray:
    """The baseline placement: expert e on rank e // (E / G) (E divisible by G)."""
    if E % G:
        raise ValueError("E must be divisible by G")
    return np.arange(E) // (E // G)


def remap(topk_idx: np.ndarray, replicas: np.ndarray, log_to_phys: np.ndarray) -> np.ndarray:
    """Step 4: logical ids [T, k] -> physical ids [T, k]; slot (t, i) of expert e
    goes to copy t mod replicas[e].  Ids outside [0, E) map to -1."""
    T, k = topk_idx.shape
    E = len(replicas)
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        for i in range(k):
            e = int(topk_idx[t, i])
            if 0 <= e < E:
                out[t, i] = log_to_phys[e, t % int(replicas[e])]
    return out


def rank_slot_counts(ids: np.ndarray, rank_of: np.ndarray, G: int) -> np.ndarray:
    """Token slots per rank: ``ids`` are (physical or logical) expert ids,
    ``rank_of[id]`` their rank; ids < 0 are ignored."""
    counts = np.zeros(G, dtype=np.int64)
    for e in ids.reshape(-1):
        if e >= 0:
            counts[rank_of[e]] += 1
    return counts


def imbalance_factor(rank_loads) -> float:
    """The pages' imbalance factor: busiest rank's load over the mean load."""
    r = np.asarray(rank_loads, dtype=np.float64)
    m = r.mean()
    return float(r.max() / m) if m > 0 else 1.0


def predicted_rank_loads(load, replicas, phys_to_log, G: int) -> np.ndarray:
    """Exact (rational) rank loads of a plan, each copy carrying load / replicas."""
    P = len(phys_to_log)
    S = P // G
    out = []
    for g in range(G):
        s = Fraction(0)
        for p in range(g * S, (g + 1) * S):
            e = int(phys_to_log[p])
            s += Fraction(int(load[e]), int(replicas[e]))
        out.append(s)
    return np.asarray([float(v) for v in out])
