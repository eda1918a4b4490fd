"""Oracle for the planning half of the path: histogram, Theorem-1 plan, route.

Test infrastructure only (see ``oracle/__init__.py``).

Notation follows the pages: E experts, R EP ranks, S tokens per rank, K
distinct experts per token, so every rank must end up with exactly S*K token
slots ([K3-blog] "MoonEP：从「完全平衡」这个目标出发"; [TSR] §6.4).  Rank r
owns the E/R experts ``[r*n, (r+1)*n)``, n = E/R: the weight tensor keeps E/R
rows per rank in rank order ([MoonEP-news] "核心思想：动态冗余专家", rows
[0, E)).  Token t of source rank r_s is global token ``r_s*S + s``; its k-th
routing entry is slot ``i = t*K + k`` (flat (token, k) order of ``topk_ids``).

Readings taken where the pages leave a step open (each also listed in the
design notes):

* donor choice -- the overloaded rank with the largest load, ties to the
  lowest id; receiver -- the lowest-id rank that is currently underloaded
  ([K3-blog] "定理 1" says only "pick one of each");
* the donor gives its own experts in ascending id, continuing across its
  donations, and within an expert the earliest slots (in (token, k) order)
  that it still holds; experts it no longer holds slots of are skipped;
* a receiver's redundant experts are the distinct experts of its one fill,
  ascending; prefetch slot b holds the b-th of them; in inference mode the
  ones beyond B are "overflow" and keep the home weight row e
  ([MoonEP-news] "核心思想", B policy);
* per rank, the S*K buffer is grouped by weight row j in ascending order
  (home rows j < E, overflow rows j < E, prefetch rows E+b), and inside a
  segment slots stay in ascending (token, k) order;
* cu_seqlens has E+B+1 entries per rank: cu[0] = 0, cu[E+B] = S*K.

Parity: exact integer results.  Pinned by tests/test_oracle_plan.py:
invariants of Theorem 1 and its lemma ([MoonEP-fr] "Le théorème"), the
Theorem-2 bound, worked examples in tests/golden/, an independent slot-queue
simulation of the same rules on small inputs, and brute-force optima.
"""
from dataclasses import dataclass

import numpy as np

STATUS_BAD_ID = 1        # an id outside [0, E) was seen
STATUS_UNBALANCED = 2    # loads do not sum to R*S*K (only with bad ids)
STATUS_CAPACITY = 4      # train mode needed more than B prefetch slots


@dataclass(frozen=True)
class Cfg:
    R: int
    S: int
    E: int
    K: int
    H: int
    Hp: int
    B: int
    mode: int = 0        # 0 = train, 1 = inference

    @property
    def n(self):
        return self.E // self.R

    @property
    def SK(self):
        return self.S * self.K


@dataclass
class Plan:
    counts: np.ndarray        # [E]            T_e
    load0: np.ndarray         # [R]            initial per-rank load
    rank_in_expert: np.ndarray  # [R*S*K]      p_i = #{j < i : id_j = id_i}
    moves: np.ndarray         # [n_moves, 4]   (e, dst, lo, hi) in fill order
    fills: list               # [(u, o, first_move, end_move)] in fill order
    taken: np.ndarray         # [E]            slots of e moved away from home
    n_redundant: np.ndarray   # [R]
    src_rank: np.ndarray      # [R]            single donor, or -1
    slot_expert: np.ndarray   # [R, B]         expert in prefetch slot, or -1
    seg_len: np.ndarray       # [R, E+B]       rows of each weight row per rank
    cu_seqlens: np.ndarray    # [R, E+B+1]
    route: np.ndarray         # [R*S*K]        destination row r*S*K + offset
    status: int = 0


def histogram(topk_ids, E):
    """T_e = number of routing entries that name expert e.

    [MoonEP-news] "MoonEP 针对的问题": T_e is the token count routed to e.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    return np.bincount(ids, minlength=E).astype(np.int64)


def home_loads(counts, R):
    """Initial load of rank r = sum of T_e over its E/R home experts.

    [K3-blog] "定理 1": ranks are classed by their local token count.
    """
    n = len(counts) // R
    return np.asarray(counts, np.int64).reshape(R, n).sum(axis=1)


def stable_rank(topk_ids, E):
    """p_i = number of earlier slots (flat (token, k) order) naming id_i."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    order = np.argsort(ids, kind="stable")
    counts = np.bincount(ids, minlength=E)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    p = np.empty(len(ids), dtype=np.int64)
    p[order] = np.arange(len(ids)) - start[ids[order]]
    return p


POLICY_ASCENDING, POLICY_LARGEST = 0, 1


def theorem1_fills(counts, cfg, policy=POLICY_ASCENDING):
    """The constructive procedure of Theorem 1, made deterministic.

    [K3-blog] "定理 1" / [MoonEP-fr] "Le théorème": while some rank holds
    fewer than S*K slots, pick an underloaded rank u and an overloaded rank
    o and move slots from o to u until u holds exactly S*K; o may stay
    overloaded, become balanced, or become underloaded and go back to the
    pool.  Each fill balances one rank for good, so there are at most R-1
    fills, and each receiver's remote slots come from a single rank.

    Which of the donor's home experts give the slots:
      POLICY_ASCENDING -- ascending id, continuing from where the donor's
        previous donation stopped (the construction as the proof states it);
      POLICY_LARGEST -- the expert with the most slots still at home first
        (ties: lowest id), then the next, until the need is met.  Theorem 1
        allows any subset of the donor's experts (the lemma only needs a
        single donor); the pages' planner is a near-optimal heuristic checked
        against an offline integer program ([MoonEP-fr] "La planification en
        ligne"), and taking big experts first needs fewer distinct experts.
    Either way an expert gives its earliest slots still at home, and a
    fill's moves are listed in ascending expert id.

    Returns (moves, fills, taken) where a move (e, u, lo, hi) gives u the
    slots of expert e with in-expert rank p in [lo, hi).
    """
    R, E, n, SK = cfg.R, cfg.E, cfg.n, cfg.SK
    T = [int(c) for c in counts]
    load = [int(v) for v in home_loads(counts, R)]
    taken = [0] * E
    cursor = [r * n for r in range(R)]       # next home expert the donor gives
    moves, fills = [], []
    while True:
        under = [r for r in range(R) if load[r] < SK]
        if not under:
            break
        u = min(under)
        o = max(range(R), key=lambda r: (load[r], -r))
        if load[o] <= SK:                    # cannot happen when sum = R*S*K
            raise ValueError("no overloaded rank while %d is underloaded" % u)
        need = SK - load[u]
        d = need
        first = len(moves)
        if policy == POLICY_LARGEST:
            rem = {e: T[e] - taken[e] for e in range(o * n, (o + 1) * n)}
            take = {}
            while d > 0:
                e = max(rem, key=lambda x: (rem[x], -x))
                if rem[e] == 0:
                    raise AssertionError("donor ran out of home slots")
                m = min(d, rem[e])
                take[e] = m
                rem[e] -= m
                d -= m
            for e in sorted(take):
                moves.append((e, u, taken[e], taken[e] + take[e]))
                taken[e] += take[e]
        while d > 0:
            e = cursor[o]
            # a donor never received slots, so its load is its remaining home
            # slots, which exceed S*K > d: it cannot run out here
            if e >= (o + 1) * n:
                raise AssertionError("donor ran out of home slots")
            avail = T[e] - taken[e]
            if avail == 0:
                cursor[o] += 1
                continue
            m = min(d, avail)
            moves.append((e, u, taken[e], taken[e] + m))
            taken[e] += m
            d -= m
            if taken[e] == T[e]:
                cursor[o] += 1
        fills.append((u, o, first, len(moves)))
        load[o] -= need
        load[u] = SK
    mv = np.array(moves, dtype=np.int64).reshape(-1, 4)
    return mv, fills, np.array(taken, dtype=np.int64)


def make_plan(topk_ids, cfg, policy=POLICY_ASCENDING):
    """Full plan: histogram, fills, slot map, cu_seqlens and route.

    [K3-blog] "在线规划、零拷贝、静态 shape": the planner fixes every token's
    destination, so permute writes each row straight into its expert-grouped
    place on the destination rank.  [MoonEP-news] "核心思想": cu_seqlens over
    the E+B weight rows selects the active rows; rows [E, E+B) are the local
    prefetch slots; in inference B < E/R and extra experts are read from
    their home rows.
    """
    R, E, B, SK, n = cfg.R, cfg.E, cfg.B, cfg.SK, cfg.n
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    if ids.size != R * cfg.S * cfg.K:
        raise ValueError("topk_ids must hold R*S*K entries")
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    T = histogram(ids, E)
    load0 = home_loads(T, R)
    p = stable_rank(ids, E)
    moves, fills, taken = theorem1_fills(T, cfg, policy)

    n_red = np.zeros(R, np.int64)
    src = np.full(R, -1, np.int64)
    slot_expert = np.full((R, B), -1, np.int64)
    seg_len = np.zeros((R, E + B), np.int64)
    status = 0
    # row of each move on its receiver: prefetch row E+b, or the home row e
    # when b >= B (inference overflow)
    move_row = np.zeros(len(moves), np.int64)
    for (u, o, m0, m1) in fills:
        n_red[u] = m1 - m0
        src[u] = o
        for b, m in enumerate(range(m0, m1)):
            e, _, lo, hi = moves[m]
            row = E + b if b < B else e
            if b < B:
                slot_expert[u, b] = e
            elif cfg.mode == 0:
                status |= STATUS_CAPACITY
            move_row[m] = row
            seg_len[u, row] += hi - lo
    for e in range(E):
        seg_len[e // n, e] += T[e] - taken[e]
    cu = np.zeros((R, E + B + 1), np.int64)
    cu[:, 1:] = np.cumsum(seg_len, axis=1)
    assert np.all(cu[:, -1] == SK)

    # route: slots of expert e in p order; the first taken[e] went away in
    # the moves of e (ascending lo), the rest stay home after offset taken[e]
    route = np.full(ids.size, -1, np.int64)
    by_expert = np.argsort(ids, kind="stable")          # slot indices, p order
    start = np.concatenate([[0], np.cumsum(T)])
    for e in range(E):
        slots_e = by_expert[start[e]:start[e + 1]]
        h = e // n
        keep = slots_e[taken[e]:]
        route[keep] = h * SK + cu[h, e] + np.arange(len(keep))
    for m, (e, u, lo, hi) in enumerate(moves):
        slots_e = by_expert[start[e]:start[e + 1]]
        route[slots_e[lo:hi]] = u * SK + cu[u, move_row[m]] + np.arange(hi - lo)
    return Plan(counts=T, load0=load0, rank_in_expert=p, moves=moves,
                fills=fills, taken=taken, n_redundant=n_red, src_rank=src,
                slot_expert=slot_expert, seg_len=seg_len, cu_seqlens=cu,
                route=route, status=status)


def failed_plan(topk_ids, cfg):
    """The plan state when the ids cannot be planned: no plan at all.

    The pages define the planner for valid router output only; an id outside
    [0, E) has no expert to go to.  Reading taken for the library's error
    contract: the ids that name a real expert are still counted (T_e and the
    home loads over them), but nothing is moved and no slot gets a place --
    no fills, every rank's buffer empty (cu_seqlens all zero), no prefetch
    slot in use, every route -1 -- and the status carries STATUS_BAD_ID and,
    since the valid slots then fall short of R*S*K, STATUS_UNBALANCED.  Every
    later step then has no routes and no segments to work on.
    """
    R, E, B = cfg.R, cfg.E, cfg.B
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    if ids.size != R * cfg.S * cfg.K:
        raise ValueError("topk_ids must hold R*S*K entries")
    ok = (ids >= 0) & (ids < E)
    if ok.all():
        raise ValueError("every id is valid: use make_plan")
    T = histogram(ids[ok], E)
    return Plan(counts=T, load0=home_loads(T, R),
                rank_in_expert=np.full(ids.size, -1, np.int64),
                moves=np.zeros((0, 4), np.int64), fills=[], taken=np.zeros(E, np.int64),
                n_redundant=np.zeros(R, np.int64), src_rank=np.full(R, -1, np.int64),
                slot_expert=np.full((R, B), -1, np.int64),
                seg_len=np.zeros((R, E + B), np.int64),
                cu_seqlens=np.zeros((R, E + B + 1), np.int64),
                route=np.full(ids.size, -1, np.int64),
                status=STATUS_BAD_ID | STATUS_UNBALANCED)
