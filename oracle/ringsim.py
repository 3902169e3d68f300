"""Simulator of the full/empty ring protocol between producer and consumer waves.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What it models (pages on warp specialization):
  * a ring of S staging buffers; tile t goes through buffer t mod S
    ("Producer-Consumer Warp Specialization for TMA Operations", the
    paragraph enumerating tiles 0..3 over buffers 0, 1, 0, 1; the pwwt.cn
    article, section 3.4, uses tile % stages);
  * two barriers per buffer, "full" (data landed) and "empty" (data drained)
    (same post; pwwt.cn section 3.4 argues one barrier per stage is not
    enough);
  * a barrier is a counter with an expected number of arrivals; the last
    arrival completes the phase, flips the phase bit and re-arms the count
    (pwwt.cn section 2.2);
  * wait(p) proceeds once the phase of parity p has completed, i.e. once the
    phase bit differs from p: wait(0) passes on a 0->1 flip, wait(1) on a 1->0
    flip; for tile t the full wait uses p = (t / S) & 1 (the post's phase-bit
    paragraphs, which print the two-buffer case t / 2);
  * producers: wait for a free buffer, fill it, signal full; consumers: wait
    for a full buffer, use it, signal empty (aicassindra "GPU warp
    specialization", sections "The architecture: every piece explained" and
    "End-to-end flow").

Readings where the pages are silent or garbled:
  * the post writes the buffer index as i/2 yet enumerates i mod 2; the
    enumeration and the pwwt.cn pseudo-code agree on t mod S;
  * the empty wait of tile t waits for the release of tile t - S, i.e. parity
    ((t / S) & 1) ^ 1, which passes at once on a fresh barrier for t < S;
  * flags start at phase 0 with the full expected count pending;
  * with several waves per role, full completes after all P producer waves
    arrived for that tile and empty after all C consumer waves released it.

Modes: `explore` enumerates every interleaving of the atomic steps and checks
safety (no read before fill, no overwrite before release, slot in range, no
wait that passes on a stale or future phase) and liveness (no reachable
deadlock); `timed` runs the same loops with a load latency and a compute time.
"""
from __future__ import annotations

import dataclasses
import random
from typing import Dict, List, Optional, Tuple

# Protocol variants. "standard" is the protocol as read from the pages; the
# others are mistakes the checker must catch.
VARIANTS = (
    "standard",
    "one_barrier",          # a single barrier per buffer for both directions
    "empty_same_parity",    # empty wait with (t/S)&1, i.e. no released first lap
    "slot_div2",            # buffer index t // 2 as printed, instead of t mod 2
    "drop_release",         # consumer 0 never releases tile 0
    "no_empty_wait",        # producer never waits for a free buffer
    "full_parity_flipped",  # consumer waits full with ((t/S)&1) ^ 1
)


def slot_of(t: int, S: int, variant: str = "standard") -> int:
    """Buffer used by tile t."""
    if variant == "slot_div2":
        return t // 2
    return t % S


def full_parity(t: int, S: int, variant: str = "standard") -> int:
    """Parity a consumer passes to the full-barrier wait for tile t."""
    p = (t // S) & 1
    return p ^ 1 if variant == "full_parity_flipped" else p


def empty_parity(t: int, S: int, variant: str = "standard") -> int:
    """Parity a producer passes to the empty-barrier wait for tile t."""
    p = (t // S) & 1
    return p if variant == "empty_same_parity" else p ^ 1


def schedule(S: int, T: int, variant: str = "standard") -> List[Tuple[int, int, int, int]]:
    """(tile, buffer, full-wait parity, empty-wait parity) for tiles 0..T-1."""
    return [(t, slot_of(t, S, variant), full_parity(t, S, variant), empty_parity(t, S, variant))
            for t in range(T)]


class ProtocolViolation(AssertionError):
    pass


@dataclasses.dataclass(frozen=True)
class Result:
    states: int
    deadlock: bool
    violation: Optional[str]
    max_lead: int           # largest (tiles filled) - (tiles fully released) seen
    reach_pairs: frozenset  # (tile a consumer holds, newest tile a producer has begun)


# ---------------------------------------------------------------------------
# Barrier: (phase bit, pending arrivals, completed phases)
# ---------------------------------------------------------------------------

def _arrive(flag: Tuple[int, int, int], expected: int) -> Tuple[int, int, int]:
    phase, pending, done = flag
    pending -= 1
    if pending == 0:
        return (phase ^ 1, expected, done + 1)
    return (phase, pending, done)


def _may_pass(flag: Tuple[int, int, int], parity: int) -> bool:
    return flag[0] != parity


# A second encoding of the same barrier, for expected counts that are powers
# of two: a plain arrival counter whose bit log2(E) is the phase bit. The
# simulator runs either encoding through the same checks; ("counter", c)
# flags are adapted to the (phase, pending, completed) view below.

def _counter_view(count: int, expected: int) -> Tuple[int, int, int]:
    shift = expected.bit_length() - 1
    return ((count >> shift) & 1, expected - (count % expected), count // expected)


def _is_pow2(x: int) -> bool:
    return x > 0 and (x & (x - 1)) == 0


def _pow2_at_least(x: int) -> int:
    e = 1
    while e < x:
        e *= 2
    return e


# ---------------------------------------------------------------------------
# Exhaustive interleavings
# ---------------------------------------------------------------------------
# Producer steps per tile: 0 wait empty, 1 write its share of the buffer,
# 2 arrive on full. Consumer steps per tile: 0 wait full, 1 read the buffer,
# 2 arrive on empty. Every step is one atomic scheduling point.

def explore(S: int, T: int, P: int = 1, C: int = 1, variant: str = "standard",
            max_states: int = 5_000_000, encoding: str = "phase", lookahead: int = 0) -> Result:
    """encoding: "phase" (phase bit + pending count) or "counter" (arrival
    counter whose bit log2(E) is the phase bit). With the counter, a role
    whose wave count n is not a power of two counts E = the next power of two
    per phase, and its last wave arrives with weight E - n + 1 (the device's
    seven attention consumers: six add 1, the seventh 2).

    lookahead = 0: each producer fills a buffer and signals it in one go.
    lookahead = D >= 1: asynchronous fills, as on the device: a producer keeps
    up to D tiles issued but not yet signalled; before waiting for the next
    free buffer it completes (the data lands) and signals the oldest one when
    D are in flight, and after the last tile it drains the rest. A buffer is
    checked for overwrite when its fill is issued; its data becomes readable
    only when the fill completes."""
    if variant not in VARIANTS:
        raise ValueError(variant)
    one = variant == "one_barrier"
    exp_full = P + C if one else P
    exp_empty = C
    w_prod = [1] * P  # weight of each wave's arrival (counter encoding)
    w_cons = [1] * C
    if encoding == "counter":
        if one and not _is_pow2(exp_full):
            raise ValueError("the single-barrier counter encoding needs a power-of-two arrival count")
        if not one:
            w_prod[-1] += _pow2_at_least(P) - P
        w_cons[-1] += _pow2_at_least(C) - C

        # flags are stored as raw counters and viewed through _counter_view
        def arrive(flag, expected, w=1):
            return flag + w

        def view(flag, expected):
            return _counter_view(flag, _pow2_at_least(expected))
        init_flag_full = 0
        init_flag_empty = 0
    elif encoding == "phase":
        def arrive(flag, expected, w=1):
            return _arrive(flag, expected)

        def view(flag, expected):
            return flag
        init_flag_full = (0, exp_full, 0)
        init_flag_empty = (0, exp_empty, 0)
    else:
        raise ValueError(encoding)
    # state: (prod pcs, cons pcs, full flags, empty flags, buffer tags)
    # pc = (tile, step); buffer tags: per buffer a tuple of P producer tags
    if lookahead and variant == "one_barrier":
        raise ValueError("lookahead is modelled for the two-barrier protocol only")
    init = (
        tuple(((0, False, 0) if lookahead else (0, 0)) for _ in range(P)),
        tuple((0, 0) for _ in range(C)),
        tuple(init_flag_full for _ in range(S)),
        tuple(init_flag_empty for _ in range(S)),
        tuple(tuple(-1 for _ in range(P)) for _ in range(S)),
    )

    seen = set()
    stack = [init]
    deadlock = False
    violation = None
    max_lead = 0
    reach = set()

    def overwrite_check(i, t, s, conss):
        for c, (tc, sc) in enumerate(conss):
            for tt in range(tc if sc <= 1 else tc + 1, T):
                if tt >= t:
                    break
                if slot_of(tt, S, variant) == s:
                    raise ProtocolViolation(
                        "producer %d overwrote buffer %d with tile %d while consumer %d "
                        "had not yet read tile %d" % (i, s, t, c, tt))

    def producer_moves_async(i, prod, st):
        # prod = (next tile to issue, passed its empty wait?, tiles in flight)
        prods, conss, fulls, empties, bufs = st
        t, waited, inflight = prod
        out = []

        def with_prod(newp, nf=fulls, nb=bufs):
            np_ = list(prods)
            np_[i] = newp
            return (tuple(np_), conss, nf, empties, nb)

        if inflight == lookahead or (t >= T and inflight > 0):
            old = t - inflight
            so = slot_of(old, S, variant)
            nb = list(bufs)
            tags = list(nb[so])
            tags[i] = old
            nb[so] = tuple(tags)
            nf = list(fulls)
            nf[so] = arrive(nf[so], exp_full, w_prod[i])
            out.append(with_prod((t, waited, inflight - 1), tuple(nf), tuple(nb)))
            return out
        if t >= T:
            return out
        s = slot_of(t, S, variant)
        if not 0 <= s < S:
            raise ProtocolViolation("tile %d mapped to buffer %d outside 0..%d" % (t, s, S - 1))
        if not waited:
            ok = True if variant == "no_empty_wait" else _may_pass(view(empties[s], exp_empty),
                                                                  empty_parity(t, S, variant))
            if ok:
                if variant != "no_empty_wait":
                    done = view(empties[s], exp_empty)[2]
                    if done != t // S:
                        raise ProtocolViolation(
                            "producer %d passed the empty wait of tile %d on completion %d, expected %d"
                            % (i, t, done, t // S))
                out.append(with_prod((t, True, inflight)))
            return out
        overwrite_check(i, t, s, conss)
        nb = list(bufs)
        tags = list(nb[s])
        tags[i] = -2  # in transit: not readable until the fill completes
        nb[s] = tuple(tags)
        out.append(with_prod((t + 1, False, inflight + 1), fulls, tuple(nb)))
        return out

    def successors(st):
        prods, conss, fulls, empties, bufs = st
        out = []
        for i, prod in enumerate(prods):
            if lookahead:
                out.extend(producer_moves_async(i, prod, st))
                continue
            t, step = prod
            if t >= T:
                continue
            s = slot_of(t, S, variant)
            if not 0 <= s < S:
                raise ProtocolViolation("tile %d mapped to buffer %d outside 0..%d" % (t, s, S - 1))
            if step == 0:
                if variant == "no_empty_wait":
                    ok = True
                elif one:
                    ok = _may_pass(view(fulls[s], exp_full), empty_parity(t, S))
                else:
                    ok = _may_pass(view(empties[s], exp_empty), empty_parity(t, S, variant))
                if ok:
                    if not one and variant != "no_empty_wait":
                        # the release awaited is that of tile t - S
                        want = t // S
                        done = view(empties[s], exp_empty)[2]
                        if done != want:
                            raise ProtocolViolation(
                                "producer %d passed the empty wait of tile %d on completion %d, expected %d"
                                % (i, t, done, want))
                    np_ = list(prods)
                    np_[i] = (t, 1)
                    out.append((tuple(np_), conss, fulls, empties, bufs))
            elif step == 1:
                # nobody may still have tile t - S (or any other tile) to read in buffer s
                for c, (tc, sc) in enumerate(conss):
                    for tt in range(tc if sc <= 1 else tc + 1, T):
                        if tt >= t:
                            break
                        if slot_of(tt, S, variant) == s:
                            raise ProtocolViolation(
                                "producer %d overwrote buffer %d with tile %d while consumer %d "
                                "had not yet read tile %d" % (i, s, t, c, tt))
                nb = list(bufs)
                tags = list(nb[s])
                tags[i] = t
                nb[s] = tuple(tags)
                np_ = list(prods)
                np_[i] = (t, 2)
                out.append((tuple(np_), conss, fulls, empties, tuple(nb)))
            else:
                nf = list(fulls)
                nf[s] = arrive(nf[s], exp_full, w_prod[i])
                np_ = list(prods)
                np_[i] = (t + 1, 0)
                out.append((tuple(np_), conss, tuple(nf), empties, bufs))
        for j, (t, step) in enumerate(conss):
            if t >= T:
                continue
            s = slot_of(t, S, variant)
            if not 0 <= s < S:
                raise ProtocolViolation("tile %d mapped to buffer %d outside 0..%d" % (t, s, S - 1))
            if step == 0:
                if _may_pass(view(fulls[s], exp_full), full_parity(t, S, variant)):
                    if not one:
                        want = t // S + 1
                        done = view(fulls[s], exp_full)[2]
                        if done != want:
                            raise ProtocolViolation(
                                "consumer %d passed the full wait of tile %d on completion %d, expected %d"
                                % (j, t, done, want))
                    nc = list(conss)
                    nc[j] = (t, 1)
                    out.append((prods, tuple(nc), fulls, empties, bufs))
            elif step == 1:
                if any(tag != t for tag in bufs[s]):
                    raise ProtocolViolation(
                        "consumer %d read buffer %d for tile %d but found tags %s"
                        % (j, s, t, bufs[s]))
                nc = list(conss)
                nc[j] = (t, 2)
                out.append((prods, tuple(nc), fulls, empties, bufs))
            else:
                nc = list(conss)
                nc[j] = (t + 1, 0)
                if variant == "drop_release" and j == 0 and t == 0:
                    out.append((prods, tuple(nc), fulls, empties, bufs))
                elif one:
                    nf = list(fulls)
                    nf[s] = arrive(nf[s], exp_full)
                    out.append((prods, tuple(nc), tuple(nf), empties, bufs))
                else:
                    ne = list(empties)
                    ne[s] = arrive(ne[s], exp_empty, w_cons[j])
                    out.append((prods, tuple(nc), fulls, tuple(ne), bufs))
        return out

    try:
        while stack:
            st = stack.pop()
            if st in seen:
                continue
            seen.add(st)
            if len(seen) > max_states:
                raise RuntimeError("state space above %d states" % max_states)
            prods, conss = st[0], st[1]
            if lookahead:
                filled = min(p[0] - p[2] for p in prods)
                begun = max(p[0] - 1 for p in prods)
            else:
                filled = min(t if step < 2 else t + 1 for t, step in prods) if prods else 0
                begun = max(t if step >= 1 else t - 1 for t, step in prods)
            released = min(t for t, step in conss)
            max_lead = max(max_lead, filled - released)
            for t, step in conss:
                if step in (1, 2) and t < T:
                    reach.add((t, begun))
            succ = successors(st)
            if not succ:
                prods_done = all((p[0] >= T and p[2] == 0) if lookahead else p[0] >= T for p in prods)
                if not prods_done or not all(t >= T for t, _ in conss):
                    deadlock = True
                continue
            stack.extend(succ)
    except ProtocolViolation as e:
        violation = str(e)
    return Result(states=len(seen), deadlock=deadlock, violation=violation,
                  max_lead=max_lead, reach_pairs=frozenset(reach))


def random_runs(S: int, T: int, P: int, C: int, runs: int, seed: int,
                variant: str = "standard") -> Optional[str]:
    """Seeded random schedules for larger T; returns the first problem found."""
    rng = random.Random(seed)
    for _ in range(runs):
        # a random walk through the same transition system
        one = variant == "one_barrier"
        exp_full = P + C if one else P
        prods = [[0, 0] for _ in range(P)]
        conss = [[0, 0] for _ in range(C)]
        fulls = [(0, exp_full, 0) for _ in range(S)]
        empties = [(0, C, 0) for _ in range(S)]
        bufs = [[-1] * P for _ in range(S)]
        while True:
            moves = []
            for i, (t, step) in enumerate(prods):
                if t >= T:
                    continue
                s = slot_of(t, S, variant)
                if step == 0:
                    ok = True if variant == "no_empty_wait" else _may_pass(
                        fulls[s] if one else empties[s], empty_parity(t, S, variant))
                    if ok:
                        moves.append(("p", i))
                else:
                    moves.append(("p", i))
            for j, (t, step) in enumerate(conss):
                if t >= T:
                    continue
                s = slot_of(t, S, variant)
                if step == 0:
                    if _may_pass(fulls[s], full_parity(t, S, variant)):
                        moves.append(("c", j))
                else:
                    moves.append(("c", j))
            if not moves:
                if all(t >= T for t, _ in prods) and all(t >= T for t, _ in conss):
                    break
                return "deadlock"
            kind, idx = rng.choice(moves)
            if kind == "p":
                t, step = prods[idx]
                s = slot_of(t, S, variant)
                if not 0 <= s < S:
                    return "buffer index out of range"
                if step == 0:
                    prods[idx][1] = 1
                elif step == 1:
                    for tc, sc in conss:
                        first_unread = tc if sc <= 1 else tc + 1
                        for tt in range(first_unread, t):
                            if slot_of(tt, S, variant) == s:
                                return "overwrite before release"
                    bufs[s][idx] = t
                    prods[idx][1] = 2
                else:
                    fulls[s] = _arrive(fulls[s], exp_full)
                    prods[idx] = [t + 1, 0]
            else:
                t, step = conss[idx]
                s = slot_of(t, S, variant)
                if not 0 <= s < S:
                    return "buffer index out of range"
                if step == 0:
                    conss[idx][1] = 1
                elif step == 1:
                    if any(tag != t for tag in bufs[s]):
                        return "read before fill"
                    conss[idx][1] = 2
                else:
                    if not (variant == "drop_release" and idx == 0 and t == 0):
                        if one:
                            fulls[s] = _arrive(fulls[s], exp_full)
                        else:
                            empties[s] = _arrive(empties[s], C)
                    conss[idx] = [t + 1, 0]
    return None


# ---------------------------------------------------------------------------
# Timed mode
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Timeline:
    issue: List[float]
    land: List[float]
    start: List[float]
    end: List[float]
    release: List[float]
    consumer_wait: float
    producer_wait: float
    stages: int

    def period(self) -> float:
        """Mean time per tile over the whole laps of the ring in the second half.

        Starts within one lap can be bunched, so the average is taken between
        two starts a whole number of laps apart.
        """
        n, S = len(self.start), self.stages
        a = n // 2
        laps = (n - 1 - a) // S
        if laps < 1:
            raise ValueError("need at least one full lap after the midpoint")
        b = a + laps * S
        return (self.start[b] - self.start[a]) / (b - a)


def timed(S: int, T: int, L: float, c: float, release_after: float | None = None,
          jitter: float = 0.0, seed: int = 0) -> Timeline:
    """Event times of one producer and one consumer over T tiles.

    The producer issues the fetch of tile t as soon as buffer t mod S has been
    released by tile t - S (issuing is asynchronous, so several fetches are in
    flight); the data lands L later and completes the full barrier. The
    consumer starts tile t once it has landed and tile t - 1 is done, computes
    for c, and releases the buffer `release_after` after it started (default:
    when the compute ends).
    """
    rng = random.Random(seed)
    r = c if release_after is None else release_after
    issue, land, start, end, rel = [], [], [], [], []
    cw = pw = 0.0
    for t in range(T):
        ready = rel[t - S] if t >= S else 0.0
        prev_issue = issue[-1] if issue else 0.0
        it = max(prev_issue, ready)
        pw += max(0.0, ready - prev_issue)
        lat = L + (rng.uniform(-jitter, jitter) if jitter else 0.0)
        lt = it + lat
        prev_end = end[-1] if end else 0.0
        st = max(lt, prev_end)
        if t > 0:
            cw += max(0.0, lt - prev_end)
        issue.append(it)
        land.append(lt)
        start.append(st)
        end.append(st + c)
        rel.append(st + r)
    return Timeline(issue, land, start, end, rel, cw, pw, S)


def steady_period(S: int, L: float, c: float, release_after: float | None = None) -> float:
    """Closed form of the steady-state time per tile of `timed` without jitter.

    A buffer is busy from the issue of its fetch until its release, i.e. for
    L + r per tile (r = release point, default c), and S buffers rotate, so
    the ring sustains one tile per (L + r) / S; the consumer needs c per tile.
    """
    r = c if release_after is None else release_after
    return max(c, (L + r) / S)


def min_stages(L: float, c: float, release_after: float | None = None) -> int:
    """Smallest S at which the consumer never waits in steady state."""
    r = c if release_after is None else release_after
    S = 1
    while (L + r) / S > c:
        S += 1
    return S
