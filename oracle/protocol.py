"""Protocol oracle: pipeline cursor, mbarrier model and an interleaving checker.

Test infrastructure only (see the package docstring).

Sources (pages, by title and section):
  * "cute（12）async_pipeline"
      - section 2 (PipelineState: the (index, phase, count) cursor, its ++ and
        the producer start state with phase 1) and section 6.1 (the batch
        ``advance`` rule);
      - sections 6.2-6.9 (empty barrier = arrival count only; full barrier =
        arrivals plus transaction bytes; wait(p) passes once the barrier's
        phase differs from p; producer_acquire / consumer_wait /
        consumer_release / producer_tail);
      - section 7 (the full barrier timeline of 3 stages and 8 tiles).
  * "chapter_async_barriers" (mlc.ai), sections "mbarrier" and "phase 如何区分
    不同轮次": init sets phase 0 and the pending count; a phase completes when
    the pending arrivals and the transaction count are both zero; the parity
    table for a 2-stage ring.
  * "cuda-features-10-pipelines", section 4.10.2-4.10.3: acquire/commit on the
    producer side, wait/release on the consumer side; releasing early lets the
    producer overwrite live data.
"""
from __future__ import annotations

from dataclasses import dataclass


# --------------------------------------------------------------------------
# Cursor
# --------------------------------------------------------------------------
@dataclass
class PipelineState:
    """Ring cursor over ``stages`` slots: which slot, which phase parity, how many steps."""

    stages: int
    index: int = 0
    phase: int = 0
    count: int = 0

    def inc(self) -> "PipelineState":
        """One step: next slot; wrapping from the last slot to 0 flips the phase."""
        self.index += 1
        self.count += 1
        if self.index == self.stages:
            self.index = 0
            self.phase ^= 1
        return self

    def advance(self, n: int) -> "PipelineState":
        """n steps at once ("cute（12）async_pipeline" 6.1), as n repeated
        increments: every wrap from the last slot to slot 0 flips the phase, and
        n steps from slot ``index`` wrap (index + n) // stages times, so the
        phase flips when that number is odd."""
        wraps = (self.index + n) // self.stages
        self.phase ^= wraps & 1
        self.index = (self.index + n) % self.stages
        self.count += n
        return self

    def tup(self):
        return (self.index, self.phase, self.count)

    def copy(self) -> "PipelineState":
        return PipelineState(self.stages, self.index, self.phase, self.count)


def producer_start_state(stages: int) -> PipelineState:
    """Slot 0, phase 1, count 0: the ring starts empty, so the first lap never waits."""
    return PipelineState(stages, 0, 1, 0)


def consumer_start_state(stages: int) -> PipelineState:
    return PipelineState(stages, 0, 0, 0)


def cursor_after(stages: int, k: int, start_phase: int) -> tuple:
    """(index, phase) of a cursor after k single steps from (0, start_phase)."""
    st = PipelineState(stages, 0, start_phase, 0)
    for _ in range(k):
        st.inc()
    return (st.index, st.phase)


# --------------------------------------------------------------------------
# mbarrier model
# --------------------------------------------------------------------------
class MBarrier:
    """Arrival counter + phase + transaction-byte counter.

    ``init(n)``: phase 0, n pending arrivals. A phase completes (phase flips,
    pending reloads to n) when pending arrivals and outstanding transaction
    bytes are both zero. ``try_wait(p)`` succeeds once the phase is not p.
    """

    def __init__(self, expected: int):
        self.expected = expected
        self.pending = expected
        self.phase = 0
        self.tx = 0
        self.completions = 0

    def _settle(self):
        if self.pending == 0 and self.tx == 0:
            self.phase ^= 1
            self.pending = self.expected
            self.completions += 1

    def arrive(self):
        self.pending -= 1
        self._settle()

    def arrive_and_expect_tx(self, nbytes: int):
        self.tx += nbytes
        self.pending -= 1
        self._settle()

    def complete_tx(self, nbytes: int):
        self.tx -= nbytes
        self._settle()

    def try_wait(self, parity: int) -> bool:
        return self.phase != parity

    def state(self):
        return (self.pending, self.phase, self.tx)


def counter_phase(count: int, expected: int) -> int:
    """Phase bit of a barrier kept as a bare arrival counter.

    After `count` arrivals on a barrier that expects `expected` per phase,
    floor(count / expected) phases have completed; the phase bit is the parity
    of that number ("completed-phase count, parity = that & 1"). An MBarrier
    without transaction bytes that has seen the same arrivals is in this phase.
    """
    return (count // expected) & 1


# --------------------------------------------------------------------------
# Lock-step timeline (the order in which the pages walk through the ring)
# --------------------------------------------------------------------------
def lockstep_timeline(stages: int, tiles: int, tile_bytes: int = 16384,
                      consumers: int = 1):
    """Run producer and consumers one tile at a time and record each handshake.

    Per tile: the producer acquires (waits on empty), arrives with expect_tx,
    the copy lands (complete_tx), the consumers wait on full and release
    empty. Returns one dict per tile with the cursor values and barrier phase
    changes, the quantities printed in the pages' timeline table.
    """
    full = [MBarrier(1) for _ in range(stages)]
    empty = [MBarrier(consumers) for _ in range(stages)]
    w = producer_start_state(stages)
    r = consumer_start_state(stages)
    rows = []
    for t in range(tiles):
        s = w.index
        row = {"tile": t, "write": (w.index, w.phase), "empty_wait_arg": w.phase,
               "empty_phase_seen": empty[s].phase,
               "producer_blocked": not empty[s].try_wait(w.phase)}
        assert empty[s].try_wait(w.phase), "lock-step schedule never blocks"
        f0 = full[s].phase
        full[s].arrive_and_expect_tx(tile_bytes)
        assert full[s].phase == f0, "arrival alone must not complete the phase"
        full[s].complete_tx(tile_bytes)
        row["full_flip"] = (f0, full[s].phase)
        assert r.index == s
        row["read"] = (r.index, r.phase)
        row["full_wait_arg"] = r.phase
        row["full_phase_seen"] = full[s].phase
        assert full[s].try_wait(r.phase)
        e0 = empty[s].phase
        for _ in range(consumers):
            empty[s].arrive()
        row["empty_flip"] = (e0, empty[s].phase)
        rows.append(row)
        w.inc()
        r.inc()
    return rows


def parity_walk(stages: int, iterations: int):
    """Single-waiter walk over a ring of full barriers with one phase variable.

    The waiter uses slot ``it % stages``, waits on the current phase variable
    and flips that variable after the last slot of each lap. Returns
    (iteration, slot, parity waited on, barrier parity after completion,
    phase variable after the iteration).
    """
    bars = [MBarrier(1) for _ in range(stages)]
    phase_var = 0
    out = []
    for it in range(iterations):
        s = it % stages
        waited = phase_var
        bars[s].arrive()  # the phase this iteration waits for completes
        assert bars[s].try_wait(waited)
        if s == stages - 1:
            phase_var ^= 1
        out.append((it, s, waited, bars[s].phase, phase_var))
    return out


# --------------------------------------------------------------------------
# Explicit-state checker of the full/empty protocol
# --------------------------------------------------------------------------
@dataclass
class ProtocolResult:
    states: int
    deadlock: bool
    completed: bool
    violations: list
    max_ahead: int


def _producer_program(S, T, mode, lag, start_phase, tail, part=0, commits=True, pgroup=1):
    """The producer's instruction list.

    "tx" mode is fully static. In "landed" mode the commits are dynamic: after
    issuing a tile the producer commits its oldest uncommitted tiles, oldest
    first, while more than ``lag`` are uncommitted ("commit_lag"), and at the
    end it commits all
    of them ("commit_all"); each commit waits until that tile's share landed.
    ``commits=False`` leaves every commit out (the omission that
    "cuda-features-10-pipelines" 4.10.2 warns starves the consumers).
    With ``pgroup`` = G > 1 (landed mode) the producer takes G consecutive
    stages at a time: it waits on all G empty barriers, then issues the G
    tiles (one load may fill parts of all G slots), then applies the commit
    rule. T must be a multiple of G.
    """
    ops = []
    cur = PipelineState(S, 0, start_phase, 0)
    if mode == "tx":
        for t in range(T):
            ops.append(("wait_empty", cur.index, cur.phase))
            ops.append(("arrive_tx", cur.index))
            ops.append(("issue", t, cur.index, part))
            cur.inc()
    elif mode == "landed":
        if pgroup < 1 or T % pgroup:
            raise ValueError("T must be a multiple of the producer group")
        for t0 in range(0, T, pgroup):
            group = []
            for t in range(t0, t0 + pgroup):
                ops.append(("wait_empty", cur.index, cur.phase))
                group.append((t, cur.index))
                cur.inc()
            ops += [("issue", t, s_, part) for t, s_ in group]
            if commits:
                ops.append(("commit_lag",))
        if commits:
            ops.append(("commit_all",))
    else:
        raise ValueError(mode)
    if tail:
        for _ in range(S):
            ops.append(("wait_empty", cur.index, cur.phase))
            cur.inc()
    return ops


def _consumer_program(S, T, release_before_read, group=1):
    """The consumer's instruction list.

    ``group`` = 1 is the pages' consumer: wait on a stage, use it, release it.
    With ``group`` = G > 1 the consumer takes G consecutive stages at a time:
    it waits on all G, uses them, then releases all G (a consumer that stores
    a row of G neighbouring tiles in one pass). T must be a multiple of G.
    """
    if group < 1 or T % group:
        raise ValueError("T must be a multiple of the group")
    ops = []
    cur = PipelineState(S, 0, 0, 0)
    for t0 in range(0, T, group):
        tiles = []
        for t in range(t0, t0 + group):
            ops.append(("wait_full", cur.index, cur.phase))
            tiles.append((t, cur.index))
            cur.inc()
        if release_before_read:
            ops += [("arrive_empty", s_) for _, s_ in tiles]
            ops += [("read", t, s_) for t, s_ in tiles]
        else:
            ops += [("read", t, s_) for t, s_ in tiles]
            ops += [("arrive_empty", s_) for _, s_ in tiles]
    return ops


def check_protocol(S: int, T: int, C: int, *, mode: str = "tx", lag: int = 0,
                   producers: int = 1, producer_start_phase: int = 1, full_expected=None,
                   empty_expected=None, release_before_read: bool = False,
                   tail: bool = True, eager_min: int = 0, tile_bytes: int = 16384,
                   group: int = 1, commits: bool = True, producer_group: int = 1,
                   max_states: int = 2_000_000) -> ProtocolResult:
    """Explore every interleaving of the producers, C consumers and the copy engine.

    ``mode="tx"``: the producer arrives with expect_tx before issuing the copy
    and the copy's landing performs complete_tx (the mbarrier design).
    ``mode="landed"``: each of ``producers`` producer agents issues its share of
    every tile, and ``lag`` tiles later waits until that share has landed and
    then arrives on full (a counter barrier with no transaction bytes, which
    expects one arrival per producer by default). With ``eager_min`` > 0 a
    producer whose acquire finds the slot still in use, while it has at least
    ``eager_min`` uncommitted tiles, commits its oldest uncommitted tile first
    (waiting for that tile to land), then polls again. With ``group`` = G
    every consumer waits on G consecutive stages before it uses and releases
    them (see ``_consumer_program``). With ``producer_group`` = G the
    producers acquire and issue G consecutive stages at a time (see
    ``_producer_program``).

    Checked: (I1) a consumer reads a slot only after every share of that tile
    landed; (I2) a slot is not overwritten before all consumers of its previous
    tile are done with it; (I3) no reachable deadlock and all tiles consumed;
    (I4) the producers are at most S tiles ahead of the slowest consumer.
    """
    P = producers
    if mode == "tx" and P != 1:
        raise ValueError("the transaction-count model has a single producer")
    if full_expected is None:
        full_expected = P
    if empty_expected is None:
        empty_expected = C
    if eager_min and mode != "landed":
        raise ValueError("eager commits exist in the landed mode only")
    if not commits and mode != "landed":
        raise ValueError("commits can be left out in the landed mode only")
    if producer_group != 1 and mode != "landed":
        raise ValueError("grouped producers exist in the landed mode only")
    progs = [_producer_program(S, T, mode, lag, producer_start_phase, tail, part=i,
                               commits=commits, pgroup=producer_group) for i in range(P)]
    Q = _consumer_program(S, T, release_before_read, group)
    nQ = len(Q)
    # tiles a consumer at program counter pc has released
    released_at = [0]
    for op in Q:
        released_at.append(released_at[-1] + (op[0] == "arrive_empty"))
    nbar = 2 * S
    all_parts = frozenset(range(P))

    def bar_exp(b):
        return full_expected if b < S else empty_expected

    def settle(bars, b):
        pend, ph, tx = bars[b]
        if pend == 0 and tx == 0:
            bars[b] = (bar_exp(b), ph ^ 1, 0)

    # slot: None or (tile, landed parts); inflight: frozenset of (tile, part)
    init_bars = tuple((bar_exp(b), 0, 0) for b in range(nbar))
    # producer i: (pc, tiles committed, 1 while blocked in an eager commit)
    init = (((0, 0, 0),) * P, (0,) * C, init_bars, (None,) * S, frozenset())
    seen = {init}
    stack = [init]
    violations = set()
    deadlock = False
    completed = False
    max_ahead = 0

    def released_tiles(qpc):
        return released_at[qpc]

    while stack:
        if len(seen) > max_states:
            raise RuntimeError("state bound exceeded")
        st = stack.pop()
        ppcs, qpcs, bars, slots, inflight = st
        succ = []
        for i in range(P):
            ppc, done, flushing = ppcs[i]
            prog = progs[i]
            if ppc >= len(prog):
                continue
            op = prog[ppc]
            kind = op[0]

            def at(pc, committed=done, fl=0, i=i):
                return ppcs[:i] + ((pc, committed, fl),) + ppcs[i + 1:]

            def commit_oldest(next_pc, fl=0, i=i, done=done):
                # wait until the oldest uncommitted tile's share landed, then arrive
                if (done, i) in inflight:
                    return None
                b = list(bars)
                pend, ph, tx = b[done % S]
                b[done % S] = (pend - 1, ph, tx)
                settle(b, done % S)
                return (at(next_pc, done + 1, fl), qpcs, tuple(b), slots, inflight)

            issued = sum(1 for o in prog[:ppc] if o[0] == "issue")
            npp = at(ppc + 1)
            if kind == "wait_empty":
                _, s_, ph = op
                if flushing:
                    n = commit_oldest(ppc)
                    if n is not None:
                        succ.append(n)
                elif bars[S + s_][1] != ph:
                    succ.append((npp, qpcs, bars, slots, inflight))
                elif eager_min > 0 and issued - done >= eager_min:
                    succ.append((at(ppc, done, 1), qpcs, bars, slots, inflight))
            elif kind == "arrive_tx":
                s_ = op[1]
                b = list(bars)
                pend, ph, tx = b[s_]
                b[s_] = (pend - 1, ph, tx + tile_bytes)
                settle(b, s_)
                succ.append((npp, qpcs, tuple(b), slots, inflight))
            elif kind == "issue":
                _, t, s_, part = op
                slowest = min(released_tiles(q) for q in qpcs)
                ahead = (t + 1) - slowest
                max_ahead = max(max_ahead, ahead)
                if ahead > S:
                    violations.add(("I4", t, ahead))
                sl = list(slots)
                if sl[s_] is None or sl[s_][0] != t:
                    sl[s_] = (t, frozenset())          # older contents destroyed
                succ.append((npp, qpcs, bars, tuple(sl), inflight | {(t, part)}))
            elif kind == "commit_lag":
                # commit the oldest uncommitted tile while more than `lag` are
                # uncommitted (after a single issue that is at most one tile)
                if issued - done > lag:
                    n = commit_oldest(ppc)
                    if n is not None:
                        succ.append(n)
                else:
                    succ.append((npp, qpcs, bars, slots, inflight))
            elif kind == "commit_all":
                if issued > done:
                    n = commit_oldest(ppc)
                    if n is not None:
                        succ.append(n)
                else:
                    succ.append((npp, qpcs, bars, slots, inflight))
        # copy engine: any in-flight share may land
        for (t, part) in inflight:
            s_ = t % S
            sl = list(slots)
            if sl[s_] is not None and sl[s_][0] == t:
                sl[s_] = (t, sl[s_][1] | {part})
            b = bars
            if mode == "tx":
                b = list(bars)
                pend, ph, tx = b[s_]
                b[s_] = (pend, ph, tx - tile_bytes)
                settle(b, s_)
                b = tuple(b)
            succ.append((ppcs, qpcs, b, tuple(sl), inflight - {(t, part)}))
        for c in range(C):
            qpc = qpcs[c]
            if qpc >= nQ:
                continue
            op = Q[qpc]
            kind = op[0]
            nq = qpcs[:c] + (qpc + 1,) + qpcs[c + 1:]
            if kind == "wait_full":
                _, s_, ph = op
                if bars[s_][1] != ph:
                    succ.append((ppcs, nq, bars, slots, inflight))
            elif kind == "read":
                _, t, s_ = op
                if slots[s_] != (t, all_parts):
                    tag = "I1" if slots[s_] is not None and slots[s_][0] == t else "I2"
                    violations.add((tag, t, c, slots[s_]))
                succ.append((ppcs, nq, bars, slots, inflight))
            elif kind == "arrive_empty":
                s_ = op[1]
                b = list(bars)
                pend, ph, tx = b[S + s_]
                b[S + s_] = (pend - 1, ph, tx)
                settle(b, S + s_)
                succ.append((ppcs, nq, tuple(b), slots, inflight))
        if not succ:
            if (all(pc[0] == len(progs[i]) for i, pc in enumerate(ppcs))
                    and all(q == nQ for q in qpcs) and not inflight):
                completed = True
            else:
                deadlock = True
            continue
        for n in succ:
            if n not in seen:
                seen.add(n)
                stack.append(n)
    return ProtocolResult(len(seen), deadlock, completed and not deadlock,
                          sorted(violations, key=repr), max_ahead)


# --------------------------------------------------------------------------
# Shared storage of the pages' pipeline
# --------------------------------------------------------------------------
def page_shared_storage_bytes(stages: int, tile_rows: int, tile_cols: int, elem_bytes: int = 2,
                              barrier_bytes: int = 8, data_align: int = 128) -> dict:
    """Byte layout of the pages' SharedStorage ("cute（12）async_pipeline" 5.1-5.2):
    a full and an empty mbarrier of ``barrier_bytes`` per stage first, then the
    stage buffers at the next ``data_align`` boundary."""
    pipeline = stages * 2 * barrier_bytes
    data = stages * tile_rows * tile_cols * elem_bytes
    data_offset = -(-pipeline // data_align) * data_align
    return {"pipeline_bytes": pipeline, "data_bytes": data, "total_bytes": data_offset + data}
