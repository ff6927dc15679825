"""Pins of the protocol oracle against the pages' printed tables, closed forms
and exhaustive exploration (CPU)."""
import pytest

from oracle import protocol as P
from tests.conftest import golden_lines


def _golden(name):
    out = {}
    for ln in golden_lines("cursor_3stage.txt"):
        k, *v = ln.split()
        out.setdefault(k, []).append(tuple(int(x) for x in v))
    return out[name]


def test_consumer_increment_table():
    st = P.consumer_start_state(3)
    seq = [st.tup()]
    for _ in range(6):
        seq.append(st.inc().tup())
    assert seq == _golden("consumer_inc")


def test_producer_and_consumer_tile_lists():
    assert [P.cursor_after(3, k, 1) for k in range(8)] == _golden("producer_tile")
    assert [P.cursor_after(3, k, 0) for k in range(5)] == _golden("consumer_tile")
    assert [P.cursor_after(3, k, 1) for k in range(4)] == _golden("trace_producer")
    assert [P.cursor_after(3, k, 0) for k in range(4)] == _golden("trace_consumer")
    assert P.producer_start_state(3).tup() == (0, 1, 0)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])
def test_advance_equals_repeated_increment(S):
    for i0 in range(S):
        for p0 in (0, 1):
            for n in range(0, 40):
                a = P.PipelineState(S, i0, p0, 7).advance(n)
                b = P.PipelineState(S, i0, p0, 7)
                for _ in range(n):
                    b.inc()
                assert a.tup() == b.tup(), (S, i0, p0, n)
                # closed form: index (i0+n) mod S, phase flips per lap crossed
                assert a.tup() == ((i0 + n) % S, p0 ^ (((i0 + n) // S) & 1), 7 + n)


def test_timeline_matches_page_table():
    rows = golden_lines("timeline_3stage_8tiles.csv")[1:]
    got = P.lockstep_timeline(3, 8)
    for ln, g in zip(rows, got):
        v = [int(x) for x in ln.split(",")]
        assert v[0] == g["tile"]
        assert (v[1], v[2]) == g["write"]
        assert v[3] == g["empty_phase_seen"]
        assert (v[4], v[5]) == g["full_flip"]
        assert (v[6], v[7]) == g["read"]
        assert v[8] == g["full_phase_seen"]
        assert (v[9], v[10]) == g["empty_flip"]
        assert g["empty_wait_arg"] == g["write"][1]
        assert g["full_wait_arg"] == g["read"][1]
    assert len(got) == len(rows) == 8


def test_parity_walk_matches_page_table():
    rows = [tuple(int(x) for x in ln.split(",")) for ln in golden_lines("parity_2stage.csv")[1:]]
    assert P.parity_walk(2, 4) == rows


def test_mbarrier_needs_arrivals_and_bytes():
    b = P.MBarrier(1)
    b.arrive_and_expect_tx(2048)
    assert b.phase == 0
    b.complete_tx(1024)
    assert b.phase == 0
    b.complete_tx(1024)
    assert b.phase == 1 and b.pending == 1 and b.tx == 0
    # two copies of 2048 bytes complete one phase only when both landed
    b2 = P.MBarrier(1)
    b2.arrive_and_expect_tx(4096)
    b2.complete_tx(2048)
    assert not b2.try_wait(0)
    b2.complete_tx(2048)
    assert b2.try_wait(0)


@pytest.mark.parametrize("S,T,C", [(1, 4, 1), (1, 3, 3), (2, 5, 2), (2, 4, 3), (3, 7, 1),
                                   (3, 5, 2), (3, 4, 3)])
@pytest.mark.parametrize("mode", ["tx", "landed"])
def test_protocol_safe_and_live(S, T, C, mode):
    r = P.check_protocol(S, T, C, mode=mode, lag=S - 1 if mode == "landed" else 0)
    assert r.completed and not r.deadlock
    assert r.violations == []
    assert r.max_ahead <= S
    # the ring fills completely in some interleaving (producer S tiles ahead)
    assert r.max_ahead == min(S, T)


def test_start_phase_zero_deadlocks():
    r = P.check_protocol(3, 4, 2, producer_start_phase=0)
    assert r.deadlock and not r.completed


def test_full_expected_arrivals_mismatch_deadlocks():
    r = P.check_protocol(3, 4, 1, full_expected=32)
    assert r.deadlock and not r.completed


def test_release_before_read_overwrites_live_data():
    r = P.check_protocol(2, 4, 2, release_before_read=True)
    assert any(v[0] == "I2" for v in r.violations)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 6, 8])
def test_commit_lag_rule(S):
    """A counter barrier without transaction bytes: committing tile t-L after
    issuing tile t is live iff L <= S-1."""
    for L in range(0, S + 1):
        r = P.check_protocol(S, S + 2, 1, mode="landed", lag=L)
        if L <= S - 1:
            assert r.completed and r.violations == [], (S, L)
        else:
            assert r.deadlock, (S, L)


@pytest.mark.parametrize("S,T", [(3, 2), (2, 5)])
def test_missing_commit_starves_the_consumers(S, T):
    """A producer that acquires and issues but never commits: the consumers
    never see a full phase ("cuda-features-10-pipelines" 4.10.2). With T <= S
    the producer finishes its issues and only the consumers wait; with T > S it
    also runs out of writable stages."""
    r = P.check_protocol(S, T, 1, mode="landed", lag=0, commits=False, tail=False)
    assert r.deadlock and not r.completed
    ok = P.check_protocol(S, T, 1, mode="landed", lag=0, tail=False)
    assert ok.completed and not ok.deadlock
    with pytest.raises(ValueError):
        P.check_protocol(S, T, 1, mode="tx", commits=False)


def test_no_tail_still_consumes_everything():
    r = P.check_protocol(2, 3, 2, tail=False)
    assert r.completed


@pytest.mark.parametrize("S,T,C", [(1, 3, 2), (2, 4, 2), (3, 4, 2), (3, 5, 1), (4, 5, 1)])
def test_two_producer_waves_safe_and_live(S, T, C):
    """Each producer wave moves its share of every tile and arrives on full,
    which expects one arrival per producer wave."""
    r = P.check_protocol(S, T, C, mode="landed", lag=S - 1, producers=2)
    assert r.completed and not r.deadlock and r.violations == []
    assert r.max_ahead == min(S, T)


def test_full_expecting_fewer_arrivals_than_producers_reads_half_landed_tiles():
    r = P.check_protocol(2, 3, 1, mode="landed", lag=1, producers=2, full_expected=1)
    assert any(v[0] == "I1" for v in r.violations)


@pytest.mark.parametrize("S", [1, 2, 3])
def test_two_producer_commit_lag_rule(S):
    for L in range(0, S + 1):
        r = P.check_protocol(S, S + 1, 1, mode="landed", lag=L, producers=2)
        if L <= S - 1:
            assert r.completed and r.violations == [], (S, L)
        else:
            assert r.deadlock, (S, L)


@pytest.mark.parametrize("S,T,C,producers", [(5, 7, 1, 1), (6, 8, 2, 1), (8, 10, 1, 1),
                                             (8, 9, 2, 1), (5, 6, 1, 2), (6, 7, 1, 2),
                                             (2, 3, 1, 4)])
def test_deep_rings_and_four_producer_waves_safe_and_live(S, T, C, producers):
    """Rings deeper than 4 stages, with the commit lag at its liveness bound S-1,
    and four producer waves each moving a quarter of every tile."""
    r = P.check_protocol(S, T, C, mode="landed", lag=S - 1, producers=producers)
    assert r.completed and not r.deadlock and r.violations == []
    assert r.max_ahead == min(S, T)


@pytest.mark.parametrize("S,T,C,producers", [(1, 3, 2, 1), (2, 5, 2, 1), (3, 5, 2, 1),
                                             (4, 6, 1, 1), (6, 8, 1, 1), (2, 4, 1, 2),
                                             (3, 4, 1, 2)])
@pytest.mark.parametrize("eager_min", [1, 2])
def test_eager_commit_safe_and_live(S, T, C, producers, eager_min):
    """Committing the oldest landed tile while the acquire is blocked never
    publishes a tile early and never loses a slot."""
    r = P.check_protocol(S, T, C, mode="landed", lag=S - 1, producers=producers,
                         eager_min=eager_min)
    assert r.completed and not r.deadlock and r.violations == []
    assert r.max_ahead == min(S, T)


@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_eager_commit_lifts_the_lag_bound(S):
    """Without eager commits a lag of S tiles deadlocks (the producer holds back
    the tile the consumers need while it waits for them); with them any lag is live."""
    for L in (S, S + 2):
        assert P.check_protocol(S, S + 2, 1, mode="landed", lag=L).deadlock
        r = P.check_protocol(S, S + 2, 1, mode="landed", lag=L, eager_min=1)
        assert r.completed and r.violations == [], (S, L)
        # skipping the newest tile in flight: live as soon as S >= 2 tiles can be pending
        r2 = P.check_protocol(S, S + 2, 1, mode="landed", lag=L, eager_min=2)
        assert r2.completed == (S >= 2) and r2.deadlock == (S < 2), (S, L)


@pytest.mark.parametrize("S,G", [(2, 2), (3, 2), (4, 2), (8, 2), (4, 4), (5, 4), (6, 4), (8, 4)])
def test_grouped_consumer_lag_bound(S, G):
    """A consumer that holds G stages at once (it waits on G consecutive
    stages before releasing any) is live exactly when the producer's commit
    lag L is at most S - G. Closed form: the producer commits tile j only
    after issuing tile j + L, which needs the slot of tile j + L - S released;
    that tile must lie in an earlier group than j's, i.e. j + L - S < j - (G - 1)
    for the first tile j of a group."""
    T = S + 2 * G if S + 2 * G <= 16 else 4 * G
    T -= T % G
    for L in range(S):
        r = P.check_protocol(S, T, 1, mode="landed", lag=L, group=G)
        live = L <= S - G
        assert r.completed == live and r.deadlock == (not live), (S, G, L)
        assert r.violations == []
    # two consumers and two producers at the bound
    r = P.check_protocol(S, 2 * G, 2, mode="landed", lag=S - G, group=G, producers=2)
    assert r.completed and not r.deadlock and r.violations == []
    assert r.max_ahead <= S


def test_grouped_consumer_needs_whole_groups():
    with pytest.raises(ValueError):
        P.check_protocol(4, 6, 1, mode="landed", lag=0, group=4)


def test_eager_commit_needs_landed_mode():
    with pytest.raises(ValueError):
        P.check_protocol(2, 3, 1, mode="tx", eager_min=1)


def test_store_side_ring_of_the_gemm_epilogue():
    """The bf16 epilogue's staging ring: one slot, two producer waves (an MFMA
    wave pair writes a chunk, synchronously: lag 0) and one consumer (the store
    wave), 4 chunks per tile over 3 tiles."""
    r = P.check_protocol(1, 12, 1, mode="landed", lag=0, producers=2)
    assert r.completed and not r.deadlock and r.violations == []
    assert r.max_ahead == 1


@pytest.mark.parametrize("expected", [1, 2, 3, 4, 8])
def test_counter_phase_equals_mbarrier_phase(expected):
    """A barrier kept as a bare monotonic arrival counter (parity of the number of
    completed phases) passes and blocks exactly where the mbarrier model does."""
    b = P.MBarrier(expected)
    for count in range(0, 20 * expected + 1):
        if count:
            b.arrive()
        assert P.counter_phase(count, expected) == b.phase
        for parity in (0, 1):
            assert (P.counter_phase(count, expected) != parity) == b.try_wait(parity)


def test_counter_phase_survives_the_32_bit_wrap_for_powers_of_two():
    """The device counter is 32 bits. For power-of-two arrival counts per phase,
    2**32 / expected is even, so the phase read from the wrapped counter is the
    phase of the true count."""
    for expected in (1, 2, 4, 8):
        for count in range(2 ** 32 - 5 * expected, 2 ** 32 + 5 * expected):
            assert P.counter_phase(count % 2 ** 32, expected) == P.counter_phase(count, expected)
    # not so for 3: which is why the host bounds the arrivals per slot
    assert any(P.counter_phase(c % 2 ** 32, 3) != P.counter_phase(c, 3)
               for c in range(2 ** 32, 2 ** 32 + 6))


def test_page_shared_storage_arithmetic(golden):
    """The 3-stage program's printed shared-memory sizes follow from two 8-byte
    barriers per stage placed first and 128-byte aligned 16 KiB tile buffers;
    one tile is the printed transaction size, and 128 x 64 tiles of a 256 x 128
    matrix make the printed 2 x 2 grid."""
    kv = {ln.split()[0]: [int(x) for x in ln.split()[1:]] for ln in golden("shared_storage_12.txt")}
    got = P.page_shared_storage_bytes(kv["stages"][0], kv["tile_rows"][0], kv["tile_cols"][0])
    assert got == {"pipeline_bytes": kv["pipeline_bytes"][0], "data_bytes": kv["data_bytes"][0],
                   "total_bytes": kv["total_bytes"][0]}
    tile = P.page_shared_storage_bytes(1, kv["tile_rows"][0], kv["tile_cols"][0])["data_bytes"]
    assert tile == kv["tx_bytes"][0]
    assert [256 // kv["tile_rows"][0], 128 // kv["tile_cols"][0]] == kv["grid_256x128"]
    # a plausible misreading (one barrier per stage, or unaligned data) misses the printed total
    assert P.page_shared_storage_bytes(3, 128, 64, data_align=8)["total_bytes"] != kv["total_bytes"][0]


@pytest.mark.parametrize("S,G", [(4, 4), (8, 4), (4, 2), (6, 2)])
@pytest.mark.parametrize("C", [1, 2])
def test_grouped_producer_lag_boundary(S, G, C):
    """A producer that acquires G consecutive stages, issues loads spanning all
    G and then applies the commit rule, feeding consumers that take the same G
    stages at a time: live and safe while the commit lag (in tiles) is at most
    S - G -- the bound the grouped-load copy keeps -- and deadlocked one tile
    beyond it (the producer then needs the slots of a group it has not yet
    committed)."""
    T = S + G   # the ring wraps: the last group reuses the slots of the first
    ok = P.check_protocol(S, T, C, mode="landed", lag=S - G, group=G, producer_group=G)
    assert ok.completed and not ok.deadlock and not ok.violations, ok
    assert ok.max_ahead <= S
    bad = P.check_protocol(S, T, C, mode="landed", lag=S - G + 1, group=G, producer_group=G)
    assert bad.deadlock and not bad.violations, bad


def test_grouped_producer_with_two_producer_waves():
    r = P.check_protocol(4, 8, 1, mode="landed", lag=0, producers=2, group=4, producer_group=4)
    assert r.completed and not r.deadlock and not r.violations, r
