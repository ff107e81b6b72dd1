"""CPU model of the packed-row tile schedules of the forward kernel.

Packed KV rows (512 INT8 / FP8-E4M3 codes, the bf16 rope, four fp32 scales;
the KV quant sparse flash attention blog, 数据格式 and 计算公式) are gathered
raw into LDS, decoded once per tile into a bf16 tile that every head-holding
wave reads twice (K for the scores, V^T for the values).  This file restates
tile schedules as per-wave lists of events and checks, for every tile count
and every split of the waves into head holders and helpers, what the GPU
cannot check without faulting:

* every wave reaches the same number of workgroup barriers (a wave that
  skips one deadlocks or desynchronises the workgroup);
* no gather is issued for a tile at or past the split's tile count (the row
  table holds entries for the resolved tiles and one tile of empty entries
  after them, nothing further; a gather past that reads stale LDS as a row
  address);
* a raw stage is decoded only after every wave's share of its gather has
  landed, and is not refilled before that decode ends;
* a decoded tile is written only in a barrier interval in which no wave reads
  that buffer, and read only after the interval that wrote it;
* every head-holding wave reads the scores (K) and then the values (V) of
  tiles 0, 1, ..., nt-1, in that order, once each (the online softmax order).

Two schedules are modelled.  `lockstep` is the one the packed kernels run
(every wave in the same phase: wait, barrier, gather two tiles ahead, decode
a share, barrier, scores and values).  `staggered` is a two-phase design in
which half the waves compute scores while the other half compute values of
the previous tile, over two decoded buffers; it was checked here first, then
built, and on the GPU it matched the oracle and the lockstep kernel bit for
bit but ran 2 % slower (237 vs 232 us on the 32-query packed workload), so
the kernels keep the lockstep schedule.  Planted mistakes (a gather one tile
too far, a missing barrier on one group, a decode into the buffer still being
read) must each be caught, which shows the checks can fail.
"""

import itertools

import pytest


# ---------------------------------------------------------------------------
# the schedules, restated from the kernel's loops
# ---------------------------------------------------------------------------

def staggered(nt, n_waves=8, n_a=4, raw_stages=2, dec_bufs=2, plant=None):
    """Two-phase design for the eight-wave kernel.  Group A = waves 0..3,
    group B = waves 4..7.  Every wave runs the same loop, scores of tile t,
    barrier, values of tile t, barrier; B starts one barrier later (and A
    takes one more at the end), so B's scores of tile t run beside A's values
    of tile t and B's values of tile t beside A's scores of tile t+1.  A alone
    gathers and decodes:

      prologue : A issues raw(0) -> R0, waits, issues raw(1) -> R1; barrier;
                 A decodes tile 0 into D0; barrier; B: one barrier
      loop t   : A issues raw(t+2) -> R[t%2] (t+2 < nt); scores of tile t
                 (D[t%2]); A waits for raw(t+1); barrier;
                 values of tile t (D[t%2]); A decodes raw(t+1) (R[(t+1)%2])
                 into D[(t+1)%2]; barrier
      after    : A: one barrier
    """
    ev = {w: [] for w in range(n_waves)}
    R = lambda t: t % raw_stages
    D = lambda t: t % dec_bufs
    for w in range(n_waves):
        e = ev[w]
        a = w < n_a
        if a and nt > 0:
            e.append(("issue", 0, R(0)))
        if a:
            e.append(("wait", 0))
        if a and (nt > 1 or (plant == "gather_past_end" and w == 0 and nt > 0)):
            e.append(("issue", 1, R(1)))
        e.append(("barrier",))
        if a and nt > 0:
            e.append(("decode", 0, R(0), D(0)))
        e.append(("barrier",))
        if not a and plant != "missing_barrier":
            e.append(("barrier",))                # B lags one phase
        for t in range(nt):
            if a and (t + 2 < nt or (plant == "gather_past_end" and w == 0 and t + 2 == nt)):
                e.append(("issue", t + 2, R(t)))
            e.append(("k", t, D(t)))
            if a and t + 1 < nt:
                e.append(("wait", t + 1))
            e.append(("barrier",))
            e.append(("v", t, D(t)))
            if a and t + 1 < nt:
                dst = D(t) if plant == "decode_into_live_buffer" else D(t + 1)
                e.append(("decode", t + 1, R(t + 1), dst))
            e.append(("barrier",))
        if a:
            e.append(("barrier",))
    return ev


def lockstep(nt, n_waves=8, raw_stages=3):
    """The packed kernels (eight waves; wave pairs): one decoded buffer,
    three raw stages, every wave in the same phase:

      prologue : all issue raw(0) -> R0 and wait, issue raw(1) -> R1
      step(t)  : every wave waits for its own raw(t); barrier; all issue
                 raw(t+2) -> R[(t+2)%3]; all decode raw(t) into D0 (their
                 share); barrier; scores and values of tile t (D0)
    (the pair's own score exchange barrier inside the scores is the same
    for every wave and is left out)
    """
    ev = {w: [] for w in range(n_waves)}
    for w in range(n_waves):
        e = ev[w]
        if nt > 0:
            e.append(("issue", 0, 0))
        e.append(("wait", 0))
        if nt > 1:
            e.append(("issue", 1, 1))
        for t in range(nt):
            e.append(("wait", t))
            e.append(("barrier",))
            if t + 2 < nt:
                e.append(("issue", t + 2, (t + 2) % raw_stages))
            e.append(("decode_share", t, t % raw_stages, 0))
            e.append(("barrier",))
            e.append(("k", t, 0))
            e.append(("v", t, 0))
    return ev


def lockstep_value(nt, n_waves=8, raw_stages=2):
    """The packed kernels with a value tensor: two raw stages, each holding a
    tile's key rows and value codes, one decoded buffer:

      prologue : all issue raw(0) -> R0 and wait, issue raw(1) -> R1
      step(t)  : every wave waits for its own raw(t); barrier; decode the key
                 codes of raw(t) (a share) into D0; barrier; scores of tile t
                 (K from D0); barrier; decode the value codes of raw(t) into
                 D0's nope columns; barrier; issue raw(t+2) -> R[t%2];
                 values of tile t (V from D0)
    """
    ev = {w: [] for w in range(n_waves)}
    for w in range(n_waves):
        e = ev[w]
        if nt > 0:
            e.append(("issue", 0, 0))
        e.append(("wait", 0))
        if nt > 1:
            e.append(("issue", 1, 1 % raw_stages))
        for t in range(nt):
            r = t % raw_stages
            e.append(("wait", t))
            e.append(("barrier",))
            e.append(("decode_share", t, r, 0))
            e.append(("barrier",))
            e.append(("k", t, 0))
            e.append(("barrier",))
            e.append(("decode_value_share", t, r, 0))
            e.append(("barrier",))
            if t + 2 < nt:
                e.append(("issue", t + 2, r))
            e.append(("v", t, 0))
    return ev


# ---------------------------------------------------------------------------
# the checker
# ---------------------------------------------------------------------------

class ScheduleError(AssertionError):
    pass


def check(ev, nt, head_waves):
    waves = sorted(ev)
    nbar = {w: sum(1 for x in ev[w] if x[0] == "barrier") for w in waves}
    if len(set(nbar.values())) != 1:
        raise ScheduleError("barrier counts differ between waves: %s" % nbar)
    # place every event in its barrier interval
    placed = []                                   # (interval, wave, event)
    for w in waves:
        k = 0
        for x in ev[w]:
            if x[0] == "barrier":
                k += 1
            else:
                placed.append((k, w, x))
    issues = [(k, w, x) for k, w, x in placed if x[0] == "issue"]
    for k, w, x in issues:
        if not 0 <= x[1] < nt:
            raise ScheduleError("wave %d gathers tile %d of %d" % (w, x[1], nt))
    # the waves that gather each issue their share of every tile, once
    loaders = sorted(set(w for k, w, x in issues))
    if nt > 0 and not loaders:
        raise ScheduleError("no wave gathers")
    for w in loaders:
        got = sorted(x[1] for k, ww, x in issues if ww == w)
        if got != list(range(nt)):
            raise ScheduleError("wave %d gathers tiles %s, not 0..%d" % (w, got, nt - 1))
    # raw stages: a decode reads stage r in interval I; every wave issued its
    # share of that tile into r and waited for it before interval I, and no
    # wave refills r from that issue through interval I
    decodes = [(k, w, x) for k, w, x in placed if x[0] in ("decode", "decode_share")]
    dec_tiles = sorted(set(x[1] for k, w, x in decodes))
    if dec_tiles != list(range(nt)):
        raise ScheduleError("decoded tiles %s, not 0..%d" % (dec_tiles, nt - 1))
    for k, w, x in decodes:
        t, r = x[1], x[2]
        for ww in loaders:
            iss = [(kk, xx) for kk, w2, xx in issues if w2 == ww and xx[1] == t]
            if len(iss) != 1 or iss[0][1][2] != r:
                raise ScheduleError("tile %d not gathered into stage %d by wave %d" % (t, r, ww))
            waited = [kk for kk, w2, xx in placed if w2 == ww and xx[0] == "wait" and xx[1] == t]
            if not waited or min(waited) >= k:
                raise ScheduleError("wave %d has not waited for tile %d before its decode" % (ww, t))
            k_iss = iss[0][0]
            for kk, w2, xx in issues:
                if xx[2] == r and xx[1] != t and k_iss <= kk <= k:
                    raise ScheduleError("stage %d refilled with tile %d before tile %d is decoded"
                                        % (r, xx[1], t))
    # decoded buffers: writer interval vs readers
    writes = {}                                   # tile -> (interval, buffer)
    for k, w, x in decodes:
        writes.setdefault(x[1], set()).add((k, x[3]))
    for t, s in writes.items():
        if len(s) != 1:
            raise ScheduleError("tile %d decoded in several intervals or buffers: %s" % (t, s))
    reads = [(k, w, x) for k, w, x in placed if x[0] in ("k", "v")]
    for k, w, x in reads:
        t, d = x[1], x[2]
        (kw, dw), = writes[t]
        if d != dw:
            raise ScheduleError("wave %d reads tile %d from buffer %d, written to %d" % (w, t, d, dw))
        if k <= kw:
            raise ScheduleError("wave %d reads tile %d in interval %d, decoded in %d" % (w, t, k, kw))
        # no later tile overwrote buffer d before this read
        for t2, s2 in writes.items():
            (k2, d2), = s2
            if d2 == d and t2 != t and kw < k2 <= k:
                raise ScheduleError("buffer %d holding tile %d is overwritten by tile %d before "
                                    "wave %d reads it" % (d, t, t2, w))
    for k, w, x in decodes:
        for kr, wr, xr in reads:
            if kr == k and xr[2] == x[3]:
                raise ScheduleError("interval %d: buffer %d decoded into while wave %d reads it"
                                    % (k, x[3], wr))
    # value decodes (value codes over the nope columns of the key tile): after
    # every wave's scores of that tile, before any wave's values of it, and
    # reading a raw stage that still holds the tile (not refilled yet)
    vdec = [(k, w, x) for k, w, x in placed if x[0] == "decode_value_share"]
    for t in sorted(set(x[1] for k, w, x in vdec)):
        ks = [k for k, w, x in vdec if x[1] == t]
        if len(set(ks)) != 1:
            raise ScheduleError("value codes of tile %d decoded in several intervals" % t)
        kv = ks[0]
        for kr, wr, xr in reads:
            if xr[1] == t and xr[0] == "k" and kr >= kv:
                raise ScheduleError("wave %d reads K of tile %d after its values replaced it" % (wr, t))
            if xr[1] == t and xr[0] == "v" and kr <= kv:
                raise ScheduleError("wave %d reads V of tile %d before it is decoded" % (wr, t))
        r = [x[2] for k, w, x in vdec if x[1] == t][0]
        k_iss = min(k for k, w, x in issues if x[1] == t)
        for kk, w2, xx in issues:
            if xx[2] == r and xx[1] != t and k_iss <= kk <= kv:
                raise ScheduleError("stage %d refilled with tile %d before tile %d's value codes "
                                    "are decoded" % (r, xx[1], t))
    if vdec and sorted(set(x[1] for k, w, x in vdec)) != list(range(nt)):
        raise ScheduleError("value codes decoded for tiles %s" % sorted(set(x[1] for k, w, x in vdec)))
    # every head wave: k(0) v(0) k(1) v(1) ... in order
    for w in head_waves:
        seq = [(x[0], x[1]) for x in ev[w] if x[0] in ("k", "v")]
        want = [(c, t) for t in range(nt) for c in ("k", "v")]
        if seq != want:
            raise ScheduleError("wave %d reads %s" % (w, seq))


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

TILES = list(range(0, 9)) + [16, 31, 64]


@pytest.mark.parametrize("nt", TILES)
@pytest.mark.parametrize("head_waves", [8, 4, 2, 1, 0])
def test_staggered_schedule_is_sound(nt, head_waves):
    # waves past the head-holding ones take the same barriers and gathers;
    # their reads are skipped in the kernel (no heads), which the model
    # shows by dropping them
    ev = staggered(nt)
    for w in range(head_waves, 8):
        ev[w] = [x for x in ev[w] if x[0] not in ("k", "v")]
    check(ev, nt, range(head_waves))


@pytest.mark.parametrize("nt", TILES)
def test_lockstep_schedule_is_sound(nt):
    check(lockstep(nt), nt, range(8))


@pytest.mark.parametrize("nt", TILES)
@pytest.mark.parametrize("head_waves", [8, 2, 0])
def test_value_tensor_schedule_is_sound(nt, head_waves):
    ev = lockstep_value(nt)
    for w in range(head_waves, 8):
        ev[w] = [x for x in ev[w] if x[0] not in ("k", "v")]
    check(ev, nt, range(head_waves))


def test_value_tensor_schedule_mistakes_are_caught():
    """Refilling the stage before the value codes are decoded (issuing the
    tile two ahead right after the key decode), or one raw stage, must fail."""
    for nt in (3, 4):
        ev = lockstep_value(nt)
        for w in ev:                               # move each issue before the value decode
            e = ev[w]
            for i, x in enumerate(list(e)):
                if x[0] == "issue" and x[1] >= 2:
                    e.remove(x)
                    j = max(k for k, y in enumerate(e[:i]) if y[0] == "decode_share")
                    e.insert(j + 1, x)
        with pytest.raises(ScheduleError):
            check(ev, nt, range(8))
        with pytest.raises(ScheduleError):
            check(lockstep_value(nt, raw_stages=1), nt, range(8))


@pytest.mark.parametrize("plant", ["gather_past_end", "missing_barrier", "decode_into_live_buffer"])
@pytest.mark.parametrize("nt", [1, 2, 3, 5])
def test_planted_schedule_mistakes_are_caught(plant, nt):
    ev = staggered(nt, plant=plant)
    if plant == "decode_into_live_buffer" and nt < 2:
        pytest.skip("no decode inside the loop")
    with pytest.raises(ScheduleError):
        check(ev, nt, range(8))


def test_one_decoded_buffer_is_not_enough_for_the_staggered_schedule():
    """With a single decoded buffer, group A's decode of tile t+1 lands in
    the buffer group B still reads tile t from; the checker must refuse it."""
    for nt in (2, 3, 4):
        with pytest.raises(ScheduleError):
            check(staggered(nt, dec_bufs=1), nt, range(8))


def test_model_raw_stages_match_the_kernels_lds_budget():
    """The staggered kernel holds two raw stages and two decoded tiles; one
    raw stage would refill the stage being decoded."""
    for nt in (3, 4, 6):
        with pytest.raises(ScheduleError):
            check(staggered(nt, raw_stages=1), nt, range(8))
    for nt, hw in itertools.product((3, 4, 6), (8, 4)):
        check(staggered(nt, raw_stages=2), nt, range(hw))
