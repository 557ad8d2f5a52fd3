"""Model check of the attention core's LDS ring protocol (host only).

The core streams K, key codes and V tiles into a 4-stage LDS ring (tile t in
stage t % 4); each of the 4 waves loads its own rows of every tile, so a tile
is readable only after a workgroup barrier, and a stage may be refilled only
after every wave has read it.  This file restates the core's schedule as a
list of events per wave -- loads issued, waits for the wave's own loads,
barriers, LDS reads -- and checks, for every tile count up to 6 and every
combination of per-wave tile counts (waves whose rows end early compute a
prefix of the tiles and only keep the ring going):

* every wave takes the same barriers (unequal counts would hang);
* every read of a tile part finds every wave's rows of it landed before a
  barrier that the reader has passed;
* no wave's later load into the same stage and part can land before every
  wave has read it (the load is issued only after a barrier the readers
  reach after their reads).

The schedule mirrors pair_sync, pair_rest, step and finish_last in
csrc/attn_bf16.hip (one barrier per two tiles); the planted-mistake cases
show that the checker rejects a schedule that is wrong.
"""
import itertools

import pytest


def wave_events(nuse, ntiles, *, final_av_needs_barrier=True, k_ahead=(2, 3)):
    ev = []

    def issue(part, t):
        ev.append(("issue", part, t, t & 3))

    def read(part, t):
        ev.append(("read", part, t, t & 3))

    def pair_sync(it):                      # even tiles only
        ev.append(("wait",))                # all of this wave's loads landed
        ev.append(("bar", it))
        for d in k_ahead:
            issue("K", it + d)
            issue("C", it + d)

    def pair_rest(it):                      # mid-step of an even tile
        for d in (1, 2):
            issue("V", it + d)

    for t in (0, 1):                        # before the first barrier
        issue("K", t)
        issue("C", t)
    issue("V", 0)
    if nuse > 0:
        pair_sync(0)
        read("K", 0)
        read("C", 0)
        pair_rest(0)
        for it in range(1, nuse):           # step it: S(it), then A(it-1) V(it-1)
            even = it % 2 == 0
            if even:
                pair_sync(it)
            read("K", it)
            read("C", it)
            if even:
                pair_rest(it)
            read("V", it - 1)
        if nuse % 2 == 1 or not final_av_needs_barrier:
            read("V", nuse - 1)             # the last tile's A V
    rest = nuse
    if final_av_needs_barrier and nuse > 0 and nuse % 2 == 0:
        pair_sync(nuse)
        read("V", nuse - 1)
        pair_rest(nuse)
        rest = nuse + 2
    it = (rest + 1) & ~1
    while it <= ntiles:
        pair_sync(it)
        pair_rest(it)
        it += 2
    return ev


def check(nuses, ntiles, **kw):
    evs = [wave_events(n, ntiles, **kw) for n in nuses]
    bars = [[e[1] for e in ev if e[0] == "bar"] for ev in evs]
    if any(b != bars[0] for b in bars):
        return "barrier counts differ"
    nbar = []
    for ev in evs:                          # barriers passed before each event
        k, out = 0, []
        for e in ev:
            k += e[0] == "bar"
            out.append(k)
        nbar.append(out)

    def landed_by(v, j):                    # the barrier by which load j of wave v has landed
        for i in range(j + 1, len(evs[v])):
            if evs[v][i][0] == "wait":
                return nbar[v][i] + 1
        return None

    for w, ev in enumerate(evs):
        for ri, e in enumerate(ev):
            if e[0] != "read":
                continue
            _, part, t, st = e
            passed = nbar[w][ri]
            for v in range(len(evs)):
                loads = [j for j, x in enumerate(evs[v]) if x[0] == "issue" and x[1] == part and x[2] == t]
                if not loads:
                    return f"tile {t} {part} never loaded"
                lb = landed_by(v, loads[-1])
                if lb is None or lb > passed:
                    return f"wave {w} reads {part}{t} before wave {v}'s rows landed"
                for j in range(loads[-1] + 1, len(evs[v])):
                    x = evs[v][j]
                    if x[0] == "issue" and x[1] == part and x[3] == st and nbar[v][j] <= passed:
                        return f"wave {v} refills the stage of {part}{t} before wave {w} read it"
    return None


def all_cases(max_tiles=6, waves=4):
    for ntiles in range(max_tiles + 1):
        for nuses in itertools.product(range(ntiles + 1), repeat=waves):
            yield nuses, ntiles


def test_paired_barrier_schedule_is_race_free():
    bad = [(n, t, r) for n, t in all_cases() if (r := check(n, t))]
    assert not bad, bad[:3]


@pytest.mark.parametrize("mistake", [
    {"final_av_needs_barrier": False},      # an odd last tile's A V without the next barrier
    {"k_ahead": (1, 2)},                    # K of the next tile loaded after its own barrier
])
def test_checker_rejects_a_wrong_schedule(mistake):
    assert any(check(n, t, **mistake) for n, t in all_cases())
