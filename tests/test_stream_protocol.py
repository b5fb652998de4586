"""CPU model of the NVFP4 expert stream's hand-out protocol (the ordering argument of
fp4_expert_stream, not its arithmetic).

Eight k-waves (optionally fewer, plus waves without k work) run the stream's control flow
at random relative speeds: a ring of DEPTH pairs per wave, one reduction barrier per tile,
wave 0 asking the work counter for the tile after next when its loads enter a tile and
publishing the answer before its next barrier, every wave reading a hand-out when its loads
reach that tile.  The model checks that no wave ever reads a hand-out before it is published
(the kernel does not wait for one), that no barrier deadlocks, and that all waves agree on
where the stream stops.  A variant that publishes one barrier late must fail the check, so
the model can tell a broken ordering from a sound one.
"""
import random


def _run(seed, n_static, n_dyn, depth, npt, n_kwaves=8, max_tiles=64, waves=8, late_publish=False):
    rnd = random.Random(seed)
    handed = {}          # dynamic sequence -> tile (published)
    counter = [0]
    END = -1
    arrivals = {}
    bad = []

    class Wave:
        pass

    st = [Wave() for _ in range(waves)]
    for x in st:
        x.pos, x.pending, x.got, x.bars, x.ends = 0, False, None, 0, 0

    def tile_at(w, s):
        if s < n_static:
            return s
        k = s - n_static
        if k not in handed:
            bad.append((w, s))
            return END
        return handed[k]

    def request(w):
        x = st[w]
        if w == 0 and x.pos + 1 >= n_static:
            i = counter[0]
            counter[0] += 1
            x.got = 1000 + i if i < n_dyn else END
            x.pending = True

    def publish(w):
        x = st[w]
        if x.pending:
            handed[x.pos + 1 - n_static] = x.got
            x.pending = False

    def barrier(w):
        x = st[w]
        b = x.bars
        x.bars += 1
        arrivals[b] = arrivals.get(b, 0) + 1
        while arrivals[b] < waves:
            yield "wait"

    def advance(w):
        publish(w)
        x = st[w]
        s = x.pos + 1
        if s >= max_tiles:
            return False
        if tile_at(w, s) == END:
            return False
        x.pos = s
        request(w)
        return True

    def tile_end(w):
        if not late_publish:
            publish(w)
        yield from barrier(w)
        if late_publish:
            publish(w)
        st[w].ends += 1

    def kwave(w):
        request(w)
        yield "prologue"
        publish(w)
        yield from barrier(w)
        ip, cp, more = depth, 0, True
        if ip == npt:
            more = advance(w)
            ip = 0
        while more:
            yield "ring"
            cp += depth
            if cp == npt:
                yield from tile_end(w)
                cp = 0
            ip += depth
            if ip == npt:
                more = advance(w)
                ip = 0
        yield "tail"
        yield from tile_end(w)
        publish(w)
        yield from barrier(w)

    def idle_wave(w):
        yield from barrier(w)
        while True:
            more = advance(w)
            yield from tile_end(w)
            if not more:
                break
        yield from barrier(w)

    gens = [kwave(w) if w < n_kwaves else idle_wave(w) for w in range(waves)]
    alive = set(range(waves))
    speed = [rnd.uniform(0.05, 1.0) for _ in range(waves)]
    stuck = 0
    while alive:
        w = rnd.choices(sorted(alive), weights=[speed[i] for i in sorted(alive)])[0]
        try:
            r = next(gens[w])
            stuck = stuck + 1 if r == "wait" else 0
            if stuck > 50000:
                return "deadlock"
        except StopIteration:
            alive.discard(w)
    if bad:
        return "unpublished read"
    if len({x.pos for x in st}) != 1 or len({x.bars for x in st}) != 1 or len({x.ends for x in st}) != 1:
        return "waves disagree"
    return "ok"


CASES = [(4, 8), (2, 8), (8, 8), (1, 1), (1, 8), (2, 2)]


def test_handouts_are_published_before_they_are_read():
    for seed in range(240):
        depth, npt = CASES[seed % len(CASES)]
        r = _run(seed, n_static=seed % 9, n_dyn=seed % 13, depth=depth, npt=npt,
                 n_kwaves=8 if seed % 3 else 6, max_tiles=[64, 5, 3][seed % 3])
        assert r == "ok", (seed, r)


def test_publishing_after_the_barrier_is_caught():
    fails = 0
    for seed in range(120):
        depth, npt = CASES[seed % 2]
        r = _run(seed, n_static=0, n_dyn=12, depth=depth, npt=npt, late_publish=True)
        fails += r != "ok"
    assert fails > 0
