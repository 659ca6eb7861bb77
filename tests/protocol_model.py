"""A CPU model of the chunk decoder's LDS protocol (test infrastructure).

The GPU decoder runs one workgroup per chunk whose waves talk only through
LDS counters: a feeder that streams the compressed block into an input ring
with asynchronous DMA, a walker that parses sequences (one per lane with a
sequence index, else one after another, handing entries to a recorder wave),
and builder waves that take 1 KiB tiles of the decoded stream in order,
build them in a history ring and write them out; a builder announces a tile
as built before its write-out, and as written out after it.  This module re-states
that protocol in Python, role by role, with the same counters, ring sizes,
window rule, record-ring rule, tile order and history-slot reuse rule, and
runs it under random interleavings: every role is a generator that yields
at each access to shared state, a scheduler picks which role takes the
next step, and in-flight DMA segments land after random delays.

It checks what the protocol must guarantee, at the moment of every access:
  - every input byte a role reads has landed and has not been overwritten
    (its ring slot holds that byte's segment);
  - every record a builder reads is still in its ring slot;
  - every history byte a tile's match reads belongs to a final tile (or to
    bytes of the same tile built before it), in the slot that holds it;
  - a tile overwrites a history slot only after every tile that reads the
    slot's previous tile is built and the previous tile is written out;
  - a tile's write-out reads only its own bytes (its slot is not reused
    while the write-out runs);
  - no interleaving deadlocks (a step bound far above the work);
and at the end that the decoded chunk equals the expected bytes.

With `static_tiles` builder b takes tiles b, b + nb, b + 2 nb, ... (the
matrix-product mode) instead of the next tile from the shared counter.

With `checksum` one builder's wave hashes the compressed bytes instead (a
reader that announces its position like the others) and the feeder streams
every block to its end.

`fault` plants one protocol mistake in the model (test of the model
itself): "hasher_silent" (the hasher never announces its position), "no_window" (the feeder ignores the readers' bound), "early_need"
(a builder releases its tile's input before building it), "no_slot_rule"
(a builder skips the history-slot reuse wait), "no_write_rule" (a
builder overwrites a slot without waiting for the old tile's write-out),
"no_split" (the walker
waits for the bytes after a literal run without announcing the run).

The model follows the kernel's structure, not its instruction-level
details: a builder's tile build is one step (its input and history reads
are protected from before the build until after the write-out, so an
atomic build sees the same protection), and the walker's fast paths are
represented by its byte-by-byte step, which is where its waits happen.
"""
from __future__ import annotations

import random

SEG = 1024
TILE = 1024
RING = 368
FF = 0xFFFFFFFF
ST_RUN, ST_DONE, ST_FAIL = 0, 1, 2
W_LAST, W_END, W_LIT, W_CONT = 1, 2, 4, 8


class ProtocolError(AssertionError):
    pass


def classes(hlog):
    """(history bytes, input ring bytes, chain entries) of a ring class."""
    if hlog == 16:
        return 1 << 16, 1 << 13, 32
    if hlog == 14:
        return 1 << 14, 1 << 14, 128
    raise ValueError(hlog)


def parse_block(blk):
    """The block's sequences as (token pos, literal start, L, dist, M) and its
    decoded bytes (plain byte-serial decode; the block must be valid)."""
    b = list(blk)
    seqs, out, y = [], bytearray(), 0
    while True:
        p = y
        t = b[y]
        y += 1
        L = t >> 4
        if L == 15:
            while True:
                v = b[y]
                y += 1
                L += v
                if v != 255:
                    break
        ys = y
        out += bytes(b[y:y + L])
        y += L
        if y == len(b):
            seqs.append((p, ys, L, 0, 0))
            return seqs, bytes(out)
        dist = b[y] | (b[y + 1] << 8)
        y += 2
        M = (t & 15) + 4
        if (t & 15) == 15:
            while True:
                v = b[y]
                y += 1
                M += v
                if v != 255:
                    break
        for _ in range(M):
            out.append(out[-dist])
        seqs.append((p, ys, L, dist, M))


class Chunk:
    """One chunk's decode under the protocol, with a seeded schedule."""

    def __init__(self, blk, n_out, index=None, hlog=14, dmax=65535, head=0, seed=0, builders=None, fault=None,
                 checksum=False, static_tiles=False, spec=False):
        self.fault = fault
        self.spec = spec      # the byte-output kernel's speculative build
        self.nspec = 0        # tiles built that way
        self.static_tiles = static_tiles
        self.checksum = checksum
        self.blk = bytes(blk)
        self.N = n_out
        self.hlog = hlog
        self.HIST, self.INR, self.CHAIN = classes(hlog)
        self.HTILES = self.HIST // TILE
        self.QMAX = self.INR // SEG
        self.dmax = dmax
        self.head = head
        self.y_end = head + len(self.blk)
        self.stream = bytes(head) + self.blk          # the 16-byte aligned blocks the feeder reads
        self.index = None if index is None else [head + int(v) for v in index]
        self.direct = self.index is not None and len(self.index) > 0
        self.nb = (builders if builders is not None else 5) + (1 if self.direct else 0) - (1 if checksum else 0)
        self.rng = random.Random(seed)
        self.seqs, self.expect = parse_block(self.blk)
        assert len(self.expect) == n_out
        self.ntiles = (n_out + TILE - 1) // TILE
        self.nseg = (self.y_end + SEG - 1) // SEG
        # shared state (the Ctl counters)
        self.in_avail = 0
        self.need = [0 if (i <= self.nb or (checksum and i == 7)) else FF for i in range(8)]
        self.bk = [0 if i < self.nb else FF for i in range(8)]
        self.next_tile = [i if i < self.nb else FF for i in range(8)]
        self.built_to = [i if i < self.nb else FF for i in range(8)]   # the kernel's built[]
        self.nrec = 0
        self.cov = 0
        self.wcnt = 0
        self.rcons = 0
        self.pstate = ST_RUN
        self.nfinished = 0
        self.tile_ctr = self.nb
        self.status = 0
        # rings
        self.inr_seg = [-1] * self.QMAX         # segment held by each input-ring slot (-1: none)
        self.inr_landed = [False] * self.QMAX
        self.recs = [None] * RING               # (record id, record)
        self.chain = [None] * self.CHAIN
        self.hist = bytearray(self.HIST)
        self.hist_tile = [-1] * self.HTILES     # tile held by each history slot
        self.hist_owner = [-1] * self.HIST      # tile whose byte each history byte holds
        self.final = [False] * self.ntiles        # history bytes final (built)
        self.written = [False] * self.ntiles      # written out too
        self.out = bytearray(n_out)
        self.built = [0] * self.ntiles
        self.inflight = []                      # [segment, steps until it lands]
        self.readers_of = self._readers()

    # ---------------------------------------------------------- checks
    def _readers(self):
        """For every tile, the tiles whose matches read it (from the true
        sequence list): a tile may only be overwritten after they are final."""
        readers = [set() for _ in range(self.ntiles)]
        o = 0
        for (_, _, L, dist, M) in self.seqs:
            o += L
            for q in range(o, o + M):
                src = q - dist
                if src // TILE != q // TILE:
                    readers[src // TILE].add(q // TILE)
            o += M
        return readers

    def read_input(self, a, b, who):
        for p in range(a, b):
            s = p // SEG
            slot = s % self.QMAX
            if self.inr_seg[slot] != s or not self.inr_landed[slot]:
                raise ProtocolError("%s read input byte %d: slot %d holds segment %d (landed %s)" % (
                    who, p, slot, self.inr_seg[slot], self.inr_landed[slot]))
        return self.stream[a:b]

    def read_record(self, j, who):
        e = self.recs[j % RING]
        if e is None or e[0] != j:
            raise ProtocolError("%s read record %d: slot holds %s" % (who, j, None if e is None else e[0]))
        return e[1]

    # ---------------------------------------------------------- roles
    def feeder(self):
        issued = landed = 0
        limit = min(self.QMAX, self.nseg)
        while True:
            while issued < limit and issued - landed < self.QMAX:
                slot = issued % self.QMAX
                self.inr_seg[slot] = issued
                self.inr_landed[slot] = False
                self.inflight.append([issued, self.rng.randint(1, 40)])
                issued += 1
                yield
            if issued == landed:
                if landed == self.nseg:
                    break
                yield
                if not self.checksum and self.nfinished == self.nb and self.need[0] == FF:
                    break
                used = min(self.need)
                yield
                limit = min(used // SEG + self.QMAX, self.nseg)
                if issued == limit:
                    yield
                continue
            # the readers' bound is read before the wait for the oldest segment
            used = min(self.need)
            yield
            while not self.inr_landed[landed % self.QMAX] or self.inr_seg[landed % self.QMAX] != landed:
                yield
            landed += 1
            self.in_avail = landed * SEG
            yield
            limit = min(used // SEG + self.QMAX, self.nseg)
            if self.fault == "no_window":
                limit = self.nseg
        while self.inflight:
            yield

    def memory(self):
        """Lands in-flight DMA segments in issue order after their delays."""
        while True:
            if self.inflight:
                seg = self.inflight[0]
                seg[1] -= 1
                if seg[1] <= 0:
                    self.inflight.pop(0)
                    slot = seg[0] % self.QMAX
                    if self.inr_seg[slot] == seg[0]:
                        self.inr_landed[slot] = True
            yield

    # records: (o, ys, L, dist, fill or None, flags)
    def rec_batch(self, st, ents):
        """The recorder's batch (Rec::batch): writes records for as many
        entries as the ring has room for, up to an announced literal run."""
        while st["nrec"] - st["rec_free"] >= RING:
            m = min(self.bk)
            yield
            st["rec_free"] = st["nrec"] if m == FF else m
            if st["nrec"] - st["rec_free"] < RING:
                break
            yield
        space = RING - (st["nrec"] - st["rec_free"])
        n = min(len(ents), space)
        for i in range(n):
            if ents[i][4] & W_LIT:
                n = i + 1
                break
        took = 0
        for i in range(n):
            ys, L, M, dist, flags, lastlit = ents[i]
            o = st["op"]
            if flags & W_LAST:
                if o + L != self.N:
                    return took, 4
                rec = (o, ys, L, 0, None, W_LAST)
                st["op"] = o + L
            elif flags & W_LIT:
                rec = (o, ys, L, 0, None, W_LIT)
                st["op"] = o + L
                st["pending"] = True
            else:
                if dist == 0 or dist > o + L or dist > self.dmax:
                    return took, 2
                fill = None
                if dist == 1:
                    if L > 0:
                        fill = lastlit
                    elif st["fill"] is not None:
                        fill = st["fill"]
                rec = (o, ys, L, dist, fill, 0)
                st["op"] = o + L + M
                st["fill"] = fill if dist == 1 else None
            self.recs[st["nrec"] % RING] = (st["nrec"], rec)
            st["nrec"] += 1
            took += 1
            yield
        if took:
            self.nrec, self.cov = st["nrec"], st["op"]
            yield
        if n and (ents[n - 1][4] & W_LAST) and took == n:
            return took, 0
        return took, None

    def rec_cont(self, st, M, dist, lastlit):
        """The match of an announced literal run (Rec::cont)."""
        o_end = st["op"]
        if dist == 0 or dist > o_end or dist > self.dmax:
            return 2
        j = st["nrec"] - 1
        _, rec = self.recs[j % RING]
        fill = lastlit if dist == 1 else None
        self.recs[j % RING] = (j, (rec[0], rec[1], rec[2], dist, fill, 0))
        st["op"] = o_end + M
        st["fill"] = fill
        st["pending"] = False
        self.cov = st["op"]
        yield
        return None

    def walker(self):
        st = {"nrec": 0, "rec_free": 0, "op": 0, "fill": None, "pending": False}
        self.wst = st
        w = {"y": self.head, "wy": None, "avail": 0, "pend": None, "split": False, "cnt": 0, "cons": 0,
             "pub": 0, "stop": False, "fin": None}

        def emit(ent):
            if self.direct:
                if ent[4] & W_END:
                    w["fin"] = ent[2]
                    w["stop"] = True
                    return
                if ent[4] & W_CONT:
                    r = yield from self.rec_cont(st, ent[2], ent[3], ent[5])
                else:
                    _, r = yield from self.rec_batch(st, [ent])
                if r is not None:
                    w["fin"] = r
                    w["stop"] = True
                return
            while w["cnt"] - w["cons"] >= self.CHAIN:
                w["cons"] = self.rcons
                yield
                if w["cnt"] - w["cons"] < self.CHAIN:
                    break
                if self.pstate != ST_RUN:
                    w["stop"] = True
                    return
                yield
            self.chain[w["cnt"] % self.CHAIN] = ent
            w["cnt"] += 1
            self.wcnt = w["cnt"]
            yield

        def need_input(upto):
            upto = min(upto, self.y_end)
            if w["avail"] >= upto:
                return
            w["avail"] = self.in_avail
            yield
            if w["avail"] >= upto:
                return
            if w["pend"] is not None and self.fault != "no_split":
                ys, L = w["pend"]
                w["pend"] = None
                w["split"] = True
                yield from emit((ys, L, 0, 0, W_LIT, 0))
            while w["avail"] < upto:
                yield
                w["avail"] = self.in_avail

        def byte_at(p):
            if w["wy"] is None or not (w["wy"] <= p < w["wy"] + 256):
                w["wy"] = p & ~3
                self.need[0] = w["wy"]
                yield
                yield from need_input(w["wy"] + 256)
                self.read_input(w["wy"], min(w["wy"] + 256, w["avail"], self.y_end), "walker window")
            return self.stream[p]

        def ext(q, v):
            while True:
                if q >= self.y_end:
                    return q, v, 1
                b = yield from byte_at(q)
                q += 1
                v += b
                if v > self.N:
                    return q, v, 3
                if b != 255:
                    return q, v, None

        def slow_step():
            y = w["y"]
            if y >= self.y_end:
                yield from emit((0, 0, 1, 0, W_END, 0))
                return False
            token = yield from byte_at(y)
            y += 1
            L = token >> 4
            if L == 15:
                y, L, e = yield from ext(y, L)
                if e:
                    yield from emit((0, 0, e, 0, W_END, 0))
                    return False
            if L > self.y_end - y:
                yield from emit((0, 0, 1, 0, W_END, 0))
                return False
            ys, e = y, y + L
            if e == self.y_end:
                yield from emit((ys, L, 0, 0, W_LAST, 0))
                return False
            if self.y_end - e < 2:
                yield from emit((0, 0, 1, 0, W_END, 0))
                return False
            w["pend"] = (ys, L) if L > 0 else None
            w["split"] = False
            lastlit = (yield from byte_at(e - 1)) if L else 0
            d0 = yield from byte_at(e)
            d1 = yield from byte_at(e + 1)
            dist = d0 | (d1 << 8)
            y = e + 2
            M = (token & 15) + 4
            if (token & 15) == 15:
                y, M, err = yield from ext(y, M)
                if err:
                    w["pend"] = None
                    yield from emit((0, 0, err, 0, W_END, 0))
                    return False
            w["y"] = y
            w["pend"] = None
            if w["split"]:
                yield from emit((0, 0, M, dist, W_CONT, lastlit))
            else:
                yield from emit((ys, L, M, dist, 0, lastlit))
            return not w["stop"]

        def index_batch(ij):
            """Listed sequences side by side; returns how many were taken
            (0: the next one needs the byte-by-byte step)."""
            idx = self.index
            left = len(idx) - ij
            nmax = min(64, left - 1)
            if nmax <= 0 or idx[ij] != w["y"]:
                return 0
            hi0 = min(idx[ij + 1] + 16, self.y_end)
            if hi0 > w["avail"]:
                if idx[ij + 1] - w["y"] + 16 > self.INR // 2:
                    return 0
                w["avail"] = self.in_avail
                yield
                if hi0 > w["avail"]:
                    w["pub"] = w["y"]
                    self.need[0] = w["pub"]
                    yield
                    while hi0 > w["avail"]:
                        yield
                        w["avail"] = self.in_avail
            ents = []
            for i in range(nmax):
                p, pn = idx[ij + i], idx[ij + i + 1]
                hi = min(pn + 16, self.y_end)
                if hi > w["avail"]:
                    break
                blk = self.read_input(p, hi, "walker batch")
                t = blk[0]
                k = 1
                L = t >> 4
                if L == 15:
                    while True:
                        v = blk[k]
                        k += 1
                        L += v
                        if v != 255:
                            break
                    if k - 1 > 13:
                        break
                ys = p + k
                q = ys + L
                lastlit = self.stream[q - 1] if L else 0
                dist = self.stream[q] | (self.stream[q + 1] << 8)
                M = (t & 15) + 4
                nxt = q + 2
                if (t & 15) == 15:
                    k2 = 0
                    while True:
                        v = self.stream[nxt]
                        nxt += 1
                        k2 += 1
                        M += v
                        if v != 255:
                            break
                    if k2 > 11:
                        break
                if nxt != pn:
                    yield from emit((0, 0, 5, 0, W_END, 0))
                    return -1
                ents.append((ys, L, M, dist, 0, lastlit))
            if not ents:
                return 0
            took, r = yield from self.rec_batch(st, ents)
            if r is not None:
                w["fin"] = r
                w["stop"] = True
                return -1
            w["y"] = idx[ij + took]
            if w["y"] - w["pub"] >= SEG:
                w["pub"] = w["y"]
                self.need[0] = w["pub"]
                yield
            return took

        if self.direct:
            ij = 0
            while not w["stop"]:
                if ij == len(self.index):
                    w["fin"] = 5
                    break
                took = yield from index_batch(ij)
                if took < 0:
                    break
                if took > 0:
                    ij += took
                    continue
                if w["y"] != self.index[ij]:
                    w["fin"] = 5
                    break
                ij += 1
                if not (yield from slow_step()):
                    break
        else:
            while not w["stop"]:
                if not (yield from slow_step()):
                    break
        self.need[0] = FF
        yield
        if self.direct:
            fin = w["fin"] if w["fin"] is not None else 5
            self.status = fin
            self.pstate = ST_DONE if fin == 0 else ST_FAIL
            yield

    def recorder(self):
        st = {"nrec": 0, "rec_free": 0, "op": 0, "fill": None, "pending": False}
        taken = 0
        final = None
        while final is None:
            while self.wcnt == taken:
                yield
            avail = self.wcnt
            if st["pending"]:
                ent = self.chain[taken % self.CHAIN]
                if ent[4] & W_END:
                    final = ent[2]
                    break
                r = yield from self.rec_cont(st, ent[2], ent[3], ent[5])
                if r is not None:
                    final = r
                    break
                taken += 1
                self.rcons = taken
                yield
                continue
            n = min(avail - taken, 64)
            ents = [self.chain[(taken + i) % self.CHAIN] for i in range(n)]
            for i, e in enumerate(ents):
                if e[4] & W_END:
                    if i == 0:
                        final = e[2]
                    ents = ents[:i]
                    break
            if final is not None:
                break
            took, r = yield from self.rec_batch(st, ents)
            taken += took
            if r is not None:
                final = r
                break
            self.rcons = taken
            yield
        self.status = final
        self.pstate = ST_DONE if final == 0 else ST_FAIL
        yield

    def hasher(self):
        """With checksums: hashes whole 1 KiB blocks of the compressed bytes in
        order as they land (two at a time when both have), announcing in
        need[7] the first byte it still reads; then the tail (the last
        partial block and the last 64 bytes)."""
        head, n = self.head, len(self.blk)
        hblocks = (n - 1) // 1024 if n > 240 else 0
        tail = min(1024 * hblocks, n - 64) if n > 240 else 0
        hb = avail = 0
        while hb < hblocks:
            while avail < head + 1024 * (hb + 1):
                avail = self.in_avail
                yield
            while hb < hblocks and head + 1024 * (hb + 1) <= avail:
                k = 2 if hb + 1 < hblocks and head + 1024 * (hb + 2) <= avail else 1
                self.read_input(head + 1024 * hb, head + 1024 * (hb + k), "hasher")
                hb += k
                yield
            if self.fault != "hasher_silent":
                self.need[7] = head + (1024 * hb if hb < hblocks else tail)
            yield
        while avail < self.y_end:
            avail = self.in_avail
            yield
        self.read_input(head + tail, self.y_end, "hasher tail")
        self.hashed = True
        self.need[7] = FF
        yield

    def builder(self, b):
        k = 0
        nrec = cov = 0
        avail = 0
        done = fdone = 0
        need_pub = 0
        reach = (self.dmax + TILE - 1) // TILE
        t = b
        who = "builder %d" % b

        def rec(j):
            return self.read_record(j, who)

        def start_of(j):
            return rec(j)[0] if j < nrec else cov

        def find_k(T):
            nonlocal k
            kk = k
            while kk + 1 < nrec and rec(kk + 1)[0] <= T:
                kk += 1
            if kk > k:
                k = kk
                self.bk[b] = k
                yield

        def wait_done(tiles, written):
            nonlocal done, fdone
            while done < tiles or fdone < written:
                done = min(self.built_to)
                yield
                fdone = min(self.next_tile)
                yield
                if done >= tiles and fdone >= written:
                    break
                if self.pstate == ST_FAIL:
                    return False
                yield
            return True

        def announce(T, r):
            nonlocal need_pub
            o, ys, L = r[0], r[1], r[2]
            off = min(max(T - o, 0), L)
            nd = ys + off
            if nd > need_pub:
                need_pub = nd
                self.need[1 + b] = nd
                yield

        while t < self.ntiles:
            if self.static_tiles:     # builder b takes tiles b, b + nb, ...
                u = t + self.nb
            else:
                u = self.tile_ctr
                self.tile_ctr += 1
            yield
            T, Tend = t * TILE, min(t * TILE + TILE, self.N)
            ok = True
            while cov < Tend:
                nrec, cov = self.nrec, self.cov
                yield
                if cov >= Tend:
                    break
                if self.pstate != ST_RUN:
                    nrec, cov = self.nrec, self.cov
                    yield
                    ok = cov >= Tend
                    break
                if nrec > 0:
                    yield from find_k(T)
                    yield from announce(T, rec(k))
                yield
            if not ok:
                break
            yield from find_k(T)
            yield from announce(T, rec(k))
            if self.fault == "early_need":
                j_last = k
                while j_last + 1 < nrec and rec(j_last + 1)[0] < Tend:
                    j_last += 1
                yield from announce(Tend, rec(j_last))
            # the records that meet the tile, and what they read
            js = []
            j = k
            while j < nrec and rec(j)[0] < Tend:
                js.append(j)
                j += 1
            m = len(js)
            seen = m < 64
            hard = not seen
            extra = src_need = in_end = 0
            for i, j in enumerate(js):
                o, ys, L, dist, fill, flags = rec(j)
                re = start_of(j + 1)
                le = o + L
                base = max(le, T)
                pend = min(re, Tend)
                copy = base < pend and fill is None and not (flags & (W_LAST | W_LIT))
                if le > T:
                    in_end = max(in_end, ys + (min(le, Tend) - o))
                if copy:
                    s_hi = base if dist == 1 else pend - dist
                    if seen and dist > 1 and (dist < 16 or dist < pend - base):
                        hard = True
                    if seen and s_hi > T:
                        extra += 1
                    src_need = max(src_need, min(s_hi, T))
            if seen and m > 16 and 2 * (1 + extra) > m:
                hard = True
            need_tiles = (src_need + TILE - 1) // TILE
            slot_tiles = written = 0
            if t >= self.HTILES and self.fault != "no_slot_rule":
                if reach < self.HTILES:
                    slot_tiles = t - self.HTILES + reach + 1
                    need_tiles = max(need_tiles, slot_tiles)
                else:
                    hard = hard or extra > 0
                    need_tiles = slot_tiles = t
                if self.fault != "no_write_rule":
                    written = t - self.HTILES + 1
            # speculative build: while the sources are not all built, wait
            # for the slot rule alone, build at once, then wait for the
            # sources and make the copies again in record order
            spec = False
            if self.spec and not hard and slot_tiles < need_tiles:
                if done < need_tiles or fdone < written:
                    done = min(self.built_to)
                    yield
                    fdone = min(self.next_tile)
                    yield
                spec = done < need_tiles or fdone < written
            ok = yield from wait_done(slot_tiles if spec else need_tiles, written)
            if not ok:
                break
            while avail < in_end:
                avail = self.in_avail
                yield
                if avail < in_end:
                    if self.pstate == ST_FAIL:
                        ok = False
                        break
                    yield
            if not ok:
                break
            # build the tile (one step: its reads are protected throughout)
            slot = t % self.HTILES
            old = self.hist_tile[slot]
            if old >= 0:
                pending = [x for x in self.readers_of[old] if not self.final[x] and x != t]
                if pending:
                    raise ProtocolError("%s overwrote tile %d's history while tiles %s still read it" % (
                        who, old, pending[:4]))
                if not self.written[old]:
                    raise ProtocolError("%s overwrote tile %d's history before its write-out" % (who, old))
            self.hist_tile[slot] = t
            if spec:   # literals and known-byte runs final, copies not yet
                self.nspec += 1
                for j in js:
                    o, ys, L, dist, fill, flags = rec(j)
                    a, e = max(o, T), min(o + L, Tend)
                    if a < e:
                        lit = self.read_input(ys + (a - o), ys + (e - o), who + " literals")
                        for q in range(a, e):
                            self.hist[q % self.HIST] = lit[q - a]
                            self.hist_owner[q % self.HIST] = t
                    for q in range(max(o + L, T), min(start_of(j + 1), Tend)):
                        self.hist_owner[q % self.HIST] = t
                        self.hist[q % self.HIST] = fill if fill is not None else self.rng.randrange(256)
                yield
                if self.fault != "spec_no_wait":
                    ok = yield from wait_done(need_tiles, written)
                    if not ok:
                        break
            for j in js:
                o, ys, L, dist, fill, flags = rec(j)
                re = start_of(j + 1)
                a, e = max(o, T), min(o + L, Tend)
                if a < e and not spec:
                    lit = self.read_input(ys + (a - o), ys + (e - o), who + " literals")
                    for q in range(a, e):
                        self.hist[q % self.HIST] = lit[q - a]
                        self.hist_owner[q % self.HIST] = t
                a, e = max(o + L, T), min(re, Tend)
                for q in range(a, e):
                    self.hist_owner[q % self.HIST] = t
                    if fill is not None:
                        self.hist[q % self.HIST] = fill
                        continue
                    src = q - dist
                    st_ = src // TILE
                    # the source byte must still hold tile st_'s byte (a
                    # source in this tile's own slot, a ring length back,
                    # lies ahead of the bytes written so far), and that
                    # tile must be final unless it is this one
                    own = self.hist_owner[src % self.HIST]
                    if own != st_ or (st_ != t and not self.final[st_]):
                        raise ProtocolError("%s tile %d read byte %d of tile %d (final %s, byte holds tile %d)" % (
                            who, t, src, st_, self.final[st_], own))
                    self.hist[q % self.HIST] = self.hist[src % self.HIST]
            self.built[t] += 1
            self.final[t] = True
            self.built_to[b] = u
            yield
            # the write-out reads the tile's slot, in two steps; tiles that
            # copy from it may be built meanwhile
            for a, e in ((T, min(T + TILE // 2, Tend)), (min(T + TILE // 2, Tend), Tend)):
                for q in range(a, e):
                    if self.hist_owner[q % self.HIST] != t:
                        raise ProtocolError("%s write-out of tile %d read byte %d after tile %d overwrote it" % (
                            who, t, q, self.hist_owner[q % self.HIST]))
                    self.out[q] = self.hist[q % self.HIST]
                yield
            self.written[t] = True
            self.next_tile[b] = u
            yield
            t = u
        self.need[1 + b] = FF
        self.bk[b] = FF
        self.built_to[b] = FF
        self.next_tile[b] = FF
        yield
        self.nfinished += 1
        yield

    # ---------------------------------------------------------- run
    def run(self, max_steps=None):
        roles = {"feeder": self.feeder(), "memory": self.memory(), "walker": self.walker()}
        builders = list(range(self.nb - 1)) + ([self.nb - 1] if self.direct else [])
        if not self.direct:
            roles["recorder"] = self.recorder()
            builders = list(range(self.nb))
        if self.checksum:   # one builder wave fewer (nb counts it already)
            roles["hasher"] = self.hasher()
            self.hashed = False
        for b in builders:
            roles["builder %d" % b] = self.builder(b)
        # uneven speeds: each role gets a random weight
        names = [n for n in roles if n != "memory"]
        weights = {n: self.rng.choice((1, 2, 4, 8)) for n in names}
        live = set(names)
        work = len(self.seqs) + self.ntiles + self.nseg
        max_steps = max_steps or 4000 * work + 200000
        steps = 0
        while live:
            steps += 1
            if steps > max_steps:
                raise ProtocolError("no progress after %d steps: live roles %s, nrec %d cov %d in_avail %d "
                                    "need %s next_tile %s" % (steps, sorted(live), self.nrec, self.cov,
                                                              self.in_avail, self.need, self.next_tile))
            next(roles["memory"])
            ls = sorted(live)
            n = self.rng.choices(ls, weights=[weights[x] for x in ls])[0]
            try:
                next(roles[n])
            except StopIteration:
                live.discard(n)
        return self.status, bytes(self.out), steps
