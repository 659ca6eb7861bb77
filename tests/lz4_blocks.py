"""Host-side walk over LZ4 raw blocks, for checks that need the sequence
structure (not the decoded bytes) of a block the packer wrote."""


def max_match_distance(blk):
    """Largest match distance in a valid LZ4 block (host-side walk)."""
    b = [int(v) for v in blk]
    y, best = 0, 0
    while True:
        t = b[y]; y += 1
        L = t >> 4
        if L == 15:
            while True:
                v = b[y]; y += 1; L += v
                if v != 255: break
        y += L
        if y >= len(b):
            return best
        best = max(best, b[y] | (b[y + 1] << 8))
        y += 2
        if (t & 15) == 15:
            while True:
                v = b[y]; y += 1
                if v != 255: break


def sequence_starts(blk):
    """Offsets of the sequences (tokens) of an LZ4 block, in order; the walk
    stops after the literal-only last sequence or at the sequence that
    breaks the format (that one is still listed)."""
    b = [int(v) for v in blk]
    n, y, out = len(b), 0, []
    while y < n:
        out.append(y)
        t = b[y]
        y += 1
        L = t >> 4
        if L == 15:
            while True:
                if y >= n:
                    return out
                v = b[y]
                y += 1
                L += v
                if v != 255:
                    break
        if L > n - y:
            return out
        y += L
        if y == n or n - y < 2:
            return out
        y += 2
        if (t & 15) == 15:
            while True:
                if y >= n:
                    return out
                v = b[y]
                y += 1
                if v != 255:
                    break
    return out


def matches(blk):
    """(distance, length) of every match of a valid LZ4 block, in order."""
    b = [int(v) for v in blk]
    y, out = 0, []
    while True:
        t = b[y]; y += 1
        L = t >> 4
        if L == 15:
            while True:
                v = b[y]; y += 1; L += v
                if v != 255: break
        y += L
        if y >= len(b):
            return out
        d = b[y] | (b[y + 1] << 8)
        y += 2
        M = (t & 15) + 4
        if (t & 15) == 15:
            while True:
                v = b[y]; y += 1; M += v
                if v != 255: break
        out.append((d, M))
