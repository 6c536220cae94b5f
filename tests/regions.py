"""Region layout helpers for the tests (written from the layout reading, not
shared with either the oracle or the library).

Part c of m holds, for each width class k (q = 2, 4, 8, and 16 when a plan
has the 16-bit class; C lists the classes' counts), the stream positions
[base_k + floor(c C_k / m), base_k + floor((c+1) C_k / m)).  Its region is:
codes of the 2-bit, 4-bit, 8-bit (16-bit) super-groups (32 q bytes each),
then one fp32 scale unit per super-group, zero padding to 16 bytes, then 16
UINT8 group codes per super-group.  Code i sits at bit q*i of its payload,
LSB first.
"""
import numpy as np

QS = (2, 4, 8, 16)


def class_bases(C):
    return [int(sum(int(x) for x in C[:k])) for k in range(len(C))]


def part_ranges(C, m, c):
    """[(lo, count)] in stream positions for each class of C."""
    base = class_bases(C)
    out = []
    for k in range(len(C)):
        a = (c * int(C[k])) // m
        b = ((c + 1) * int(C[k])) // m
        out.append((base[k] + a, b - a))
    return out


def layout(counts):
    off = 0
    codes = []
    for k in range(len(counts)):
        codes.append(off)
        off += int(counts[k]) * 32 * QS[k]
    N = int(sum(counts))
    off_s = off
    off += 4 * N
    off = (off + 15) // 16 * 16
    off_c = off
    off += 16 * N
    return {"codes": codes, "s": off_s, "c": off_c, "bytes": off, "N": N}


def region_bytes(C, m, c):
    return layout([n for _, n in part_ranges(C, m, c)])["bytes"]


def sg_fields(region, C, m, c, pos):
    """(class k, codes[256], s float32, cg[16] uint8) of stream position pos."""
    rng = part_ranges(C, m, c)
    counts = [n for _, n in rng]
    lay = layout(counts)
    for k in range(len(C)):
        lo, n = rng[k]
        if lo <= pos < lo + n:
            idx = pos - lo
            local = sum(counts[:k]) + idx
            q = QS[k]
            raw = np.asarray(region[lay["codes"][k] + idx * 32 * q: lay["codes"][k] + (idx + 1) * 32 * q],
                             dtype=np.uint8)
            codes = unpack(raw, q)
            s = np.frombuffer(bytes(np.asarray(region[lay["s"] + 4 * local: lay["s"] + 4 * local + 4],
                                               dtype=np.uint8)), np.float32)[0]
            cg = np.asarray(region[lay["c"] + 16 * local: lay["c"] + 16 * local + 16], dtype=np.uint8)
            return k, codes, s, cg
    raise ValueError("position not in part")


def sg_raw(region, C, m, c, pos):
    """Raw bytes (codes, s, cg) of stream position pos, for bit-exact compares."""
    rng = part_ranges(C, m, c)
    counts = [n for _, n in rng]
    lay = layout(counts)
    for k in range(len(C)):
        lo, n = rng[k]
        if lo <= pos < lo + n:
            idx = pos - lo
            local = sum(counts[:k]) + idx
            q = QS[k]
            a = lay["codes"][k] + idx * 32 * q
            return (bytes(region[a:a + 32 * q]), bytes(region[lay["s"] + 4 * local: lay["s"] + 4 * local + 4]),
                    bytes(region[lay["c"] + 16 * local: lay["c"] + 16 * local + 16]))
    raise ValueError("position not in part")


def unpack(raw, q):
    raw = np.asarray(raw, dtype=np.uint8)
    bits = np.unpackbits(raw, bitorder="little").reshape(256, q)
    weights = (1 << np.arange(q)).astype(np.uint32)
    return (bits.astype(np.uint32) * weights).sum(1).astype(np.uint16 if q > 8 else np.uint8)


def part_positions(C, m, c):
    """Stream positions of part c of m, in the part's order (class by class)."""
    return [p for lo, n in part_ranges(C, m, c) for p in range(lo, lo + n)]


def decode_sg(region, C, m, c, pos, levels):
    """Decoded values of stream position pos: fl(fl(c_g s) L[code]) per
    coordinate; levels[k] is the level table of class k."""
    k, codes, s, cg = sg_fields(region, C, m, c, pos)
    sigma = (cg.astype(np.float32) * np.float32(s)).astype(np.float32)
    L = np.asarray(levels[k], np.float32)
    return (np.repeat(sigma, 16) * L[codes]).astype(np.float32)
