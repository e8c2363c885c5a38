"""Reader for the packed message format, written from its specification
(stream header, block table, per-segment DGC / AdaComp blocks with escapes
and checkpoints).  Used by tests to decode streams; it does not share code
with either encoder."""
import struct

MAGIC_STREAM = b"GCP2"
MAGIC_DGC = b"DGC1"
MAGIC_ADA = b"ADC1"
CKPT = 4096  # codes between checkpoints


def unpack(buf: bytes, seg_offsets):
    """Returns (kind, [ (entries, meta) per segment ]) where entries is a list of
    (flat_index, value) and meta holds n_s, E, the entry count, and k_s or
    scale."""
    assert buf[0:4] == MAGIC_STREAM, "bad stream magic"
    kind, nseg, zero = struct.unpack_from("<III", buf, 4)
    assert zero == 0 and nseg == len(seg_offsets)
    table = [struct.unpack_from("<QII", buf, 16 + 16 * s) for s in range(nseg)]
    pos = 16 + 16 * nseg
    segs = []
    for s in range(nseg):
        t_off, t_E, t_cnt = table[s]
        assert t_off == pos, "table offset must be where the block lies"
        magic = buf[pos:pos + 4]
        n_s, E = struct.unpack_from("<II", buf, pos + 4)
        assert E == t_E
        if kind == 1:
            assert magic == MAGIC_DGC
            (k_s,) = struct.unpack_from("<I", buf, pos + 12)
            meta = dict(n=n_s, E=E, count=t_cnt, k=k_s)
        else:
            assert magic == MAGIC_ADA
            (scale,) = struct.unpack_from("<f", buf, pos + 12)
            meta = dict(n=n_s, E=E, count=t_cnt, scale=scale)
        pos += 16
        codes = struct.unpack_from(f"<{E}H", buf, pos)
        pad = E % 2
        if pad:
            assert struct.unpack_from("<H", buf, pos + 2 * E)[0] == 0, "pad must be zero"
        pos += 2 * E + 2 * pad
        if kind == 1:
            vals = struct.unpack_from(f"<{E}f", buf, pos)
            pos += 4 * E
        nck = (E + CKPT - 1) // CKPT
        ckpts = [struct.unpack_from("<II", buf, pos + 8 * c) for c in range(nck)]
        pos += 8 * nck
        entries, p = [], 0
        for e, c in enumerate(codes):
            if e % CKPT == 0:
                assert ckpts[e // CKPT] == (len(entries), p), "checkpoint: entries and position before the code"
            if kind == 1:
                if c == 0xFFFF:
                    assert struct.pack("<f", vals[e]) == b"\0\0\0\0", "escape value must be +0.0"
                    p += 0xFFFF
                    continue
                rel = p + c
                entries.append((seg_offsets[s] + rel, vals[e]))
            else:
                if c == 0x7FFF:
                    p += 0x7FFF
                    continue
                rel = p + (c & 0x7FFF)
                entries.append((seg_offsets[s] + rel, -meta["scale"] if c & 0x8000 else meta["scale"]))
            p = rel + 1
            assert rel < n_s
        assert len(entries) == t_cnt
        if kind == 1:
            assert len(entries) == meta["k"]
        segs.append((entries, meta))
    assert pos == len(buf), "trailing bytes"
    return kind, segs
