"""Lattice point sets shared by the CPU tests (no library imports)."""
import numpy as np

from oracle import golay, leech


def shell2_vectors() -> np.ndarray:
    """Every minimal vector of the Leech lattice (norm 32 in the sqrt(8)
    frame), built from the three classical forms: (+-4, +-4, 0^22), +-2 on an
    octad with an even number of minus signs, and (-+3, +-1^23) along a
    codeword; the membership rule keeps the 196,560 lattice points."""
    out = []
    for i in range(24):
        for j in range(i + 1, 24):
            for si in (-4, 4):
                for sj in (-4, 4):
                    v = np.zeros(24, dtype=np.int8)
                    v[i], v[j] = si, sj
                    out.append(v)
    octads = [int(w) for w in golay.codewords() if golay.weight(w) == 8]
    for o in octads:
        pos = [i for i in range(24) if (o >> i) & 1]
        for s in range(256):
            if bin(s).count("1") % 2:
                continue
            v = np.zeros(24, dtype=np.int8)
            for t, p in enumerate(pos):
                v[p] = -2 if (s >> t) & 1 else 2
            out.append(v)
    words = golay.codewords()
    bits = ((words[:, None].astype(np.int64) >> np.arange(24)) & 1).astype(np.int8)
    base = np.where(bits == 1, -1, 1).astype(np.int8)  # x = 3 mod 4 on the codeword
    for p in range(24):
        v = base.copy()
        v[:, p] = np.where(bits[:, p] == 1, 3, -3)
        out.extend(v)
    x = np.array(out, dtype=np.int8)
    x = x[leech.is_leech_batch(x)]
    return x
