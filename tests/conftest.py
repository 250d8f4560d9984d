import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large CPU-side work (full-size oracle runs)")


def first_difference(a, b):
    """None when two byte strings (or equal-length lists of them) are equal,
    else a short account of where they first differ.  A failed `==` on long
    byte strings makes pytest run difflib over their reprs, which at stream
    sizes takes minutes; the tests compare through this instead."""
    if isinstance(a, (list, tuple)) and isinstance(b, (list, tuple)):
        if len(a) != len(b):
            return f"{len(a)} items vs {len(b)}"
        for i, (x, y) in enumerate(zip(a, b)):
            d = first_difference(x, y)
            if d is not None:
                return f"item {i}: {d}"
        return None
    a, b = bytes(a), bytes(b)
    if a == b:
        return None
    m = min(len(a), len(b))
    idx = np.flatnonzero(np.frombuffer(a, np.uint8, m) != np.frombuffer(b, np.uint8, m))
    if idx.size == 0:
        return f"lengths {len(a)} vs {len(b)}, equal over the first {m} bytes"
    i = int(idx[0])
    return (f"lengths {len(a)} vs {len(b)}, {idx.size} differing bytes, first at {i}: "
            f"{a[i:i + 8].hex()} vs {b[i:i + 8].hex()}")


def assert_same_bytes(got, want, what=""):
    d = first_difference(got, want)
    if d is not None:
        raise AssertionError(f"{what}: {d}" if what else d)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a golden fixture: `key = value` lines, `#` comments, `---`
    separates cases.  Returns a list of dicts of raw strings."""
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line == "---":
                cases.append(cur)
                cur = {}
                continue
            k, v = line.split("=", 1)
            cur[k.strip()] = v.strip()
    cases.append(cur)
    return cases


def escape_order_input(g):
    """The tensor of golden/escape_order.txt: +1, -1 alternating, with the
    listed (+4, -4) and (0, 0) pairs."""
    import numpy as np
    x = np.tile(np.array([0x3F80, 0xBF80], dtype=np.uint16), int(g["N"]) // 2)
    for i in (int(t) for t in g["pos4"].split()):
        x[i], x[i + 1] = 0x4080, 0xC080
    for i in (int(t) for t in g["zero_pairs"].split()):
        x[i], x[i + 1] = 0, 0
    return x


def check_escape_order_stream(s, g):
    """Assert that stream bytes s are the hand-derived stream of
    golden/escape_order.txt."""
    import numpy as np
    le = lambda o, n: int.from_bytes(s[o:o + n], "little")
    N, K = int(g["N"]), int(g["K"])
    G = -(-N // 2048)
    assert le(0, 4) == 0x3142435A and le(4, 2) == 1 and s[6] == int(g["L"]) and s[7] == 0
    assert le(8, 8) == N and le(16, 4) == int(g["chunk"]) and le(20, 4) == K
    assert le(24, 8) == int(g["E"]) and le(32, 8) == int(g["total"]) == len(s)
    code_off, sm_off, esc_off = int(g["code_off"]), int(g["sm_off"]), int(g["esc_off"])
    assert (le(40, 8), le(48, 8), le(56, 8)) == (code_off, sm_off, esc_off)
    assert [le(64 + 4 * k, 4) for k in range(K + 1)] == [int(t) for t in g["table"].split()]
    goff = 64 + 4 * (K + 1)
    assert [le(goff + 2 * i, 2) for i in range(G)] == [int(t) for t in g["gtab"].split()]
    assert not any(s[goff + 2 * G:code_off])
    words = np.frombuffer(s[code_off:sm_off], dtype="<u4").reshape(G, 3, 64)
    assert (words[:, 0, :] == 0xFFFFFFFF).all() and (words[:, 2, :] == 0xFFFFFFFF).all()
    want = np.zeros((G, 64), dtype=np.uint32)
    for item in g["plane1"].split():
        gl, w = item.split("=")
        gi, li = (int(t) for t in gl.split(":"))
        want[gi, li] = int(w, 16)
    assert np.array_equal(words[:, 1, :], want)
    x = escape_order_input(g)
    sm = np.where((x >> 15) == 1, 0x80, 0).astype(np.uint8)
    assert np.array_equal(np.frombuffer(s[sm_off:esc_off], dtype=np.uint8), sm)
    assert_same_bytes(s[esc_off:], bytes(int(t, 16) for t in g["escapes"].split()), "escapes")
