"""Replays ``tests/golden/manager_trace.txt`` against a block-manager adapter.

An adapter exposes: ``create(seq, n)``, ``fork(p, c)``, ``append(seq) ->
(slot, pair|None)``, ``cow(seq, lb) -> pair|None``, ``release(seq)``,
``table(seq)``, ``length(seq)``, ``refcount(b)``, ``free_order()`` (blocks in
hand-out order) and raises ``exhausted`` on an empty pool.
"""

import os

TRACE = os.path.join(os.path.dirname(__file__), "golden", "manager_trace.txt")


def load():
    lines = []
    with open(TRACE) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if line:
                lines.append(line)
    return lines


def replay(make, exhausted):
    """``make(num_blocks, block_size, free_order)`` builds the adapter."""
    lines = load()
    head = lines[0].split()
    assert head[0] == "pool"
    nb, bs = int(head[1]), int(head[2])
    mgr = make(nb, bs, [int(x) for x in head[3:]])
    checked = 0
    for line in lines[1:]:
        if line.startswith("expect"):
            parts = line.split()
            what, args = parts[1], [int(x) for x in parts[2:]]
            if what == "table":
                assert list(mgr.table(args[0])) == args[1:], line
            elif what == "len":
                assert mgr.length(args[0]) == args[1], line
            elif what == "rc":
                assert mgr.refcount(args[0]) == args[1], line
            elif what == "free":
                assert list(mgr.free_order()) == args, line
            else:
                raise ValueError(line)
            checked += 1
            continue
        call, result = [x.strip() for x in line.split("=>")]
        op, *args = call.split()
        args = [int(x) for x in args]
        res = result.split()
        if res[0] == "enomem":
            try:
                getattr(mgr, op)(*args)
            except exhausted:
                checked += 1
                continue
            raise AssertionError(f"expected exhaustion: {line}")
        out = getattr(mgr, op)(*args)
        if op == "append":
            slot, pair = out
            assert res[0] == "slot" and slot == int(res[1]), line
            want = (int(res[3]), int(res[4])) if len(res) > 2 else None
            assert (tuple(pair) if pair is not None else None) == want, line
        elif op == "cow":
            want = None if res[0] == "none" else (int(res[1]), int(res[2]))
            assert (tuple(out) if out is not None else None) == want, line
        else:
            assert res == ["ok"], line
        checked += 1
    return checked
