"""Barrier / load / wait placement of the K-64 ping-pong GEMM (gemm_pp64_kernel), checked on the CPU.

The kernel's two wave groups (waves 0-3 and 4-7) share a 2-slot LDS ring of B A rows and B W
rows per stage (B = 256 or 128, the tile edge). Group g's wave of column quarter q multiplies A rows
[B/2 g, B/2 (g + 1)) by W rows [B/4 q, B/4 (q + 1)). Group 0's wave q loads A rows [B/4 q, B/4 (q + 1));
group 1's wave q loads W rows [B/4 q, B/4 (q + 1)), the rows it multiplies itself. This model writes out, per wave, the order of its
load issues, fragment reads, vmcnt waits and block barriers as the kernel's two loops place them,
and checks, for every stage count, that
  * all waves pass the same number of barriers;
  * a wave refills rows of a slot only after a barrier that every other reader of those rows passed
    after reading the slot's previous stage (its own reads complete before its later issues);
  * a wave reads a stage only after a barrier that follows the wait of every wave that loaded rows it
    reads;
  * every A and W row of a stage is loaded.
The split in which every wave loads 1/8 of A and 1/8 of W, with group 1 refilling right after its own
reads, fails the second check: that is the cross-wave race this ownership avoids.
"""
import pytest


def reads_of(w, B):
    g, q = divmod(w, 4)
    h, f = B // 2, B // 4
    return {("A", r) for r in range(h * g, h * g + h)} | {("W", r) for r in range(f * q, f * q + f)}


def loads_of(w, B, owner=True):
    g, q = divmod(w, 4)
    e, f = B // 8, B // 4
    if not owner:
        return {("A", r) for r in range(e * w, e * w + e)} | {("W", r) for r in range(e * w, e * w + e)}
    return {("A" if g == 0 else "W", r) for r in range(f * q, f * q + f)}


def program(grp, nk, L):
    ev = [("issue", 0)] + ([("issue", 1), ("wait", L)] if nk > 1 else [("wait", 0)]) + [("sync",)]
    for k in range(nk):
        if grp == 0:
            if 1 <= k and k + 1 < nk:
                ev.append(("issue", k + 1))
            ev += [("read", k), ("sync",)]
            if k + 1 < nk:
                ev.append(("wait", 0))
            ev.append(("sync",))
        else:
            if k == 0:
                ev.append(("sync",))
            ev.append(("read", k))
            if k + 2 < nk:
                ev.append(("issue", k + 2))
            if k + 1 < nk:
                ev.append(("wait", L if k + 2 < nk else 0))
            ev.append(("sync",))
            if k + 1 < nk:
                ev.append(("sync",))
    return ev + [("wait", 0)]


def violations(nk, B=256, owner=True):
    L = B // 32       # 8-row loads per wave per stage
    waves = [program(w // 4, nk, L) for w in range(8)]
    if len({sum(e[0] == "sync" for e in p) for p in waves}) != 1:
        return ["barrier counts differ"]
    info = []
    for p in waves:
        b, issued, rows = 0, [], []
        for e in p:
            if e[0] == "sync":
                b += 1
            elif e[0] == "issue":
                issued.append(e[1])
                rows.append(("issue", e[1], b))
            elif e[0] == "read":
                rows.append(("read", e[1], b))
            else:   # wait_vm<n>: all of this wave's loads but the newest n / L stages
                rows.append(("wait", set(issued[:len(issued) - e[1] // L]), b))
        info.append(rows)
    bad = []
    for w in range(8):
        for t, j, bi in info[w]:
            if t != "issue" or j < 2:
                continue
            for v in range(8):
                if v != w and loads_of(w, B, owner) & reads_of(v, B) and \
                        any(t2 == "read" and j2 == j - 2 and br >= bi for t2, j2, br in info[v]):
                    bad.append(f"wave {w} refills stage {j} over rows wave {v} may still read")
    for v in range(8):
        for t, j, br in info[v]:
            if t != "read":
                continue
            for w in range(8):
                if loads_of(w, B, owner) & reads_of(v, B) and \
                        not any(t2 == "wait" and j in d and bw < br for t2, d, bw in info[w]):
                    bad.append(f"wave {v} reads stage {j} before wave {w}'s rows are awaited")
    if len(set().union(*[loads_of(w, B, owner) for w in range(8)])) != 2 * B:
        bad.append("a row of the stage is never loaded")
    return bad


@pytest.mark.parametrize("B", [256, 128])
@pytest.mark.parametrize("nk", range(1, 20))
def test_pp64_schedule_is_race_free(nk, B):
    assert violations(nk, B) == []


@pytest.mark.parametrize("B", [256, 128])
def test_split_loads_with_early_refill_race_is_caught(B):
    assert any("refills" in v for v in violations(4, B, owner=False))
