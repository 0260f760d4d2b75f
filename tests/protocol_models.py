"""Host-side models of the two-shot hand-offs, for tests/test_protocols.py.

Each model restates one hand-off of the reduce kernels as a set of workgroups whose shared-memory steps
(atomic reads, writes and read-modify-writes on the barrier words) a scheduler interleaves, either
exhaustively or at random.  A publish that the kernels issue as a non-returning atomic may land at any
later step of the same launch, so the models deliver those late.  No model reads anything the GPU
library produced; the tests compare their outcomes with what each protocol promises."""
from __future__ import annotations

import random

MASK32 = 0xFFFFFFFF
TAKEN = 0xFFFFFFFF


def s32(v: int) -> int:
    v &= MASK32
    return v - (1 << 32) if v & 0x80000000 else v


# ---------------------------------------------------------------------------------- XCD-local flags

def xcd_flag_outcomes(spin_limit: int, same_xcd: bool):
    """Every interleaving of one unit's producer and copier (per-unit flag of the XCD-local two-shot).

    Producer: write the stage; exchange the flag for its publish value P; if the old value was TAKEN,
    store 0.  Copier: poll up to spin_limit + 1 times; on a timeout, compare-and-swap 0 -> TAKEN (a
    success means: recompute, the producer clears the flag); otherwise clear the flag and copy if P
    names its own XCD, else recompute.  Returns the set of (final flag, copier mode, stage written
    when the copier decided) over all interleavings."""
    P = 1 if same_xcd else 2
    outcomes = set()

    def run(pp, cp, flag, stage, spins, mode, stage_at_decision, old):
        # pp: producer pc (0 write stage, 1 exchange, 2 maybe clear, 3 done)
        # cp: copier pc (0 poll, 1 cas, 2 clear and decide, 3 done)
        if pp == 3 and cp == 3:
            outcomes.add((flag, mode, stage_at_decision))
            return
        if pp < 3:
            if pp == 0:
                run(1, cp, flag, True, spins, mode, stage_at_decision, old)
            elif pp == 1:
                run(2, cp, P, stage, spins, mode, stage_at_decision, flag)
            else:
                run(3, cp, 0 if old == TAKEN else flag, stage, spins, mode, stage_at_decision, old)
        if cp < 3:
            if cp == 0:
                if flag != 0:
                    run(pp, 2, flag, stage, spins, mode, stage_at_decision, old)
                elif spins + 1 > spin_limit:
                    run(pp, 1, flag, stage, spins + 1, mode, stage_at_decision, old)
                else:
                    run(pp, 0, flag, stage, spins + 1, mode, stage_at_decision, old)
            elif cp == 1:
                if flag == 0:
                    run(pp, 3, TAKEN, stage, spins, "recompute", stage, old)
                else:
                    run(pp, 2, flag, stage, spins, mode, stage_at_decision, old)
            else:
                m = "copy" if flag == 1 else "recompute"
                run(pp, 3, 0, stage, spins, m, stage, old)

    run(0, 0, 0, False, 0, None, None, None)
    return outcomes


# ---------------------------------------------------------------------------------- per-tile flags

def tile_flag_outcomes(spin_limit: int, rearm: str):
    """Every interleaving of one phase-1 tile's producer and the phase-2 lane that waits for it
    (per-tile hand-off of the chunk kernels).  The producer writes the stage, then publishes with a
    non-returning +1 that lands at some later step.  The consumer polls (signed compare) up to
    spin_limit + 1 times, sets the error bit on a timeout, copies, and gives the release back --
    rearm "sub" subtracts 1 (the kernels), "store" stores 0 (the earlier form).  Returns the set of
    (final flag, error bit, copy saw the stage) over all interleavings."""
    outcomes = set()

    def run(pp, cp, flag, stage, spins, err, saw, pending):
        # pp: 0 write stage, 1 issue +1 (pending until delivered), 2 done; cp: 0 poll, 1 copy, 2 re-arm, 3 done
        if pp == 2 and cp == 3 and not pending:
            outcomes.add((s32(flag), err, saw))
            return
        if pending:  # deliver the in-flight +1
            run(pp, cp, (flag + 1) & MASK32, stage, spins, err, saw, False)
        if pp == 0:
            run(1, cp, flag, True, spins, err, saw, pending)
        elif pp == 1:
            run(2, cp, flag, stage, spins, err, saw, True)
        if cp == 0:
            if s32(flag) >= 1:
                run(pp, cp + 1, flag, stage, spins, err, saw, pending)
            elif spins + 1 > spin_limit:
                run(pp, cp + 1, flag, stage, spins + 1, 1, saw, pending)
            else:
                run(pp, 0, flag, stage, spins + 1, err, saw, pending)
        elif cp == 1:
            run(pp, 2, flag, stage, spins, err, stage, pending)
        elif cp == 2:
            nf = (flag - 1) & MASK32 if rearm == "sub" else 0
            run(pp, 3, nf, stage, spins, err, saw, pending)

    run(0, 0, 0, False, 0, 0, None, False)
    return outcomes


# ---------------------------------------------------------------------------------- chunk barrier

def chunk_barrier_random(t1: int, t2: int, spin_limit: int, rearm: str, rng: random.Random):
    """One chunk: t1 producers publish done1 += 1 (non-returning, delivered late); t2 consumers wait for
    done1 >= t1 (signed, bounded), then count themselves out on done2 (returning); the one that sees
    t2 - 1 re-arms: done2 = 0 and done1 -= t1 ("sub", delivered late like any non-returning atomic)
    or done1 = 0 ("store", the earlier form).  One random interleaving; returns (done1, done2, error
    bit, whether some consumer passed its wait before every producer had published) at the end."""
    done1 = done2 = 0
    err = 0
    published = 0
    early = False
    pending = []  # deltas of non-returning atomics on done1 in flight
    prod = [0] * t1  # 0 publish, 1 done
    cons = [[0, 0] for _ in range(t2)]  # [pc, spins]; pc 0 wait, 1 count out, 2 done
    while True:
        moves = [("p", i) for i in range(t1) if prod[i] == 0]
        moves += [("c", i) for i in range(t2) if cons[i][0] < 2]
        moves += [("d", i) for i in range(len(pending))]
        if not moves:
            return done1, done2, err, early
        kind, i = rng.choice(moves)
        if kind == "d":
            done1 = (done1 + pending.pop(i)) & MASK32
        elif kind == "p":
            prod[i] = 1
            published += 1
            pending.append(1)
        else:
            pc, spins = cons[i]
            if pc == 0:
                if s32(done1) >= t1:
                    cons[i][0] = 1
                    early = early or published < t1
                elif spins + 1 > spin_limit:
                    cons[i] = [1, spins + 1]
                    err = 1
                else:
                    cons[i][1] = spins + 1
            else:
                d = done2
                done2 = (done2 + 1) & MASK32
                cons[i][0] = 2
                if d == t2 - 1:
                    done2 = 0
                    if rearm == "sub":
                        pending.append(-t1)
                    else:
                        done1 = 0


# ---------------------------------------------------------------------------------- grid barrier

def grid_barrier_random(C: int, t1: int, t2: int, residency: int, rng: random.Random, max_steps: int = 200000):
    """The grid barrier's per-chunk work pools.  N = C*(t1+t2) workgroups start in a random order, at
    most `residency` at a time.  Workgroup b tries the phase-1 pools claim[c] from its home chunk b % C
    on (fetch-and-add; a value below t1 is a tile), then the phase-2 pools done2[c] (below t2 is a
    group); a phase-1 tile publishes done1[c] += 1 (non-returning, delivered late); a phase-2 group
    waits until every done1[x] >= t1; every workgroup then counts itself out on gdone, and the one that
    sees N - 1 re-arms claim, done2 and gdone to 0 and subtracts t1 from every done1.

    Returns a dict: claims (ordered list of (step, kind, chunk, ticket)), no_work (workgroups that found
    every pool empty), finished (all workgroups ended), words (final claim, done1, done2, gdone)."""
    N = C * (t1 + t2)
    claim = [0] * C
    done1 = [0] * C
    done2 = [0] * C
    gdone = 0
    pending = []  # (chunk, delta) in flight on done1
    order = list(range(N))
    rng.shuffle(order)
    started, next_start, live = 0, 0, []
    state = {}  # b -> dict(pc, i, work)
    claims, no_work = [], 0
    step = 0
    while step < max_steps:
        step += 1
        moves = []
        if next_start < N and len(live) < residency:
            moves.append(("start", None))
        moves += [("run", b) for b in live]
        moves += [("deliver", j) for j in range(len(pending))]
        if not moves:
            break
        kind, arg = rng.choice(moves)
        if kind == "start":
            b = order[next_start]
            next_start += 1
            live.append(b)
            state[b] = {"pc": "p1", "i": 0, "work": None}
            continue
        if kind == "deliver":
            c, dlt = pending.pop(arg)
            done1[c] = (done1[c] + dlt) & MASK32
            continue
        b = arg
        st = state[b]
        c0 = b % C
        if st["pc"] == "p1":  # one claim attempt on the next phase-1 pool
            cc = (c0 + st["i"]) % C
            t = claim[cc]
            claim[cc] += 1
            st["i"] += 1
            if t < t1:
                st["work"] = ("p1", cc, t)
                claims.append((step, "p1", cc, t))
                st["pc"] = "publish"
            elif st["i"] == C:
                st["pc"], st["i"] = "p2", 0
        elif st["pc"] == "p2":
            cc = (c0 + st["i"]) % C
            t = done2[cc]
            done2[cc] += 1
            st["i"] += 1
            if t < t2:
                st["work"] = ("p2", cc, t)
                claims.append((step, "p2", cc, t))
                st["pc"], st["i"] = "wait", 0
            elif st["i"] == C:
                no_work += 1
                st["pc"] = "finish"
        elif st["pc"] == "publish":
            pending.append((st["work"][1], 1))
            st["pc"] = "finish"
        elif st["pc"] == "wait":  # one poll of the next chunk's release count
            if s32(done1[st["i"]]) >= t1:
                st["i"] += 1
                if st["i"] == C:
                    st["pc"] = "finish"
        elif st["pc"] == "finish":
            d = gdone
            gdone += 1
            if d == N - 1:
                for x in range(C):
                    claim[x] = 0
                    done2[x] = 0
                    pending.append((x, -t1))
                gdone = 0
            st["pc"] = "end"
            live.remove(b)
    while pending:  # the launch ends only once every atomic has landed
        c, dlt = pending.pop()
        done1[c] = (done1[c] + dlt) & MASK32
    finished = next_start == N and not live
    return {"claims": claims, "no_work": no_work, "finished": finished,
            "words": (claim, [s32(v) for v in done1], done2, gdone)}


# ---------------------------------------------------------------------------------- last arriver

def last_arriver_random(t1: int, ratio: int, rng: random.Random):
    """Phase-1 tiles arrive in a random order on their group's count (returning fetch-and-add); the one
    whose add completes the group stores 0 and copies it.  Returns (copiers per group, whether every
    copier came after all of its group's members, final counts)."""
    t2 = -(-t1 // ratio)
    counts = [0] * t2
    arrived = [0] * t2
    copiers = [[] for _ in range(t2)]
    ok = True
    for k in rng.sample(range(t1), t1):
        q = k // ratio
        members = ratio if (q + 1) * ratio <= t1 else t1 - q * ratio
        old = counts[q]
        counts[q] += 1
        arrived[q] += 1
        if old == members - 1:
            counts[q] = 0
            copiers[q].append(k)
            ok = ok and arrived[q] == members
    return [len(c) for c in copiers], ok, counts


# ------------------------------------------------------------------- XCD-local units, last arriver

def xcd_last_random(members: int, xcc_of: list, rng: random.Random):
    """The members of one copy group publish in a random order.  Each adds 1 + (1 << (8 + 4*xcc)) to the
    group's 64-bit arrival word (xcc < 8; a larger id adds only the count); the one whose add completes
    the count stores 0 and decides: copy the group from the stage when every member's field says they
    ran on its own XCC, else recompute it.  Returns (copiers, decision, word at the end, whether every
    member had published when the decision was taken)."""
    word, published, copiers, decision, complete = 0, 0, [], None, False
    for k in rng.sample(range(members), members):
        xcc = xcc_of[k]
        add = 1 + ((1 << (8 + 4 * xcc)) if xcc < 8 else 0)
        old = word
        word = (word + add) & ((1 << 64) - 1)
        published += 1
        if (old & 0xFF) == members - 1:
            word = 0
            copiers.append(k)
            local = xcc < 8 and ((old + add) >> (8 + 4 * xcc)) & 15 == members
            decision = "copy" if local else "recompute"
            complete = published == members
    return copiers, decision, word, complete
