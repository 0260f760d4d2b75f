"""Host-side checks of the two-shot hand-offs and of the gather planner (no GPU).

* The protocol models of tests/protocol_models.py, interleaved exhaustively or at random: every work
  item claimed once, nobody waits on work that has not been handed out, no copy reads a stage tile
  before its producer published it unless the error word says so, and every barrier word is zero when
  a launch ends -- also after a bounded wait gave up.
* The library's own plans (through its planning hooks, outside the mr.h ABI) against brute force: the
  XCD-local units of the two-shot cover every pack once, and the gather's phase masks are the set of
  per-piece phase differences."""
import ctypes
import random

import numpy as np
import pytest

import all_gather_amd as mr
import protocol_models as pm


# ---------------------------------------------------------------------------------- XCD-local flags

@pytest.mark.parametrize("spin_limit", [0, 1, 2, 3])
@pytest.mark.parametrize("same_xcd", [True, False])
def test_xcd_flag_every_interleaving(spin_limit, same_xcd):
    outcomes = pm.xcd_flag_outcomes(spin_limit, same_xcd)
    assert outcomes
    for flag, mode, stage_seen in outcomes:
        assert flag == 0, "a flag was left set at the end of the launch"
        assert mode in ("copy", "recompute")
        if mode == "copy":
            assert same_xcd and stage_seen, "a copy read a stage the producer had not published on this XCD"
    if not same_xcd:
        assert {m for _, m, _ in outcomes} == {"recompute"}
    if spin_limit >= 0 and same_xcd:
        assert any(m == "copy" for _, m, _ in outcomes)


# ------------------------------------------------------------------- XCD-local units, last arriver

def test_xcd_last_arriver_copies_once_and_only_its_own_xcc():
    rng = random.Random(13)
    for _ in range(3000):
        members = rng.randint(1, 15)
        home = rng.randint(0, 9)
        if rng.random() < 0.5:
            xcc_of = [home] * members
        else:
            xcc_of = [rng.randint(0, 9) for _ in range(members)]
        copiers, decision, word, complete = pm.xcd_last_random(members, xcc_of, rng)
        assert len(copiers) == 1 and complete and word == 0
        local = all(x == xcc_of[copiers[0]] for x in xcc_of) and xcc_of[copiers[0]] < 8
        assert decision == ("copy" if local else "recompute"), (xcc_of, copiers, decision)


# ---------------------------------------------------------------------------------- per-tile flags

@pytest.mark.parametrize("spin_limit", [0, 1, 3])
def test_tile_flag_rearm_by_subtraction(spin_limit):
    outcomes = pm.tile_flag_outcomes(spin_limit, "sub")
    for flag, err, saw in outcomes:
        assert flag == 0, "a late release survived the launch"
        assert saw or err, "a copy read an unpublished stage tile without setting the error bit"


def test_tile_flag_rearm_by_store_leaves_a_late_release():
    # the earlier form: the consumer stored 0 after a timeout and the producer's late +1 survived
    assert any(flag == 1 for flag, _, _ in pm.tile_flag_outcomes(0, "store"))


# ---------------------------------------------------------------------------------- chunk barrier

def test_chunk_barrier_counts_return_to_zero():
    rng = random.Random(7)
    for _ in range(3000):
        t1, t2 = rng.randint(1, 5), rng.randint(1, 3)
        d1, d2, err, early = pm.chunk_barrier_random(t1, t2, rng.choice([0, 1, 4, 1000]), "sub", rng)
        assert (pm.s32(d1), d2) == (0, 0)
        assert not early or err, "a consumer passed its wait early without an error"


def test_chunk_barrier_store_rearm_can_leave_a_count():
    rng = random.Random(8)
    left = [pm.chunk_barrier_random(3, 2, 0, "store", rng)[0] for _ in range(2000)]
    assert any(pm.s32(d1) != 0 for d1 in left)


# ---------------------------------------------------------------------------------- grid barrier

def test_grid_barrier_pools_random_interleavings():
    """300 random schedules of the work pools: random start order (not the index order), a random
    residency limit (from one workgroup at a time to all of them), late delivery of the releases."""
    rng = random.Random(11)
    for trial in range(300):
        C = rng.randint(1, 4)
        t1, t2 = rng.randint(1, 6), rng.randint(1, 3)
        N = C * (t1 + t2)
        res = pm.grid_barrier_random(C, t1, t2, rng.randint(1, N), rng)
        assert res["finished"], f"trial {trial}: deadlock (C={C} t1={t1} t2={t2})"
        assert res["no_work"] == 0, f"trial {trial}: a workgroup found no work"
        p1 = [(c, t) for _, k, c, t in res["claims"] if k == "p1"]
        p2 = [(c, t) for _, k, c, t in res["claims"] if k == "p2"]
        assert sorted(p1) == [(c, t) for c in range(C) for t in range(t1)], "phase-1 tiles not claimed exactly once"
        assert sorted(p2) == [(c, t) for c in range(C) for t in range(t2)], "phase-2 groups not claimed exactly once"
        last_p1 = max(s for s, k, _, _ in res["claims"] if k == "p1")
        first_p2 = min(s for s, k, _, _ in res["claims"] if k == "p2")
        assert first_p2 > last_p1, "a phase-2 group was claimed before the last phase-1 tile"
        claim, done1, done2, gdone = res["words"]
        assert claim == [0] * C and done1 == [0] * C and done2 == [0] * C and gdone == 0


# ---------------------------------------------------------------------------------- last arriver

def test_last_arriver_copies_each_group_once_after_all_members():
    rng = random.Random(12)
    for _ in range(2000):
        t1, ratio = rng.randint(1, 40), rng.randint(1, 6)
        copiers, ok, counts = pm.last_arriver_random(t1, ratio, rng)
        assert copiers == [1] * len(copiers) and ok and counts == [0] * len(counts)


# ---------------------------------------------------------------------------------- library plans

@pytest.fixture(scope="module")
def L():
    lib = mr.lib()
    lib.mrx_twoshot_plan.restype = ctypes.c_int
    lib.mrx_twoshot_plan.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64),
                                     ctypes.c_int]
    lib.mrx_gather_phase_masks.restype = ctypes.c_int
    lib.mrx_gather_phase_masks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_uint16),
                                           ctypes.POINTER(ctypes.c_uint16), ctypes.c_int]
    lib.mrx_needs_realign.restype = ctypes.c_int
    lib.mrx_needs_realign.argtypes = [ctypes.c_uint16, ctypes.c_uint64]
    lib.mrx_gather_tiles.restype = ctypes.c_int
    lib.mrx_gather_tiles.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int,
                                     ctypes.c_int, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_uint16)]
    return lib


FIELDS = ("xcd", "units", "run", "run_padded", "chunks", "chunk_units", "t1", "t2", "ratio", "unit1", "sync", "vec",
          "head", "npacks", "grid", "flags")


def _plan(L, W, n, dtype, out_addr, sync, shape, wait_free=0, same_phase=1):
    f = (ctypes.c_uint64 * 16)()
    assert L.mrx_twoshot_plan(W, n, mr.DTYPE_CODE[dtype], out_addr, same_phase, mr.TWOSHOT_SYNC[sync],
                              mr.TILE_SHAPE[shape], wait_free, f, 16) == 0
    return dict(zip(FIELDS, [int(v) for v in f]))


def test_xcd_units_cover_every_pack_once(L):
    """The XCD-local two-shot's roles, as the kernel computes them from the workgroup index (run x =
    b % 8, index s = b / 8; s < run_padded reduces unit x*run + s, larger s copy four units of the run),
    replayed over the library's own plans: every unit reduced once and copied once, by a later
    workgroup of the same run, every unit inside the message, and the flag words inside the
    workspace's flag area."""
    rng = random.Random(3)
    cases = [(8, 8_388_608, "bf16", 0, "tile", "auto"), (8, 4_194_304, "fp32", 0, "tile", "auto"),
             (8, 8_388_608 + 40, "bf16", 6, "tile", "auto"), (5, 33_554_432 + 3, "fp16", 2, "auto", "auto")]
    for _ in range(40):
        W = rng.randint(1, 8)
        dt = rng.choice(["bf16", "fp16", "fp32"])
        es = 2 if dt != "fp32" else 4
        cases.append((W, rng.randint(1, 3_000_000), dt, es * rng.randint(0, 7), "tile", "wide_pair"))
    for W, n, dt, addr, sync, shape in cases:
        p = _plan(L, W, n, dt, addr, sync, shape)
        assert p["xcd"] == 1, (W, n, dt)
        units, run, runp = p["units"], p["run"], p["run_padded"]
        assert p["grid"] == 8 * (runp + runp // 4) and runp % 4 == 0 and run * 8 >= units
        produced, copied = {}, {}
        for b in range(p["grid"]):
            x, s = b % 8, b // 8
            if s < runp:
                u = x * run + s
                if s < run and u < units:
                    assert u not in produced
                    produced[u] = (x, s)
            else:
                g = s - runp
                for r in range(4):
                    i = g * 4 + r
                    if i < run and x * run + i < units:
                        u = x * run + i
                        assert u not in copied
                        copied[u] = (x, s)
        assert set(produced) == set(range(units)) == set(copied)
        assert all(produced[u][0] == copied[u][0] and produced[u][1] < copied[u][1] for u in produced)
        npacks = p["npacks"]
        assert (units - 1) * 1024 < max(npacks, 1) <= units * 1024
        assert p["flags"] == units <= mr.workspace_bytes(W, n, dt) >> 8


def test_xcd_last_arriver_groups_cover_every_unit_once(L):
    """The last-arriver form on XCD-local units, as the kernel computes it from the workgroup index
    (run x = b % 8, unit x*run + s, copy group s // 4 of the run, its 64-bit arrival word x*groups + g),
    replayed over the library's plans: every unit produced once, each group's members all in one run,
    one arrival word per group inside the flag area, and that area inside the workspace's."""
    rng = random.Random(4)
    cases = [(8, 8_388_608, "bf16", 0, "auto", "auto"), (8, 2_097_152, "fp32", 0, "auto", "auto"),
             (8, 8_388_608 + 40, "bf16", 6, "last", "auto"), (8, 131_072, "bf16", 0, "auto", "auto"),
             (5, 600_001, "fp16", 4, "auto", "auto"), (3, 7, "fp32", 0, "auto", "auto")]
    for _ in range(40):
        W = rng.randint(1, 8)
        dt = rng.choice(["bf16", "fp16", "fp32"])
        es = 2 if dt != "fp32" else 4
        cases.append((W, rng.randint(1, 3_000_000), dt, es * rng.randint(0, 7), "last", "wide_pair"))
    for W, n, dt, addr, sync, shape in cases:
        p = _plan(L, W, n, dt, addr, sync, shape)
        assert p["xcd"] == 1 and p["sync"] == 3, (W, n, dt, p)
        units, run = p["units"], p["run"]
        groups = -(-run // 4)
        assert p["grid"] == 8 * run and run * 8 >= units
        produced, words = {}, {}
        for b in range(p["grid"]):
            x, s = b % 8, b // 8
            u = x * run + s
            if u >= units:
                continue
            assert u not in produced
            produced[u] = x
            words.setdefault(x * groups + s // 4, set()).add(u)
        assert set(produced) == set(range(units))
        up = p["unit1"]
        assert up in (64, 256, 1024) and (units - 1) * up < max(p["npacks"], 1) <= units * up
        for w, us in words.items():
            x, g = divmod(w, groups)
            assert us == {x * run + g * 4 + r for r in range(4) if g * 4 + r < run and x * run + g * 4 + r < units}
            assert max(us) // run == min(us) // run == x
        assert p["flags"] == 2 * 8 * groups and p["flags"] <= mr.workspace_bytes(W, n, dt) >> 8


def test_default_hand_off_choices(L):
    def pick(W, n, dt="bf16", **kw):
        p = _plan(L, W, n, dt, 0, "auto", "auto", **kw)
        return p["sync"], p["xcd"]
    # the last arriver on XCD-local units up to 32 MiB per rank (16-byte path, W <= 8), per-tile flags
    # above (XCD-local up to 64 MiB, then the chunk tiles)
    assert pick(8, 1000) == (3, 1)
    assert pick(8, 2_097_152) == (3, 1)              # 4 MiB
    assert pick(8, 4_194_304) == (3, 1)              # 8 MiB
    assert pick(8, 8_388_608) == (3, 1)              # 16 MiB, the headline size
    assert pick(8, 4_194_304, "fp32") == (3, 1)      # 16 MiB
    assert pick(8, 16_777_216) == (3, 1)             # 32 MiB
    assert pick(8, 16_777_216 + 8) == (0, 1)         # just over 32 MiB
    assert pick(8, 33_554_432) == (0, 1)             # 64 MiB
    assert pick(8, 134_217_728) == (0, 0)            # 256 MiB
    assert pick(9, 8_388_608) == (3, 0)              # W > 8: chunk tiles
    assert pick(8, 8_388_608, same_phase=0) == (3, 1)  # realigned inputs: always the last arriver
    assert pick(8, 33_554_432, same_phase=0) == (3, 1)
    assert pick(8, 2_097_152, same_phase=0) == (3, 1)
    assert pick(12, 8_388_608, same_phase=0) == (3, 0)
    # unit size of the last arriver's XCD-local units: narrow (64 packs) below 64 Ki packs, medium (256)
    # below 512 Ki, wide (1024) from there; copier workgroups and MR_TILE_WIDE_PAIR always wide
    for n, want in ((1000, 64), (524_287, 64), (524_288, 256), (4_194_303, 256), (4_194_304, 1024)):
        assert _plan(L, 8, n, "bf16", 0, "auto", "auto")["unit1"] == want, n
    assert _plan(L, 8, 1000, "bf16", 0, "last", "wide_pair")["unit1"] == 1024
    assert _plan(L, 8, 16_777_216 + 8, "bf16", 0, "auto", "auto")["unit1"] == 1024
    # the allocation-free entry point only takes the last arriver, in which nothing waits
    for W, n in ((8, 8_388_608), (8, 1000), (12, 8_388_608), (8, 16_777_216)):
        for sync in ("chunk", "grid", "tile"):
            p = _plan(L, W, n, "bf16", 0, sync, "narrow", wait_free=1)
            assert p["sync"] == 3, (W, n, sync, p)
            assert p["xcd"] == (1 if W <= 8 else 0), (W, n, sync, p)


def _pieces(W, splits, es):
    T = sum(splits)
    O = 0
    for E in splits:
        for r in range(W):
            if E:
                yield r, (O * W + r * E) * es, (r * T + O) * es, O * es
        O += E


def test_gather_phase_masks_match_brute_force(L):
    """The planner keeps one 16-bit mask of the pieces' (destination - source) offsets mod 16 for a
    rank-major source (computed over the first 16 ranks: the phase repeats with period 16 in the rank)
    and one per rank for shard sources; a launch takes the realigning kernel build exactly when some
    piece is out of phase for the call's base pointers.  Brute force over every piece."""
    rng = random.Random(21)
    for trial in range(400):
        W = rng.choice([1, 2, 3, 4, 6, 8, 16, 17, 24, 32, 64])
        G = rng.choice([d for d in range(1, W + 1) if W % d == 0])
        dt = rng.choice(["bf16", "fp16", "fp32", "int32"])
        es = 2 if dt in ("bf16", "fp16") else 4
        P = rng.randint(1, 12)
        splits = [rng.choice([0, 1, 2, 3, 7, 8, 9, 16, 24, 31, 1000, 1023, 4096]) for _ in range(P)]
        if sum(splits) == 0:
            splits[0] = 5
        sp = (ctypes.c_uint64 * P)(*splits)
        rm = ctypes.c_uint16(0)
        rk = (ctypes.c_uint16 * 64)()
        assert L.mrx_gather_phase_masks(W, G, sp, P, mr.DTYPE_CODE[dt], ctypes.byref(rm), rk, 64) == 0
        want_rm, want_rk = 0, [0] * W
        for r, dst, src_rm, src_sh in _pieces(W, splits, es):
            want_rm |= 1 << ((dst - src_rm) % 16)
            want_rk[r] |= 1 << ((dst - src_sh) % 16)
        assert rm.value == want_rm, (trial, W, splits, dt)
        assert [rk[r] for r in range(min(W, 64))] == want_rk[:64]
        for d in range(16):  # base difference src - out, mod 16
            brute = any((dst - src_rm - d) % 16 != 0 for _, dst, src_rm, _ in _pieces(W, splits, es))
            assert L.mrx_needs_realign(rm.value, d) == int(brute), (trial, d)


def _tile_param(prefix, P, t):
    """The param-contiguous kernel's tile -> parameter search: the last s with prefix[s] <= t."""
    lo, hi = 0, P
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if prefix[mid] <= t:
            lo = mid
        else:
            hi = mid
    return lo


def test_sdma_gather_kernel_part_covers_exactly_the_small_parameters(L):
    """The SDMA gather's compute-unit part plans the whole split table but gives tiles only to parameters
    whose per-rank piece is below the threshold.  Each such parameter keeps the tile count of the full
    plan, every other parameter gets none, the kernel's tile search sends every tile to a kept parameter
    and each kept parameter receives exactly its own tiles, and the phase mask covers the kept pieces
    only (brute force)."""
    rng = random.Random(33)
    UMAX = 2 ** 64 - 1
    for trial in range(300):
        W = rng.choice([1, 2, 4, 6, 8, 16])
        G = rng.choice([d for d in range(1, W + 1) if W % d == 0])
        dt = rng.choice(["bf16", "fp16", "fp32", "int32"])
        es = 2 if dt in ("bf16", "fp16") else 4
        P = rng.randint(2, 128)
        splits = [rng.choice([0, 1, 7, 8, 9, 1000, 4095, 4096, 4097, 20_000, 131_071, 131_072, 600_000])
                  for _ in range(P)]
        if sum(splits) == 0:
            splits[-1] = 9
        cu_below = rng.choice([0, 1, 2, 8192, 8190, 262_144, 262_142, 10 ** 6, UMAX])
        sp = (ctypes.c_uint64 * P)(*splits)
        full, cut = (ctypes.c_uint32 * (P + 1))(), (ctypes.c_uint32 * (P + 1))()
        m_full, m_cut = ctypes.c_uint16(0), ctypes.c_uint16(0)
        assert L.mrx_gather_tiles(W, G, sp, P, mr.DTYPE_CODE[dt], UMAX, full, P + 1, ctypes.byref(m_full)) == 0
        assert L.mrx_gather_tiles(W, G, sp, P, mr.DTYPE_CODE[dt], cu_below, cut, P + 1, ctypes.byref(m_cut)) == 0
        kept = [E * es < cu_below for E in splits]
        for s_ in range(P):
            n_full, n_cut = full[s_ + 1] - full[s_], cut[s_ + 1] - cut[s_]
            assert n_cut == (n_full if kept[s_] else 0), (trial, s_, splits[s_], cu_below)
        got = [0] * P
        for t in range(cut[P]):
            s_ = _tile_param(cut, P, t)
            assert kept[s_] and cut[s_] <= t < cut[s_ + 1], (trial, t)
            got[s_] += 1
        assert got == [cut[i + 1] - cut[i] for i in range(P)]
        want, O, T = 0, 0, sum(splits)
        for s_, E in enumerate(splits):
            if E and kept[s_]:
                for r in range(min(W, 16)):  # the phase repeats with period 16 in the rank
                    want |= 1 << (((O * W + r * E) - (r * T + O)) * es % 16)
            O += E
        assert m_cut.value == want, (trial, splits, cu_below)
    tiny = (ctypes.c_uint32 * 2)()
    m = ctypes.c_uint16(0)
    assert L.mrx_gather_tiles(8, 4, (ctypes.c_uint64 * 1)(5), 1, 0, UMAX, tiny, 1, ctypes.byref(m)) == -1
