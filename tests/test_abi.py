"""Host-side checks of the C ABI: the library loads, exports what include/mr.h declares, and every
argument error returns its code before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import all_gather_amd as mr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mr.h")

OK, EINVAL, EDTYPE, EALIAS, EWS = 0, -1, -2, -3, -4


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mr_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mr.LIB_PATH):
        pytest.fail("libmr.so is not built; run __graft_entry__.build() first")
    return mr.lib()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(mr.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", mr.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mr_[a-z_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_version_and_status_strings(L):
    assert L.mr_version() == 105
    for code, name in mr.STATUS.items():
        assert L.mr_status_string(code).decode().startswith(name)
    assert b"unknown" in L.mr_status_string(-99)
    assert L.mr_last_hip_error() == 0


def _ptrs(*vals):
    return (ctypes.c_void_p * max(len(vals), 1))(*vals)


@pytest.mark.parametrize("W", [0, -1, 17, 1000])
def test_allreduce_rejects_bad_W(L, W):
    assert L.mr_allreduce_sum(_ptrs(0x1000), W, 16, 0, 0x9000, 0, None) == EINVAL


def test_allreduce_argument_errors(L):
    p = _ptrs(0x10000, 0x20000)
    assert L.mr_allreduce_sum(p, 2, 16, 3, 0x90000, 0, None) == EDTYPE          # int32 is not reduced
    assert L.mr_allreduce_sum(p, 2, 16, 7, 0x90000, 0, None) == EINVAL          # unknown dtype
    assert L.mr_allreduce_sum(p, 2, 16, 0, 0x90000, 2, None) == EINVAL          # unknown mode
    assert L.mr_allreduce_sum(None, 2, 16, 0, 0x90000, 0, None) == EINVAL       # no buffer array
    assert L.mr_allreduce_sum(p, 2, 16, 0, None, 0, None) == EINVAL             # no out
    assert L.mr_allreduce_sum(_ptrs(0x10000, None), 2, 16, 0, 0x90000, 0, None) == EINVAL
    assert L.mr_allreduce_sum(p, 2, 2 ** 63, 0, 0x90000, 0, None) == EINVAL     # size overflow
    # n == 0 is a no-op that enqueues nothing (null pointers allowed)
    assert L.mr_allreduce_sum(None, 2, 0, 0, None, 0, None) == OK
    assert L.mr_allreduce_sum(None, 2, 0, 0, None, 1, None) == OK


def test_allreduce_alias_rules(L):
    n, es = 64, 2
    a, b = 0x100000, 0x200000
    # out overlapping an input without being equal to it
    assert L.mr_allreduce_sum(_ptrs(a, b), 2, n, 0, a + 2, 0, None) == EALIAS
    assert L.mr_allreduce_sum(_ptrs(a, b), 2, n, 0, b - es, 1, None) == EALIAS
    assert L.mr_allreduce_sum(_ptrs(a, b), 2, n, 0, a - n * es + es, 0, None) == EALIAS
    # fp32 elements are 4 bytes: an out 64 bytes past b still overlaps 64 fp32 elements of b
    assert L.mr_allreduce_sum(_ptrs(a, b), 2, n, 2, b + 64, 0, None) == EALIAS


def test_gather_argument_errors(L):
    sp = (ctypes.c_uint64 * 3)(8, 16, 24)
    src, out = 0x100000, 0x800000
    assert L.mr_allgather_param_contig(src, 8, 3, sp, 3, 0, out, None) == EINVAL    # G does not divide W
    assert L.mr_allgather_param_contig(src, 8, 0, sp, 3, 0, out, None) == EINVAL
    assert L.mr_allgather_param_contig(src, 0, 1, sp, 3, 0, out, None) == EINVAL
    assert L.mr_allgather_param_contig(src, 70000, 1, sp, 3, 0, out, None) == EINVAL
    assert L.mr_allgather_param_contig(src, 8, 4, sp, 0, 0, out, None) == EINVAL    # no params
    assert L.mr_allgather_param_contig(src, 8, 4, None, 3, 0, out, None) == EINVAL
    assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 9, out, None) == EINVAL    # unknown dtype
    assert L.mr_allgather_param_contig(None, 8, 4, sp, 3, 0, out, None) == EINVAL
    assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 0, None, None) == EINVAL
    huge = (ctypes.c_uint64 * 2)(2 ** 62, 2 ** 62)
    assert L.mr_allgather_param_contig(src, 8, 4, huge, 2, 0, out, None) == EINVAL  # size overflow
    zero = (ctypes.c_uint64 * 2)(0, 0)
    assert L.mr_allgather_param_contig(None, 8, 4, zero, 2, 0, None, None) == OK     # empty: no-op
    # overlap of src and out (W*T*s = 8*48*2 = 768 bytes)
    assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 0, src + 766, None) == EALIAS
    assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 0, src - 766, None) == EALIAS


def test_noalloc_reduce_argument_errors(L):
    """The no-allocation reduce validates like mr_allreduce_sum and refuses rank buffers over its limit
    before any HIP call."""
    f = L.mr_allreduce_sum_noalloc
    a, b = 0x1000000, 0x9000000
    assert f(_ptrs(a, b), 0, 16, 0, 0x20000000, 1, None) == EINVAL
    assert f(_ptrs(a, b), 2, 16, 3, 0x20000000, 1, None) == EDTYPE
    assert f(_ptrs(a, b), 2, 16, 0, 0x20000000, 7, None) == EINVAL
    assert f(None, 2, 0, 0, None, 1, None) == OK
    limit = mr.NOALLOC_MAX_BYTES
    assert f(_ptrs(a, b), 2, limit // 2 + 1, 0, 0x40000000, 1, None) == EWS     # bf16, one element over
    assert f(_ptrs(a, b), 2, limit // 4 + 1, 2, 0x40000000, 0, None) == EWS     # fp32, one-shot too


def test_sdma_gather_argument_errors(L):
    """The copy-engine gather validates exactly like the kernel gather, before touching the stream."""
    sp = (ctypes.c_uint64 * 3)(8, 16, 24)
    src, out = 0x100000, 0x800000
    f = L.mr_allgather_param_contig_sdma
    assert f(src, 8, 3, sp, 3, 0, out, None) == EINVAL    # G does not divide W
    assert f(src, 0, 1, sp, 3, 0, out, None) == EINVAL
    assert f(src, 8, 4, sp, 0, 0, out, None) == EINVAL    # no params
    assert f(src, 8, 4, None, 3, 0, out, None) == EINVAL
    assert f(src, 8, 4, sp, 3, 9, out, None) == EINVAL    # unknown dtype
    assert f(None, 8, 4, sp, 3, 0, out, None) == EINVAL
    zero = (ctypes.c_uint64 * 2)(0, 0)
    assert f(None, 8, 4, zero, 2, 0, None, None) == OK     # empty: no-op
    assert f(src, 8, 4, sp, 3, 0, src + 766, None) == EALIAS
    assert L.mr_status_string(-6).decode().startswith("MR_ERR_ENGINE")


def test_workspace_sizes_and_errors(L):
    assert L.mr_workspace_bytes(8, 0, 0) >= 16384
    b = L.mr_workspace_bytes(8, 8_388_608, 0)
    assert 16384 + 8_388_608 * 2 < b < 1.05 * 8_388_608 * 2 + 65536 and b % 256 == 0
    assert L.mr_workspace_bytes(8, 1000, 2) >= 16384 + 4000
    assert L.mr_workspace_bytes(0, 1000, 0) == 0
    assert L.mr_workspace_bytes(8, 1000, 3) == 0
    assert L.mr_set_workspace(None, 0x100010, 1 << 20) == EINVAL      # not 256-byte aligned
    assert L.mr_set_workspace(None, 0x100000, 16) == EINVAL           # smaller than the barrier words
    assert L.mr_set_workspace(None, 0x100000, 16384) == EINVAL        # no room for flags and stage
    assert L.mr_workspace_check(None, None) == EINVAL


@pytest.mark.parametrize("es,dt", [(2, 0), (4, 2)])
def test_workspace_rule_covers_every_two_shot_plan(L, es, dt):
    # layout: 16 KiB of barrier words, then bytes/256 u32 flags (rounded to 256 B), then the stage.
    # The largest plan for n elements is the element-wise one: W chunks of ceil(n/W) elements in tiles
    # of 256, one flag per tile.
    for n in [1, 255, 256, 257, 4097, 65_536, 1_000_003, 10_000_019, 123_456_789]:
        for W in (1, 3, 8, 16):
            b = L.mr_workspace_bytes(W, n, dt)
            flags_cap = b >> 8
            stage_off = 16384 + ((flags_cap * 4 + 255) // 256) * 256
            tiles = -(-(-(-n // W)) // 256)
            assert W * tiles <= flags_cap, (n, W)
            assert stage_off + n * es + 256 <= b, (n, W)


def test_options_validate_and_round_trip(L):
    v = ctypes.c_int64(-7)
    assert L.mr_get_option(0, ctypes.byref(v)) == OK and v.value == 4          # size-chosen hand-off
    assert L.mr_get_option(1, ctypes.byref(v)) == OK and v.value == 1 << 22
    assert L.mr_set_option(0, 5) == EINVAL and L.mr_set_option(0, -1) == EINVAL
    assert L.mr_set_option(1, -1) == EINVAL and L.mr_set_option(1, 2 ** 32) == EINVAL
    assert L.mr_set_option(9, 0) == EINVAL and L.mr_get_option(9, ctypes.byref(v)) == EINVAL
    assert L.mr_get_option(0, None) == EINVAL
    for sync in ("chunk", "grid", "last", "tile", "auto"):
        mr.set_option("twoshot_sync", sync)
        assert mr.get_option("twoshot_sync") == sync
    mr.set_option("spin_limit", 1000)
    assert mr.get_option("spin_limit") == 1000
    mr.set_option("spin_limit", 1 << 22)
    assert L.mr_get_option(2, ctypes.byref(v)) == OK and v.value == 0          # tile shape: auto
    assert L.mr_set_option(2, 5) == EINVAL and L.mr_set_option(2, -1) == EINVAL
    for shape in ("wide", "medium", "narrow", "wide_pair", "auto"):
        mr.set_option("tile_shape", shape)
        assert mr.get_option("tile_shape") == shape
    assert L.mr_get_option(3, ctypes.byref(v)) == OK and v.value == 1 << 20  # SDMA gather: small pieces on CUs
    assert L.mr_set_option(3, -1) == EINVAL and L.mr_set_option(3, 2 ** 32) == EINVAL
    for b in (0, 2 ** 32 - 1, 1 << 20):
        mr.set_option("sdma_cu_below", b)
        assert mr.get_option("sdma_cu_below") == b


def test_environment_sets_initial_options(tmp_path):
    """MR_TWOSHOT_SYNC, MR_SPIN_LIMIT, MR_TILE_SHAPE and MR_SDMA_CU_BELOW give the options' values when the
    library loads (in a fresh process; malformed values fall back to the defaults)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import all_gather_amd as mr; "
            "print(mr.get_option('twoshot_sync'), mr.get_option('spin_limit'), mr.get_option('tile_shape'), "
            "mr.get_option('sdma_cu_below'))"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    env = dict(os.environ, MR_TWOSHOT_SYNC="2", MR_SPIN_LIMIT="77", MR_TILE_SHAPE="3", MR_SDMA_CU_BELOW="0")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["grid", "77", "narrow", "0"]
    for bad in (dict(MR_TWOSHOT_SYNC="x", MR_SPIN_LIMIT="", MR_TILE_SHAPE="3z", MR_SDMA_CU_BELOW="1k"),
                dict(MR_TWOSHOT_SYNC="9", MR_SPIN_LIMIT="-1", MR_TILE_SHAPE="5", MR_SDMA_CU_BELOW="-1"),
                dict(MR_TWOSHOT_SYNC="-2", MR_SPIN_LIMIT="4294967296", MR_TILE_SHAPE="0x10",
                     MR_SDMA_CU_BELOW="4294967296")):
        out = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, **bad), capture_output=True,
                             text=True, timeout=120)
        assert out.returncode == 0, out.stderr
        assert out.stdout.split() == ["auto", str(1 << 22), "auto", str(1 << 20)], bad


def test_binding_rejects_host_tensors():
    import torch

    x = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mr.allreduce_sum([x, x], torch.zeros_like(x))
    with pytest.raises(ValueError):
        mr.allgather_param_contig(x, 2, 1, [4], torch.zeros_like(x))


def test_product_path_does_not_import_the_oracle():
    # the package and its sources never reference the oracle or the workloads module
    pkg = os.path.join(ROOT, "all_gather_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "workloads" not in txt, f


def test_header_is_plain_c_and_links(tmp_path):
    """include/mr.h compiles as C99 with no HIP headers, and a C program links libmr.so and gets the
    documented error codes."""
    exe = tmp_path / "c_abi_check"
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    libdir = os.path.dirname(mr.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), src,
           "-L", libdir, "-lmr", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr


def test_reduce_scatter_chunk_matches_the_oracle_definition(L):
    import oracle

    off, cnt = ctypes.c_size_t(), ctypes.c_size_t()
    for dt, name in ((0, "bf16"), (1, "fp16"), (2, "fp32")):
        for n in (0, 1, 7, 8, 9, 63, 64, 65, 1000, 8_388_608, 8_388_611, 123_457):
            for W in (1, 2, 3, 8, 16):
                for rank in range(W):
                    assert L.mr_reduce_scatter_chunk(n, W, dt, rank, ctypes.byref(off), ctypes.byref(cnt)) == OK
                    a, b = oracle.reduce_scatter_chunk(n, W, name, rank)
                    assert (off.value, cnt.value) == (a, b - a), (name, n, W, rank)


def test_reduce_scatter_argument_errors(L):
    off, cnt = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.mr_reduce_scatter_chunk(100, 4, 0, 4, ctypes.byref(off), ctypes.byref(cnt)) == EINVAL
    assert L.mr_reduce_scatter_chunk(100, 4, 0, -1, ctypes.byref(off), ctypes.byref(cnt)) == EINVAL
    assert L.mr_reduce_scatter_chunk(100, 4, 3, 0, ctypes.byref(off), ctypes.byref(cnt)) == EDTYPE
    assert L.mr_reduce_scatter_chunk(100, 17, 0, 0, ctypes.byref(off), ctypes.byref(cnt)) == EINVAL
    assert L.mr_reduce_scatter_chunk(100, 4, 0, 0, None, ctypes.byref(cnt)) == EINVAL
    p = _ptrs(0x100000, 0x200000)
    assert L.mr_reduce_scatter_sum(p, 2, 64, 0, 2, 0x900000, None) == EINVAL
    assert L.mr_reduce_scatter_sum(p, 2, 64, 3, 0, 0x900000, None) == EDTYPE
    assert L.mr_reduce_scatter_sum(None, 2, 64, 0, 0, 0x900000, None) == EINVAL
    # rank 1's chunk of 64 bf16 is elements [32, 64): out 2 bytes into it overlaps without being equal
    assert L.mr_reduce_scatter_sum(p, 2, 64, 0, 1, 0x100000 + 66, None) == EALIAS
    assert L.mr_reduce_scatter_sum(p, 2, 0, 0, 1, None, None) == OK     # empty chunk: no-op
    assert L.mr_reduce_scatter_sum(p, 16, 8, 0, 15, None, None) == OK   # a trailing empty chunk


def test_cached_gather_plans_keep_validation_and_alias_checks(L):
    """Plans are cached per (W, G, P, dtype, splits); a cached plan must not let a call skip the checks
    that depend on the call's own arguments (pointers) or on any key field, and more distinct split
    sets than cache slots must keep working."""
    src, out = 0x100000, 0x800000
    for rep in range(2):  # miss, then hit
        for k in range(12):
            sp = (ctypes.c_uint64 * 3)(8 + k, 16, 24)
            T = 48 + k
            assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 0, None, None) == EINVAL, (rep, k)
            assert L.mr_allgather_param_contig(None, 8, 4, sp, 3, 0, out, None) == EINVAL, (rep, k)
            assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 0, src + 8 * T * 2 - 2, None) == EALIAS
            assert L.mr_allgather_param_contig(src, 8, 3, sp, 3, 0, out, None) == EINVAL   # G differs
            assert L.mr_allgather_param_contig(src, 8, 4, sp, 3, 9, out, None) == EINVAL   # dtype differs
            assert L.mr_allgather_param_contig(src, 8, 4, sp, 2, 0, src + 8 * 24 * 2 - 2, None) == EALIAS
    huge = (ctypes.c_uint64 * 3)(8, 2 ** 62, 2 ** 62)
    assert L.mr_allgather_param_contig(src, 8, 4, huge, 3, 0, out, None) == EINVAL     # never cached
    assert L.mr_allgather_param_contig(src, 8, 4, huge, 3, 0, out, None) == EINVAL


def test_shard_gather_argument_errors(L):
    sh = _ptrs(0x100000, 0x200000, 0x300000, 0x400000)
    outs = _ptrs(0x1100000, 0x1200000, 0x1300000, 0x1400000)
    sp = (ctypes.c_uint64 * 2)(8, 24)
    big = _ptrs(*[0x100000 * (i + 1) for i in range(65)])
    assert L.mr_allgather_into_tensor(big, 65, 32, 0, 0x9000000, None) == EINVAL          # over the table size
    assert L.mr_allgather_into_tensor(sh, 4, 32, 5, 0x9000000, None) == EINVAL             # unknown dtype
    assert L.mr_allgather_into_tensor(_ptrs(0x100000, None, 0x300000, 0x400000), 4, 32, 0, 0x9000000, None) == EINVAL
    assert L.mr_allgather_into_tensor(sh, 4, 32, 0, 0x300000 + 2, None) == EALIAS          # out over a shard
    assert L.mr_allgather_into_tensor(None, 4, 0, 0, None, None) == OK                      # T == 0
    assert L.mr_allgather_list(sh, 4, 32, 3, _ptrs(0x1100000, 0x1100000 + 64, 0x1300000, 0x1400000), None) == EALIAS
    assert L.mr_allgather_list(sh, 4, 32, 2, _ptrs(0x1100000, 0x200000 + 4, 0x1300000, 0x1400000), None) == EALIAS
    assert L.mr_allgather_list(sh, 4, 32, 2, None, None) == EINVAL
    assert L.mr_allgather_param_contig_shards(sh, 4, 3, sp, 2, 0, 0x9000000, None) == EINVAL  # G does not divide W
    assert L.mr_allgather_param_contig_shards(sh, 4, 2, sp, 0, 0, 0x9000000, None) == EINVAL  # no params
    assert L.mr_allgather_param_contig_shards(sh, 4, 2, sp, 2, 0, 0x400000 - 10, None) == EALIAS
    assert outs is not None


def test_any_alignment_is_accepted(L):
    """Pointers off the element grid are valid arguments: the reduce plans them on its byte-access path
    (the layout read through the library's planning hook; no launch here) and the gathers plan in bytes.
    Only null pointers, sizes and overlaps are refused."""
    L.mrx_reduce_shape.restype = ctypes.c_int
    L.mrx_reduce_shape.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int]
    f = (ctypes.c_uint64 * 21)()
    a, b, out = 0x100000, 0x200000, 0x900000

    def shape(ptrs, dt, o, n=64):
        assert L.mrx_reduce_shape(_ptrs(*ptrs), len(ptrs), n, dt, o, f, 21) == 0
        return {"vec": f[0], "realign": f[1], "bytes": f[2], "head": f[3], "npacks": f[4],
                "shift": [f[5 + r] for r in range(len(ptrs))]}

    assert shape((a, b), 0, out) == {"vec": 1, "realign": 0, "bytes": 0, "head": 0, "npacks": 8, "shift": [0, 0]}
    s = shape((a + 2, b + 6), 0, out + 2)           # bf16, element-aligned, two phases: realigned packs
    assert (s["vec"], s["realign"], s["bytes"], s["head"], s["shift"]) == (1, 1, 0, 7, [0, 4])
    assert shape((a + 1, b), 0, out)["bytes"] == 1  # bf16 buffer at an odd byte: byte accesses
    assert shape((a, b), 0, out + 1)["bytes"] == 1
    assert shape((a, b + 2), 2, out)["bytes"] == 1  # fp32 buffer 2 bytes in
    s = shape((a + 4, b + 12), 2, out + 8)          # fp32 on its grid, three phases
    assert (s["realign"], s["bytes"], s["shift"]) == (1, 0, [12, 4])
    # argument errors are still the documented ones
    assert L.mr_allreduce_sum(_ptrs(a + 1, None), 2, 64, 0, out, 0, None) == EINVAL
    assert L.mr_allreduce_sum(_ptrs(a + 1, b), 2, 64, 0, a + 3, 0, None) == EALIAS


def test_stream_mix_probe_rejects_bad_arguments(L):
    """The measurement probe (mr_probe.h, not mr.h) validates before it enqueues anything."""
    f = L.mrx_stream_mix
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p]
    reads = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    assert f(reads, 0, 0x300000, 4096, 1, None) == -1        # K out of range
    assert f(reads, 9, 0x300000, 4096, 1, None) == -1
    assert f(reads, 2, 0x300000, 4000 + 8, 1, None) == -1    # not a multiple of 16 bytes
    assert f(reads, 2, 0x300008, 4096, 1, None) == -1        # out not 16-byte aligned
    for bad_mode in (-1, 3):
        assert f(reads, 2, 0x300000, 4096, bad_mode, None) == -1
    assert f(reads, 2, 0x300000, 0, 2, None) == 0            # empty: no-op
