"""The C ABI library on the CPU: it loads, exports what include/armx.h
declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

import arithmetic_reduction_matrix_amd as armx

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "armx.h")


PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "armx_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(armx.LIB_PATH), "libarmx_probe.so")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for f in ("reduce_sum", "reduce_rows", "reduce_sum_fixed_order", "reduce_rows_fixed_order",
              "reduce_sum_exact", "armx_workspace_bytes", "armx_status_string", "armx_version",
              "armx_launch_plan", "reduce_sum_noalloc"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(armx.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert armx.lib.armx_version() == 8
    for st in range(0, -7, -1):
        s = armx.lib.armx_status_string(st).decode()
        assert s.startswith("ARMX_")
    assert armx.lib.armx_status_string(-99).decode() == "unknown armx status"


def test_launch_plan_reports_the_planned_shape():
    # the 2^28 sum's default persistent grid: 2 wavefronts of R = 8 per
    # compute unit (256 assumed without a device), one launch
    p = armx.launch_plan(armx.OP_SUM, 1 << 28)
    assert (p["grid_blocks"], p["block_threads"], p["chain_r"], p["launches"]) == (256, 128, 8, 1)
    assert p["waves_per_cu"] == 2.0
    assert p["workspace_bytes"] == armx.workspace_bytes(armx.OP_SUM, 1 << 28)
    # the pages' grid: one chain per wavefront
    p = armx.launch_plan(armx.OP_SUM, 1 << 28, one_chain=True, block_threads=256, chain_r=4)
    assert p["grid_blocks"] == (1 << 28) // (512 * 4 * 4) and p["launches"] == 1
    assert armx.launch_plan(armx.OP_SUM, 1 << 20, two_pass=True)["launches"] == 2
    # MMA levels: one launch per level (2^28 / (512 R) values, then / (256 R) ...)
    assert armx.launch_plan(armx.OP_SUM, 1 << 28, mma_levels=True, chain_r=8)["launches"] == 3
    # empty inputs: the zero-fill kernel, or nothing for zero rows
    assert armx.launch_plan(armx.OP_SUM, 0)["launches"] == 1
    assert armx.launch_plan(armx.OP_ROWS, 0, 100)["launches"] == 0
    assert armx.launch_plan(armx.OP_ROWS_FIXED, 10, 0)["launches"] == 1
    # a fixed-order row stream with a poorly filled last round: a second launch
    p = armx.launch_plan(armx.OP_ROWS_FIXED, 2049, 51192)
    assert p["launches"] == 2 and p["workspace_bytes"] > 0
    with pytest.raises(armx.ArmxError):
        armx.launch_plan(armx.OP_SUM, 10, block_threads=96)
    assert armx.lib.armx_launch_plan(0, 10, 0, None, None) == -1


def test_noalloc_argument_errors():
    f = armx.lib.reduce_sum_noalloc
    assert f(None, 10, FAKE, None, None) == -1                           # x NULL
    assert f(FAKE, 10, None, None, None) == -1                           # out NULL
    assert f(FAKE + 2, 10, FAKE, None, None) == -2                       # x misaligned
    assert f(FAKE, 10, FAKE, cfg(block_threads=96), None) == -3
    # a plan whose workspace exceeds the 1 MiB scratch array is refused
    # before anything is enqueued: the one-chain grid of 64-thread blocks at
    # R = 1 has 2^28 / 512 blocks, 4 bytes of block result each
    assert f(FAKE, 1 << 28, FAKE, cfg(one_chain=True, block_threads=64, chain_r=1), None) == -4
    assert armx.workspace_bytes(armx.OP_SUM, 1 << 28, one_chain=True, block_threads=64,
                                chain_r=1) > 1 << 20
    assert armx.workspace_bytes(armx.OP_SUM, 1 << 40) <= 1 << 20   # every default plan fits


def cfg(**kw):
    return ctypes.byref(armx._config(**kw))


FAKE = 1 << 20   # an aligned address; never dereferenced (calls fail first)


@pytest.mark.parametrize("fn", ["reduce_sum", "reduce_sum_fixed_order"])
def test_flat_argument_errors(fn):
    f = getattr(armx.lib, fn)
    ws = 1 << 24
    assert f(None, 10, FAKE, ws, 1 << 20, None, None) == -1          # x NULL
    assert f(FAKE, 10, None, ws, 1 << 20, None, None) == -1          # out NULL
    assert f(FAKE + 2, 10, FAKE, ws, 1 << 20, None, None) == -2      # x misaligned
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(block_threads=96), None) == -3
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(block_threads=2048), None) == -3
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(chain_r=9), None) == -3
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(grid_blocks=-1), None) == -3
    bad_flags = armx.Config(0, 0, 0, 0x100)
    assert f(FAKE, 10, FAKE, ws, 1 << 20, ctypes.byref(bad_flags), None) == -3
    assert f(FAKE, 10, FAKE, None, 0, None, None) == -1              # ws needed
    assert f(FAKE, 10, FAKE, ws + 8, 1 << 20, None, None) == -2      # ws misaligned
    assert f(FAKE, 10, FAKE, ws, 8, None, None) == -4                # ws too small
    assert f(FAKE, (1 << 40) + 1, FAKE, ws, 1 << 30, None, None) == -5


def test_fixed_order_config_rules():
    f = armx.lib.reduce_sum_fixed_order
    ws = 1 << 24
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(block_threads=192), None) == -3   # not 2^k
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(plain=True), None) == -3
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(one_chain=True), None) == -3


def test_exact_argument_errors():
    f = armx.lib.reduce_sum_exact
    ws = 1 << 24
    assert f(None, 10, FAKE, None, ws, 1 << 20, None, None) == -1          # x NULL
    assert f(FAKE, 10, None, None, ws, 1 << 20, None, None) == -1          # out NULL
    assert f(FAKE + 2, 10, FAKE, None, ws, 1 << 20, None, None) == -2      # x misaligned
    assert f(FAKE, 10, FAKE, FAKE + 4, ws, 1 << 20, None, None) == -2      # out_fixed
    for bad in (dict(plain=True), dict(one_chain=True), dict(two_pass=True),
                dict(mma_levels=True), dict(chain_r=9), dict(block_threads=96)):
        assert f(FAKE, 10, FAKE, None, ws, 1 << 20, cfg(**bad), None) == -3, bad
    assert f(FAKE, 10, FAKE, None, None, 0, None, None) == -1              # ws needed
    assert f(FAKE, 10, FAKE, None, ws, 8, None, None) == -4                # ws too small
    assert f(FAKE, (1 << 40) + 1, FAKE, None, ws, 1 << 30, None, None) == -5


def test_exact_workspace_sizes():
    # counter region + 32-byte records per block + 255 group records
    def ws(grid):
        return armx.COUNTER_BYTES + (32 * grid + 255) // 256 * 256 + 8192
    assert armx.workspace_bytes(armx.OP_EXACT, 1 << 28) == ws(256)
    assert armx.workspace_bytes(armx.OP_EXACT, 1 << 28, block_threads=64) == ws(512)
    assert armx.workspace_bytes(armx.OP_EXACT, 1000) == ws(1)
    assert armx.workspace_bytes(armx.OP_EXACT, 0) == 0
    assert armx.workspace_bytes(armx.OP_EXACT, 1 << 28, grid_blocks=3000) == ws(256)
    assert armx.workspace_bytes(armx.OP_EXACT, 1 << 28, chain_r=1, block_threads=64,
                                grid_blocks=3000) == ws(3000)


def test_fixed_to_int():
    import torch
    for v in (0, 1, -1, 2 ** 63, -(2 ** 63), 2 ** 80 + 12345, -(2 ** 80) - 7):
        lo = v & ((1 << 64) - 1)
        lo = lo - (1 << 64) if lo >= 1 << 63 else lo
        hi = v >> 64
        assert armx.fixed_to_int(torch.tensor([lo, hi], dtype=torch.int64)) == v


def test_mma_levels_config_rules():
    f = armx.lib.reduce_sum
    ws = 1 << 24
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(mma_levels=True, plain=True), None) == -3
    assert f(FAKE, 10, FAKE, ws, 1 << 20, cfg(mma_levels=True, two_pass=True), None) == -3
    assert armx.lib.reduce_sum_fixed_order(FAKE, 10, FAKE, ws, 1 << 20,
                                           cfg(mma_levels=True), None) == -3
    assert armx.lib.reduce_rows(FAKE, 4, 96, 96, FAKE, None, 0, cfg(mma_levels=True), None) == -3
    # a second level needs the level buffers
    assert f(FAKE, 1 << 20, FAKE, None, 0, cfg(mma_levels=True), None) == -1
    assert f(FAKE, 1 << 20, FAKE, ws, 256, cfg(mma_levels=True), None) == -4


def test_mma_leaves_config_rules():
    # the MFMA-leaf order belongs to the two fixed-order entry points only
    ws = 1 << 24
    assert armx.lib.reduce_sum(FAKE, 10, FAKE, ws, 1 << 20, cfg(mma_leaves=True), None) == -3
    assert armx.lib.reduce_sum_exact(FAKE, 10, FAKE, None, ws, 1 << 20, cfg(mma_leaves=True),
                                     None) == -3
    assert armx.lib.reduce_rows(FAKE, 4, 96, 96, FAKE, None, 0, cfg(mma_leaves=True), None) == -3
    assert armx.workspace_bytes(armx.OP_FIXED, 1 << 20, mma_leaves=True) == \
        armx.workspace_bytes(armx.OP_FIXED, 1 << 20)
    for cols in (96, 512, 520, 1 << 20):
        assert armx.workspace_bytes(armx.OP_ROWS_FIXED, 4, cols, mma_leaves=True) == \
            armx.workspace_bytes(armx.OP_ROWS_FIXED, 4, cols)
    # the row entry point keeps its other rules with the flag
    assert armx.lib.reduce_rows_fixed_order(FAKE, 4, 96, 96, FAKE, None, 0,
                                            cfg(mma_leaves=True, plain=True), None) == -3
    assert armx.lib.reduce_rows_fixed_order(FAKE, 4, 96, 96, FAKE, None, 0,
                                            cfg(mma_leaves=True, block_threads=192), None) == -3


def test_mma_levels_workspace_sizes():
    # counter region + level-1 values + level-2 values, each rounded to 256 B;
    # nothing when level 1 gives one value (n <= 512 R)
    def r256(v):
        return (v + 255) // 256 * 256
    for n, r in ((1 << 28, 8), (1 << 28, 1), ((1 << 20) + 1, 4), (3000, 1)):
        c1 = -(-n // (512 * r))
        c2 = -(-c1 // (256 * r))
        want = armx.COUNTER_BYTES + r256(4 * c1) + (r256(4 * c2) if c2 > 1 else 0)
        assert armx.workspace_bytes(armx.OP_SUM, n, chain_r=r, mma_levels=True) == want, (n, r)
    assert armx.workspace_bytes(armx.OP_SUM, 4096, chain_r=8, mma_levels=True) == 0
    assert armx.workspace_bytes(armx.OP_SUM, 4097, chain_r=8, mma_levels=True) == armx.COUNTER_BYTES + 256
    # the grid does not change the level buffers
    assert (armx.workspace_bytes(armx.OP_SUM, 1 << 24, mma_levels=True, block_threads=1024)
            == armx.workspace_bytes(armx.OP_SUM, 1 << 24, mma_levels=True, one_chain=True))


def test_rows_argument_errors():
    f = armx.lib.reduce_rows
    assert f(FAKE, 4, 100, 104, None, None, 0, None, None) == -1      # out NULL
    assert f(None, 4, 100, 104, FAKE, None, 0, None, None) == -1      # x NULL
    assert f(FAKE + 2, 4, 100, 104, FAKE, None, 0, None, None) == -2  # misaligned
    assert f(FAKE, 4, 100, 100, FAKE, None, 0, None, None) == -2      # ld % 8
    assert f(FAKE, 4, 100, 96, FAKE, None, 0, None, None) == -5       # ld < cols
    assert f(FAKE, 4, 100, 104, FAKE, None, 0, cfg(one_chain=True), None) == -3
    assert f(FAKE, 4, 100, 104, FAKE, None, 0, cfg(two_pass=True), None) == -3
    # nothing to do: no rows
    assert f(None, 0, 100, 104, None, None, 0, None, None) == 0


@pytest.mark.parametrize("fn", ["reduce_rows", "reduce_rows_fixed_order"])
def test_rows_split_workspace_errors(fn):
    # one row of 2^28 values is split over blocks: with a workspace it must be
    # 256-byte aligned and large enough (checked before anything is enqueued;
    # with ws NULL the call plans no split instead, which this host cannot run)
    f = getattr(armx.lib, fn)
    op = armx.OP_ROWS if fn == "reduce_rows" else armx.OP_ROWS_FIXED
    n = 1 << 28
    need = armx.workspace_bytes(op, 1, n)
    assert need > 0
    ws = 1 << 24
    assert f(FAKE, 1, n, n, FAKE, ws + 4, need, None, None) == -2         # misaligned
    assert f(FAKE, 1, n, n, FAKE, ws, need - 1, None, None) == -4         # too small
    # a pitch is irrelevant to the size: a padded second row needs the same
    assert armx.workspace_bytes(op, 2, n - 8) == armx.workspace_bytes(op, 2, n - 5)


def test_rows_fixed_argument_errors():
    f = armx.lib.reduce_rows_fixed_order
    assert f(FAKE, 4, 100, 104, None, None, 0, None, None) == -1      # out NULL
    assert f(None, 4, 100, 104, FAKE, None, 0, None, None) == -1      # x NULL
    assert f(FAKE + 2, 4, 100, 104, FAKE, None, 0, None, None) == -2  # misaligned
    assert f(FAKE, 4, 100, 100, FAKE, None, 0, None, None) == -2      # ld % 8
    assert f(FAKE, 4, 100, 96, FAKE, None, 0, None, None) == -5       # ld < cols
    assert f(FAKE, 4, 100, 104, FAKE, None, 0, cfg(block_threads=192), None) == -3
    assert f(FAKE, 4, 100, 104, FAKE, None, 0, cfg(plain=True), None) == -3
    assert f(FAKE, 4, 100, 104, FAKE, None, 0, cfg(two_pass=True), None) == -3
    # a row too long for the LDS node logs of one block
    assert f(FAKE, 2, 1 << 30, 1 << 30, FAKE, None, 0, cfg(chain_r=1), None) == -5
    assert f(None, 0, 100, 104, None, None, 0, None, None) == 0
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, 4096, 65536) == 0


def test_workspace_sizes():
    # layout: the counter region (a top counter and 255 group counters, 256
    # bytes apart) + block results (rounded to 256 bytes) + 1024 bytes of
    # group results
    assert armx.COUNTER_BYTES == 256 * 256

    def ws(grid):
        return armx.COUNTER_BYTES + (4 * grid + 255) // 256 * 256 + 1024
    # persistent grid: 256 CUs x 2 waves / 2 waves per block = 256 blocks
    n = 1 << 28
    assert armx.workspace_bytes(armx.OP_SUM, n) == ws(256)
    assert armx.workspace_bytes(armx.OP_SUM, n, block_threads=64) == ws(512)
    # 1024 threads: at least one block per CU; R = 1: 16 waves per CU
    assert armx.workspace_bytes(armx.OP_SUM, n, block_threads=1024) == ws(256)
    assert armx.workspace_bytes(armx.OP_SUM, n, chain_r=1, block_threads=256) == ws(1024)
    # one chain per wavefront: ceil(n / (512 * R * W)) blocks
    assert armx.workspace_bytes(armx.OP_SUM, n, one_chain=True, chain_r=4,
                                block_threads=256) == ws(n // (512 * 16))
    assert armx.workspace_bytes(armx.OP_SUM, 1000) == ws(1)
    assert armx.workspace_bytes(armx.OP_SUM, 0) == 0
    assert armx.workspace_bytes(armx.OP_ROWS, 4096, 65536) == 0
    # few long rows are split over wavefronts of several blocks: the counter
    # region + one partial per wavefront (256 CUs, R = 8: 512 wavefronts, so
    # one row of 2^28 values in 512 parts); the pitch does not matter, so a
    # ragged width is accepted by the query
    assert armx.workspace_bytes(armx.OP_ROWS, 1, 1 << 28) == armx.COUNTER_BYTES + 4 * 512
    assert armx.workspace_bytes(armx.OP_ROWS_FIXED, 1, 1 << 28) == armx.COUNTER_BYTES + 4 * 512
    assert armx.workspace_bytes(armx.OP_ROWS, 4, 100_003) > 0
    assert armx.workspace_bytes(armx.OP_ROWS, 3, 4096) == 0   # too short to split
    # fixed order, n = 2^26: 2^17 chunks; 256 CUs x 16/8 waves -> 256 blocks
    # of 2 waves x 256 chunks (1024 threads: still one block per CU, 256
    # blocks of 16 waves x 32 chunks; 64 threads: 512 blocks of 256 chunks)
    assert armx.workspace_bytes(armx.OP_FIXED, 1 << 26) == ws(256)
    assert armx.workspace_bytes(armx.OP_FIXED, 1 << 26, block_threads=1024) == ws(256)
    assert armx.workspace_bytes(armx.OP_FIXED, 1 << 26, block_threads=64) == ws(512)
    with pytest.raises(armx.ArmxError):
        armx.workspace_bytes(7, 10)
    with pytest.raises(armx.ArmxError):
        armx.workspace_bytes(armx.OP_SUM, 10, chain_r=0, block_threads=100)


def test_python_layer_type_checks():
    import torch
    with pytest.raises(TypeError):
        armx.reduce_sum(torch.zeros(8, dtype=torch.float32))
    with pytest.raises(ValueError):
        armx.reduce_sum(torch.zeros(8, dtype=torch.float16))      # not on a GPU
    with pytest.raises(ValueError):
        armx.reduce_rows(torch.zeros(2, 8, dtype=torch.float16))


def test_probe_library_exports_its_symbols_and_checks_arguments():
    # the read-stream probe (measurement only) rejects bad arguments before
    # any HIP call, so these run without a GPU
    lib = ctypes.CDLL(PROBE_LIB)
    names = _declared_functions(PROBE_HEADER)
    assert names == ["armx_probe_read"]
    f = lib.armx_probe_read
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    f.argtypes = [vp, sz, vp, sz, ci, ci, ci, ci, ci, vp, vp, vp]
    f.restype = ci
    fake, words = 1 << 20, 1 << 20
    assert f(None, 4096, fake, words, 1, 64, 8, 1, 0, None, None, None) == -1
    assert f(fake + 8, 4096, fake, words, 1, 64, 8, 1, 0, None, None, None) == -2
    assert f(fake, 4096, fake, words, 1, 96, 8, 1, 0, None, None, None) == -3
    assert f(fake, 4096, fake, words, 0, 64, 8, 1, 0, None, None, None) == -3
    assert f(fake, 4096, fake, words, 1, 64, 3, 1, 0, None, None, None) == -3
    assert f(fake, 4096 + 512, fake, words, 1, 64, 8, 1, 0, None, None, None) == -5
    assert f(fake, 4096, fake, 63, 1, 64, 8, 1, 0, None, None, None) == -5
    assert f(fake, 4096, fake, words, 1, 64, 8, 1, 3, None, None, None) == -3   # pause
