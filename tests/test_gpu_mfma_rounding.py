"""Characterises how v_mfma_f32_16x16x32_f16 rounds the sum it accumulates
(the kind of black-box probing of a kernel's arithmetic that "Taming Bitwise
Behavior in GPU Kernels with Tensor Core", arXiv 2609.11356, Abstract, applies
to closed libraries; here to our own tile step).  The free-order contract only
needs the result within one unit in the last place of the exact sum, which is
what is asserted; the rounding mode observed is printed.

A 512-value row goes through exactly one MFMA (one chunk), and its column 0
is the only non-zero column, so the row total is that MFMA output: the
following cross-lane adds only add zeros."""
import numpy as np
import pytest

import arithmetic_reduction_matrix_amd as armx

from _parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
CASES = {
    # name: (values placed in lane 0, exact sum, RNE result, truncated result)
    "1+3u": ([1.0, 3 * U], 1 + 3 * U, 1 + 4 * U, 1 + 2 * U),
    "-(1+3u)": ([-1.0, -3 * U], -(1 + 3 * U), -(1 + 4 * U), -(1 + 2 * U)),
    "1+u tie": ([1.0, U], 1 + U, 1.0, 1.0),
    "1+3u tie": ([1.0, U, U, U], 1 + 3 * U, 1 + 4 * U, 1 + 2 * U),
    "1+5u": ([1.0, U, U, U, U, U], 1 + 5 * U, 1 + 4 * U, 1 + 4 * U),
    "2+3u": ([2.0, U, U, U], 2 + 3 * U, 2.0, 2.0),
}


def test_mfma_sum_is_faithful_and_report_mode():
    require_gpu()
    rows = len(CASES)
    x = np.zeros((rows, 512), np.float16)
    for i, (vals, *_rest) in enumerate(CASES.values()):
        x[i, :len(vals)] = vals
    got = armx.reduce_rows(to_dev(x), chain_r=1, block_threads=64).cpu().numpy()
    modes = []
    for i, (name, (vals, exact, rne, rz)) in enumerate(CASES.items()):
        g = float(got[i])
        # faithful: the exact sum, or one of its two binary32 neighbours
        f = np.float32(exact)
        below = float(f) if float(f) <= exact else float(np.nextafter(f, np.float32(-np.inf)))
        above = below if below == exact else float(np.nextafter(np.float32(below),
                                                                np.float32(np.inf)))
        assert g in (below, above), (name, g, below, above)
        modes.append(f"{name}: got {g!r} (RNE {rne!r}, truncated {rz!r})")
    print("\n".join(modes))
