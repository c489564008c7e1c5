"""The workgroup -> tile map is a bijection for every grid (CPU build of the
same header the kernels include) and groups each XCD's tiles together."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_optimisation_amd", "csrc")

SHIM = r'''
#include "tile_schedule.hpp"
extern "C" void map_all(int64_t tm, int64_t tn, int64_t batch, int gm, int xcds, int64_t *out) {
    libgemm::TileGrid g{tm, tn, batch, gm, xcds};
    for (int64_t w = 0; w < g.count(); ++w) {
        libgemm::TileCoord t = libgemm::tile_of(g, w);
        out[3 * w] = t.batch; out[3 * w + 1] = t.tm; out[3 * w + 2] = t.tn;
    }
}
extern "C" int64_t remap(int64_t w, int64_t total, int xcds) { return libgemm::xcd_remap(w, total, xcds); }
'''


@pytest.fixture(scope="module")
def sched(tmp_path_factory):
    d = tmp_path_factory.mktemp("sched")
    src = d / "shim.cpp"
    src.write_text(SHIM)
    lib = d / "libshim.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, str(src), "-o",
                    str(lib)], check=True)
    L = ctypes.CDLL(str(lib))
    L.map_all.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.remap.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    L.remap.restype = ctypes.c_int64

    def run(tm, tn, batch, gm, xcds):
        out = np.empty((tm * tn * batch, 3), np.int64)
        L.map_all(tm, tn, batch, gm, xcds, out.ctypes.data)
        return out
    run.remap = L.remap
    return run


def assert_bijection(m, tm, tn, batch):
    assert m.shape[0] == tm * tn * batch
    assert (m[:, 0] >= 0).all() and (m[:, 0] < batch).all()
    assert (m[:, 1] >= 0).all() and (m[:, 1] < tm).all()
    assert (m[:, 2] >= 0).all() and (m[:, 2] < tn).all()
    flat = (m[:, 0] * tm + m[:, 1]) * tn + m[:, 2]
    assert np.unique(flat).size == flat.size


def test_bijection_all_small_grids(sched):
    for tm in range(1, 25):
        for tn in range(1, 25):
            for gm in (1, 3, 4, 8):
                for xcds in (1, 8):
                    assert_bijection(sched(tm, tn, 1, gm, xcds), tm, tn, 1)


@pytest.mark.parametrize("grid", [
    (16, 16, 1), (32, 32, 1), (16, 48, 1), (16, 64, 1), (32, 33, 1), (16, 17, 1), (1, 16, 1),
    (8, 8, 32), (8, 1, 32), (3, 5, 7), (1, 1, 1), (1, 1, 9)])
@pytest.mark.parametrize("gm", [1, 4, 8])
def test_bijection_workload_grids(sched, grid, gm):
    tm, tn, batch = grid
    assert_bijection(sched(tm, tn, batch, gm, 8), tm, tn, batch)


def test_xcd_remap_gives_each_xcd_a_contiguous_range(sched):
    for total in (1, 7, 8, 9, 255, 256, 257, 1056, 2048):
        logical = np.array([sched.remap(w, total, 8) for w in range(total)])
        assert np.array_equal(np.sort(logical), np.arange(total))
        for x in range(8):
            ids = np.sort(logical[np.arange(total) % 8 == x])
            if ids.size:
                assert np.array_equal(ids, np.arange(ids[0], ids[0] + ids.size))


def test_group_rasterisation_order(sched):
    # without the XCD remap, consecutive workgroups walk down a group of 4
    # tile rows before moving to the next column
    m = sched(8, 5, 1, 4, 1)
    assert m[:8, 1].tolist() == [0, 1, 2, 3, 0, 1, 2, 3]
    assert m[:8, 2].tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    # the last group (rows 4..7) follows once the first is done
    assert m[20, 1] == 4 and m[20, 2] == 0
