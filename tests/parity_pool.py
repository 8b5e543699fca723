"""Full-tensor quantizer parity on many host cores: the oracle runs chunk by
chunk (rows, or columns for columnwise copies) in spawned CPU-only worker
processes that read the input and the GPU's outputs from memory-mapped .npy
files, and each chunk is compared byte for byte.  (Spawned, not forked: the
workers never inherit the GPU process's state.)  Test infrastructure only."""

import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np


def workers():
    """Host cores to use: the process's CPU set, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class Store:
    """Arrays handed to the workers as memory-mapped .npy files in a private
    temporary directory (removed by close())."""

    def __init__(self):
        self.dir = tempfile.mkdtemp(prefix="mxq_parity_")

    def put(self, name, arr):
        path = os.path.join(self.dir, name + ".npy")
        np.save(path, np.ascontiguousarray(arr))
        return path

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)


def _load(path):
    return np.load(path, mmap_mode="r")


def _nv_r16(rows_idx, cols_idx, cols_total, seed, stream):
    from oracle.philox import element_r16
    r, c = np.meshgrid(np.asarray(rows_idx, dtype=np.int64), np.asarray(cols_idx, dtype=np.int64),
                       indexing="ij")
    return element_r16(r * cols_total + c, seed, stream, 0)


def _first_diff(a, b):
    idx = np.argwhere(np.asarray(a) != np.asarray(b))
    return None if len(idx) == 0 else (tuple(int(i) for i in idx[0]), int(np.asarray(a)[tuple(idx[0])]),
                                       int(np.asarray(b)[tuple(idx[0])]))


def _task(t):
    """One chunk: run the oracle, compare with the GPU's bytes; returns
    (label, None) or (label, description of the first difference)."""
    from oracle import formats as F, nvfp4 as ON, mxfp8 as OM
    kind, label, a0, a1, p = t
    x = _load(p["x"])
    if kind in ("nv_row", "nv_col"):
        if kind == "nv_row":
            bits = np.asarray(x[a0:a1])
            idx_r, idx_c = np.arange(a0, a1), np.arange(bits.shape[1])
        else:                                          # columns a0..a1 of x, as rows
            bits = np.ascontiguousarray(np.asarray(x[:, a0:a1]).T)
            idx_c, idx_r = np.arange(a0, a1), np.arange(bits.shape[1])
        v = F.bf16_bits_to_f64(bits)
        if p.get("S") is None:                         # per row: the oracle's own S
            S_rows = ON.second_scale(np.abs(v).max(axis=1))
            gS = _load(p["gS"])[a0:a1]
            if not np.array_equal(np.asarray(gS), S_rows):
                return label, ("S", _first_diff(gS, S_rows))
        else:
            S_rows = np.full(v.shape[0], np.float32(p["S"]), dtype=np.float32)
        r16 = None
        if p.get("rnd") == "sr":
            if kind == "nv_row":
                r16 = _nv_r16(idx_r, idx_c, x.shape[1], p["seed"], p["stream"])
            else:                                      # element (r, c) of x: index r * cols + c
                r16 = np.ascontiguousarray(_nv_r16(idx_r, idx_c, x.shape[1], p["seed"], p["stream"]).T)
        rc, rs = ON._rows_1x16(v, S_rows, p.get("rnd", "rne"), r16)
    elif kind in ("nv_tile", "nv_tile_t"):
        if kind == "nv_tile":
            v = F.bf16_bits_to_f64(np.asarray(x[a0:a1]))
        else:                                          # the transposed copy: columns a0..a1 of x, as rows
            v = F.bf16_bits_to_f64(np.ascontiguousarray(np.asarray(x[:, a0:a1]).T))
        rc, rs, _ = ON.quantize_tile16(v, "given", S_given=np.float32(p["S"]))
        gs = _load(p["scales"])[a0 // 16:a1 // 16]
        gc = _load(p["codes"])[a0:a1]
        d = _first_diff(gs, rs) or _first_diff(gc, rc)
        return label, d
    elif kind in ("mx_row", "mx_col", "mx_tile", "mx_tile_t"):
        if kind in ("mx_row", "mx_tile"):
            bits = np.asarray(x[a0:a1])
        else:
            bits = np.ascontiguousarray(np.asarray(x[:, a0:a1]).T)
        v = F.bf16_bits_to_f64(bits)
        if kind in ("mx_row", "mx_col"):
            rc, rs = OM.quantize_rowwise(v)
        else:
            rc, rs = OM.quantize_tile32(v)
            gs = _load(p["scales"])[a0 // 32:a1 // 32]
            gc = _load(p["codes"])[a0:a1]
            return label, _first_diff(gs, rs) or _first_diff(gc, rc)
    else:
        raise ValueError(kind)
    gc = _load(p["codes"])[a0:a1]
    gs = _load(p["scales"])[a0:a1]
    return label, _first_diff(gs, rs) or _first_diff(gc, rc)


def chunks(n, step, align=1):
    step = max(align, (step // align) * align)
    return [(a, min(a + step, n)) for a in range(0, n, step)]


def run(tasks, say=print):
    """Run the chunk tasks on the pool; returns the list of failures.  A worker
    that dies raises (BrokenProcessPool) instead of being replaced."""
    from concurrent.futures import ProcessPoolExecutor, as_completed
    t0 = time.time()
    bad = []
    with ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn")) as ex:
        futs = [ex.submit(_task, t) for t in tasks]
        for done, f in enumerate(as_completed(futs), 1):
            label, diff = f.result()
            if diff is not None:
                bad.append((label, diff))
            if done % max(1, len(tasks) // 10) == 0 or done == len(tasks):
                say(f"parity chunks {done}/{len(tasks)} ({time.time() - t0:.0f} s, {len(bad)} bad)")
    return bad
