"""The benchmark's metric formulas against the numbers printed on the DeepGEMM FP8
block GEMM benchmark post (section 3.2 per-shape tables, section 3.3 averages): the
post's TFLOPS and GB/s columns follow from its printed times with TFLOPS = 2mnk/t and
GB/s = (mk + kn + 2mn)/t (the extracted text dropped the '+' signs)."""
import os

import numpy as np

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def _table():
    rows = []
    for line in open(os.path.join(HERE, "golden", "deepgemm_h100_dense_table.txt")):
        if line.startswith("#") or not line.strip():
            continue
        impl, m, n, k, us, tf, gbs = line.split()
        rows.append((impl, int(m), int(n), int(k), float(us), float(tf), float(gbs)))
    return rows


def test_published_cells_follow_from_the_formulas():
    rows = _table()
    assert len(rows) == 48
    for impl, m, n, k, us, tf, gbs in rows:
        t = us * 1e-6
        assert abs(bench.gemm_flops(m, n, k) / t / 1e12 - tf) <= 0.02 * tf + 0.06, (impl, m, n, k)
        assert abs(bench.gemm_bytes(m, n, k) / t / 1e9 - gbs) <= 0.02 * gbs, (impl, m, n, k)


def test_published_averages():
    rows = _table()
    summ = {}
    for line in open(os.path.join(HERE, "golden", "deepgemm_h100_summary.txt")):
        if line.startswith("#") or not line.strip():
            continue
        impl, tf, gbs, ms, _ = line.split()
        summ[impl] = (float(tf), float(gbs))
    for impl, (tf, gbs) in summ.items():
        sel = [r for r in rows if r[0] == impl]
        assert len(sel) == 16
        assert abs(np.mean([r[5] for r in sel]) - tf) < 0.01 * tf
        assert abs(np.mean([r[6] for r in sel]) - gbs) < 0.01 * gbs


def test_masked_and_quant_byte_formulas():
    # masked: valid rows only, weights of active experts once, bf16 output
    assert bench.masked_bytes(10, 2, 256, 512) == 10 * 512 + 2 * 256 * 512 + 2 * 10 * 256
    assert bench.masked_flops(10, 256, 512) == 2 * 10 * 256 * 512
    # quant: bf16 in, e4m3 out, one 4-byte word per 512 columns per row
    assert bench.quant_bytes(3, 640) == 2 * 3 * 640 + 3 * 640 + 4 * 2 * 3
    assert bench.silu_bytes(5, 2048) == 4 * 2048 * 5 + 2048 * 5 + 4 * 4 * 5
