"""Host-side logic of bench.py that needs no GPU: kernel-name families (which
rocprofv3 rows a counter summary attributes to which kernel), the roofline
arithmetic, the measured-peak annotation, and the algorithmic work of a
small workload against a direct count."""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from workloads import make_config  # noqa: E402


@pytest.mark.parametrize("name,family", [
    ("void dsa::(anonymous namespace)::sparse_attn_kernel<576, 512, true, 2, true>(dsa::AttnArgs)",
     "attention"),
    ("void dsa::(anonymous namespace)::indexer_kernel<128, 2, unsigned short, 2>(...)",
     "indexer_cand"),
    ("void dsa::(anonymous namespace)::indexer_kernel<128, 2, unsigned short, 0>(...)", "indexer"),
    ("void dsa::(anonymous namespace)::indexer_rescue_kernel<128, 2, unsigned short>(...)",
     "indexer_rescue"),
    ("void dsa::(anonymous namespace)::indexer_fp8_kernel<2, unsigned short, true, 4, false, true>"
     "(unsigned char const*, ...)", "indexer_fp8_cand"),
    ("void dsa::(anonymous namespace)::indexer_fp8_kernel<2, float, false, 4, false, false>(...)",
     "indexer_fp8"),
    ("void dsa::(anonymous namespace)::indexer_fp8_kernel<2, unsigned short, true, 1, true, false>"
     "(...)", "indexer_fp8"),
    ("void dsa::(anonymous namespace)::indexer_rescue_fp8_kernel<2, unsigned short, true>(...)",
     "indexer_rescue_fp8"),
    ("void dsa::(anonymous namespace)::topk_radix_kernel<8, 4, true>(...)", "topk_cand"),
    ("void dsa::(anonymous namespace)::topk_radix_kernel<4, 4, false>(...)", "topk"),
    ("void dsa::(anonymous namespace)::topk_stream_kernel(...)", "topk"),
    ("void at::native::vectorized_elementwise_kernel<4, ...>", None),
])
def test_kernel_families(name, family):
    assert bench.family_of(name) == family


def test_every_family_source_exists_and_hashes():
    for fam, (src, _) in bench.KERNELS.items():
        assert os.path.exists(os.path.join(bench.CSRC, src)), fam
        assert len(bench.kernel_source_sha(fam)) == 64
    for fams in (bench.CAND_FAMILIES, bench.CAND_FAMILIES_FP8):
        assert all(f in bench.KERNELS for f in fams)


def test_roofline_entry_and_measured_peak():
    e = bench.roofline_entry("k", "mfma", 4.0e12, 2, 4.0, 2500.0, "TFLOP/s", None)
    # 2e12 FLOP per launch over 2 ms = 1000 TFLOP/s
    assert e["achieved"] == pytest.approx(1000.0) and e["frac"] == pytest.approx(0.4)
    assert e["avg_launch_ms"] == 2.0 and e["algorithmic_per_launch"] == 2.0e12
    peaks = {"bf16_mfma_tflops": 1600.0, "fp8_mfma_tflops": 4000.0, "mxfp8_mfma_tflops": 4400.0,
             "hbm_copy_gbs": 6000.0}
    bench.add_measured(e, peaks)
    assert e["measured_peak"] == 1600.0 and e["frac_of_measured"] == pytest.approx(0.625)
    f = bench.roofline_entry("k", "mfma", 2.0e12, 1, 1.0, bench.PEAK_FP8_TFLOPS, "TFLOP/s", None)
    bench.add_measured(f, peaks, mx=True)
    assert f["measured_peak"] == 4400.0
    g = bench.roofline_entry("k", "hbm", 3.0e9, 1, 1.0, bench.PEAK_HBM_GBS, "GB/s", None)
    assert g["achieved"] == pytest.approx(3000.0)
    bench.add_measured(g, peaks)
    assert g["frac_of_measured"] == pytest.approx(0.5)
    h = dict(g)
    bench.add_measured(h, None)  # no probes: nothing added
    assert h == g


def test_workload_counts_match_a_direct_count():
    """Workload 1 (one 256-token document, top-64): indexer pairs, top-K bytes
    and attention FLOP counted row by row."""
    wl = make_config(1)
    T, K = wl.T, wl.topk
    sl = np.arange(1, T + 1)  # causal lengths of one document
    c = bench.workload_counts(wl, sl)
    pairs = int(sl.sum())
    assert c["indexer_flop"] == pytest.approx(2.0 * wl.H_idx * wl.D_idx * pairs)
    # reads: the score rows longer than K, plus each row's start and length;
    # writes: K indices and the length per row
    topk_bytes = 4.0 * sl[sl > K].sum() + 8.0 * T + (4.0 * K + 4.0) * T
    assert c["topk_bytes"] == topk_bytes
    slots = np.minimum(sl, K).sum()
    assert c["attn_flop"] == pytest.approx(2.0 * (wl.D_qk + wl.D_v) * wl.H * slots, rel=1e-9)
