"""Host-side checks of the profiling summaries: the labelling of a benchmark
run's dispatches, which every per-kernel counter table rests on."""
import pytest

from fp4_fully_quantized_amd import profiling as p


def _names(steps, warmup):
    # Kernel short names as a benchmark run launches them (GEMMs included),
    # written out independently of the tables under test.
    step = ["k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_gemm<0, 256, true>",
            "k_amax<true, false>", "k_quant_dual<0, 1, 1, true, false, false, false>",
            "k_gemm<0, 256, false>", "k_gemm<0, 256, false>",
            "k_quant_cols<1, 0, true, true, false>", "k_quant_cols<1, 0, true, true, false>",
            "k_gemm<1, 256, true>"]
    extras = ["k_amax_rot_rows<true>", "k_amax_pair<true, false, true>",
              "k_quant_dual<0, 0, 1, true, false, true, false>", "k_amax_pair<true, false, true>",
              "k_quant_dual<0, 1, 1, true, false, true, false>", "k_amax<true, false>",
              "k_quant_2d<0, 0, true>", "k_amax<true, false>",
              "k_quant_dual_w3<0, 1, 1, true, false, false, true>"]
    cold = [n for n in step if not n.startswith("k_gemm")]
    return step * (warmup + steps) + extras * (2 + steps) + cold * (2 + steps)


def test_label_dispatches_accepts_a_benchmark_run():
    labels = p.label_dispatches(_names(1, 1), 1, 1)
    assert len(labels) == 2 * 12 + 3 * 9 + 3 * 8
    assert labels[0][0] == "amax X" and labels[4][0].startswith("NVFP4 GEMM fwd")
    assert labels[-1][0] == "MXFP4+Hadamard W (cold)"
    # algorithmic bytes: dual pass over X reads bf16 once, writes two orientations
    x_dual = [u for l, u, _ in labels if l.startswith("dual X (RTN")][0]
    assert x_dual == 32768 * 4096 * (2 + 2 * (0.5 + 1 / 16))
    # element-orientation counts: 2 for dual passes, 1 for amax and MXFP4 passes, 0 for GEMMs
    d = {l: e for l, _, e in labels}
    assert d["dual dY (SR both)"] == 2 * 32768 * 11008
    assert d["amax W"] == 11008 * 4096 and d["MXFP4+Hadamard X"] == 32768 * 4096
    assert d["NVFP4 GEMM wgrad (fp32 out)"] == 0


def test_label_dispatches_rejects_a_changed_run():
    names = _names(1, 1)
    with pytest.raises(ValueError):
        p.label_dispatches(names[:-1], 1, 1)
    swapped = list(names)
    swapped[0], swapped[1] = swapped[1], swapped[0]
    with pytest.raises(ValueError):
        p.label_dispatches(swapped, 1, 1)
