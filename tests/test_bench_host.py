"""The measurement harness's host logic (no GPU): the algorithmic byte and FLOP counts the
roofline fractions divide by, and the rule that picks the prefill entry point per shape."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from linear_attention_chunked_gdn_amd import inputs  # noqa: E402


def _shape(lengths, Hk, Hv, io="bf16", init_std=None):
    # tiny tensors of the right shape: only the shapes enter the counts
    return inputs.make_custom(1, lengths, Hk, Hv, io=io, init_std=init_std)


def test_algorithmic_bytes_match_the_formula():
    # T (Hk 2 Dk s + Hv (2 Dv s + 8)) + N Hv Dv Dk 4 (x 2 with an initial state), s = 2 for 16-bit I/O
    x = _shape([100, 28], 2, 4)
    assert bench.algorithmic_bytes(x) == 128 * (2 * 2 * 128 * 2 + 4 * (2 * 128 * 2 + 8)) + 2 * 4 * 128 * 128 * 4
    x = _shape([100, 28], 2, 4, init_std=0.1)
    assert bench.algorithmic_bytes(x) == 128 * (2 * 2 * 128 * 2 + 4 * (2 * 128 * 2 + 8)) + 2 * 2 * 4 * 128 * 128 * 4
    x = _shape([10], 1, 1, io="f32")
    assert bench.algorithmic_bytes(x) == 10 * (2 * 128 * 4 + (2 * 128 * 4 + 8)) + 128 * 128 * 4


def test_headline_counts():
    # the headline workload: 68.68 MB and 8.59 GFLOP of the method's own work
    # (131,072 FLOP per token and head for full 64-token chunks)
    x = inputs.make_workload(1)
    assert bench.algorithmic_bytes(x) == 68_681_728
    assert bench.algorithmic_flops(x) == 4096 * 16 * 131_072
    # a partial chunk counts its own n_c: 6 n_c Dk Dv + 2 n_c^2 Dv per value head, 2 n_c^2 Dk per key head
    y = _shape([70], 1, 2)
    per = lambda n: 2 * (6 * n * 128 * 128 + 2 * n * n * 128) + 2 * n * n * 128  # noqa: E731
    assert bench.algorithmic_flops(y) == per(64) + per(6)


@pytest.mark.parametrize("lengths,Hk,Hv,io,prologue,segments,want", [
    ([4096], 16, 16, "bf16", False, 2, "split"),   # two segments only break even
    ([4096], 16, 64, "bf16", False, 1, "split"),   # 256 chain workgroups: still one round
    ([4096], 16, 80, "bf16", False, 1, "pipe"),    # 320: the one-launch kernel
    ([100, 200], 16, 16, "bf16", False, 1, "split"),   # a packed batch
    ([4096], 4, 4, "bf16", False, 4, "seg"),       # few heads, several segments chosen
    ([4096], 4, 4, "bf16", True, 4, "split"),      # the prologue runs on the split path, not in segments
    ([4096], 4, 4, "f32", False, 4, "pipe"),       # fp32 I/O has the one-launch kernels only
])
def test_choose_path(lengths, Hk, Hv, io, prologue, segments, want):
    x = _shape(lengths, Hk, Hv, io=io)
    assert bench.choose_path(x, "auto", prologue, segments) == want
    assert bench.choose_path(x, "pipe", prologue, segments) == "pipe"


def test_headline_traffic_record_matches_the_kernel_sources():
    # bench.py reports roofline.traffic from profiles/hbm_traffic.json only while the
    # sources it was measured on are unchanged: a kernel edit needs the counters retaken
    # (or, for an edit that leaves the code as it was, the record re-keyed from them)
    rec = bench.recorded_traffic("gdn_map_kernel+kda_chain_kernel", "prefill_bf16_H16_T4096")
    assert rec is not None, "profiles/hbm_traffic.json has no current record for the headline's kernels"
    assert 2 * bench.algorithmic_bytes(inputs.make_workload(1)) < rec < 4 * bench.algorithmic_bytes(inputs.make_workload(1))
