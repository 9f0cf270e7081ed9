"""The segmented prefill (gdn_prefill_seg: the split path's map, the chain run as concurrent
segments from a zero and an identity state, then the fix-up that joins them) on the GPU
vs the fp64 CPU oracle, through the C-ABI.

Same bar as gdn_prefill: 16-bit I/O, error / rms <= 2e-2 beside the stored outputs'
rounding, outputs and final states separately.  Segment counts from 1 to more than a
sequence's chunks (empty segments), ragged tails, empty sequences, GQA, initial states,
strong decay and every chunk size; one segment is bit-identical to gdn_prefill_split.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import check, check_pair, to_device, to_f64
from linear_attention_chunked_gdn_amd import gdn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    gdn.load_library()
    yield


def _args(d):
    return d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"]


def _check_seg(x, K, chunk=64):
    print(f"\n{x.name}: lengths={x.seq_lengths().tolist()[:10]} Hk={x.Hk} Hv={x.Hv} io={x.io} "
          f"chunk={chunk} segments={K}", flush=True)
    d = to_device(x, DEV)
    o, fs = gdn.prefill_seg(*_args(d), chunk_size=chunk, segments=K)
    torch.cuda.synchronize()
    ro, rf = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)
    return d, o, fs


SMALL = [
    # (lengths, Hk, Hv, init_std)
    ([1], 1, 1, None),
    ([64], 2, 2, 0.1),
    ([65], 1, 1, None),
    ([200], 2, 4, 0.1),
    ([0, 130, 1, 64, 77], 1, 2, 0.1),
    ([129, 0], 2, 2, 0.1),
    ([700], 1, 2, 0.2),
    ([300, 45], 1, 8, 0.1),
]


@pytest.mark.parametrize("K", [2, 3, 5])
@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_seg_small_shapes(K, io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    _check_seg(inputs.make_custom(6000 + case, lengths, Hk, Hv, io=io, init_std=init_std,
                                  g_shift=0.5 * (case % 3), name=f"seg_small{case}"), K)


def test_seg_one_segment_is_the_split_path():
    x = inputs.make_custom(6100, [333, 0, 90], 2, 4, io="bf16", init_std=0.2)
    d = to_device(x, DEV)
    o1, f1 = gdn.prefill_seg(*_args(d), segments=1)
    o2, f2 = gdn.prefill_split(*_args(d))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("shift", [2.0, 4.0])
def test_seg_strong_decay(shift):
    _check_seg(inputs.make_custom(6200 + int(shift), [900, 5], 1, 2, io="bf16", g_shift=shift,
                                  init_std=0.5, name=f"seg_decay{shift}"), 4)


def test_seg_weak_decay_long_segments():
    # g near 0: the segments' state maps are far from contractive, the join carries the
    # whole start state through several hundred tokens
    _check_seg(inputs.make_custom(6250, [2048], 1, 2, io="bf16", g_shift=-3.0, init_std=0.3,
                                  name="seg_weak_decay"), 4)


@pytest.mark.parametrize("chunk", [32, 128])
@pytest.mark.parametrize("K", [2, 3])
def test_seg_other_chunk_sizes(chunk, K):
    _check_seg(inputs.make_custom(6300 + chunk + K, [31, 32, 33, 127, 128, 129, 600, 0, 1], 2, 4, io="bf16",
                                  init_std=0.2, g_shift=1.0, name=f"seg_c{chunk}_ragged"), K, chunk)


def test_seg_few_heads_long_sequence():
    # the shape segments are for: few (sequence, head) pairs, many chunks
    x = inputs.make_custom(6400, [8192], 2, 4, io="bf16", name="seg_H4_T8192")
    d, o, fs = _check_seg(x, 4)
    o1, f1 = gdn.prefill_split(*_args(d))
    torch.cuda.synchronize()
    check_pair("seg vs split o", to_f64(o), to_f64(o1), x.io)
    check_pair("seg vs split state", to_f64(fs), to_f64(f1), x.io, stored=False)


def test_seg_benched_shard_H4_T65536():
    # the shape the segmented path is measured on: one GPU's 4-head share of the H32
    # T65536 prefill, at the segment count gdn_prefill_seg_choose picks for it
    x = inputs.head_shard(inputs.make_workload(4), 8)
    K = gdn.prefill_seg_choose(x.N, x.T_tot, x.Hv)
    assert K > 1
    _check_seg(x, K)


@pytest.mark.parametrize("wid,K", [(1, 2), (3, 2), (3, 3)])
def test_seg_workloads(wid, K):
    _check_seg(inputs.make_workload(wid), K)


def test_seg_in_place_state_and_workspace_reuse():
    x = inputs.make_custom(6500, [150, 700], 2, 2, io="f16", init_std=0.2)
    d = to_device(x, DEV)
    ws = torch.empty(gdn.prefill_seg_workspace_size(x.N, x.T_tot, x.Hv, 64, 3), dtype=torch.uint8, device=DEV)
    o_ref, f_ref = gdn.prefill_seg(*_args(d), segments=3, workspace=ws)
    st = d["initial_state"].clone()
    o2, _ = gdn.prefill_seg(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu_seqlens"], segments=3,
                            final_state=st, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o2) and torch.equal(f_ref, st)


def test_seg_empty_batch_keeps_the_state():
    x = inputs.make_custom(6600, [0, 0], 1, 2, io="bf16", init_std=0.3)
    d = to_device(x, DEV)
    o, fs = gdn.prefill_seg(*_args(d), segments=4)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(fs.cpu(), torch.from_numpy(x.initial_state))


def test_seg_choose():
    # one recurrence workgroup per compute unit: N Hv 4 (2K - 1) <= CUs (4 workgroups of
    # 32 value channels per head at 64-token chunks)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for N, T, Hv in ((1, 65536, 4), (1, 4096, 16), (1, 65536, 1), (8, 4096, 2), (1, 256, 1)):
        K = gdn.prefill_seg_choose(N, T, Hv)
        assert K >= 1
        assert K == 1 or N * Hv * 4 * (2 * K - 1) <= cus
        assert K == 1 or T // 64 // N >= 4 * K


def test_seg_in_a_hip_graph():
    # three kernels captured from one call; every replay, with eager work and
    # synchronisations between replays, gives the eager call's bits
    x = inputs.make_custom(6700, [1000, 300], 1, 2, io="bf16", init_std=0.1)
    d = to_device(x, DEV)
    K = 3
    ws = torch.empty(gdn.prefill_seg_workspace_size(x.N, x.T_tot, x.Hv, 64, K), dtype=torch.uint8, device=DEV)
    o = torch.empty((x.T_tot, x.Hv, x.Dv), dtype=torch.bfloat16, device=DEV)
    fs = torch.empty((x.N, x.Hv, x.Dv, x.Dk), dtype=torch.float32, device=DEV)
    call = lambda: gdn.prefill_seg(*_args(d), segments=K, out=o, final_state=fs, workspace=ws)  # noqa: E731
    call()
    torch.cuda.synchronize()
    o_ref, f_ref = o.clone(), fs.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        o.zero_()
        fs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(fs, f_ref), f"replay {i} differs"


@pytest.mark.parametrize("K", [2, 4])
@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_kda_seg_shapes(K, io):
    # the per-key-channel decay through the same segments
    for case, (lengths, Hk, Hv, init_std) in enumerate([([700], 1, 2, 0.2), ([0, 130, 1, 64, 77], 1, 2, 0.1),
                                                          ([300, 5], 2, 2, 0.5)]):
        x = inputs.make_custom(6800 + case, lengths, Hk, Hv, io=io, init_std=init_std, per_channel=True,
                               g_shift=0.5 * case, name=f"kda_seg{case}")
        print(f"\n{x.name}: lengths={lengths} Hk={Hk} Hv={Hv} io={io} segments={K}", flush=True)
        d = to_device(x, DEV)
        o, fs = gdn.kda_prefill_seg(*_args(d), segments=K)
        torch.cuda.synchronize()
        ro, rf = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)
        check("o", to_f64(o), ro, x.io)
        check("final_state", to_f64(fs), rf, x.io)


def test_kda_seg_one_segment_is_kda_prefill():
    x = inputs.make_custom(6900, [333, 0, 90], 2, 4, io="bf16", init_std=0.2, per_channel=True)
    d = to_device(x, DEV)
    o1, f1 = gdn.kda_prefill_seg(*_args(d), segments=1)
    o2, f2 = gdn.kda_prefill(*_args(d))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
