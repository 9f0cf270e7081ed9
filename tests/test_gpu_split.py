"""The two-launch scalar-gate prefill (gdn_prefill_split: chunk-parallel map, then the WY
chain) on the GPU vs the fp64 CPU oracle, through the C-ABI.

Same bar as gdn_prefill: 16-bit I/O, error / rms <= 2e-2 beside the stored outputs'
rounding, outputs and final states separately.  Shapes span several chunks with ragged
tails, empty sequences, GQA and initial states; decays up to the strong-decay workload's.
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


def _check_all(x, chunk=64):
    print(f"\n{x.name}: lengths={x.seq_lengths().tolist()[:10]} Hk={x.Hk} Hv={x.Hv} io={x.io} chunk={chunk}",
          flush=True)
    d = to_device(x, DEV)
    o, fs = gdn.prefill_split(*_args(d), chunk_size=chunk)
    torch.cuda.synchronize()
    ro, rf = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)
    return d, o, fs


SMALL = [
    # (lengths, Hk, Hv, init_std)
    ([1], 1, 1, None),
    ([63], 1, 2, None),
    ([64], 2, 2, 0.1),
    ([65], 1, 1, None),
    ([200], 2, 4, 0.1),
    ([0, 130, 1, 64, 77], 1, 2, 0.1),
    ([129, 0], 2, 2, 0.1),
    ([300, 45], 1, 8, 0.1),
    ([190], 4, 16, None),
]


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_split_small_shapes(io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    _check_all(inputs.make_custom(5000 + case, lengths, Hk, Hv, io=io, init_std=init_std,
                                  g_shift=0.5 * (case % 3), name=f"split_small{case}"))


@pytest.mark.parametrize("shift", [2.0, 4.0])
def test_split_strong_decay(shift):
    _check_all(inputs.make_custom(5100 + int(shift), [300, 5], 1, 2, io="bf16", g_shift=shift,
                                  init_std=0.5, name=f"split_decay{shift}"))


@pytest.mark.parametrize("wid,io", [(1, "bf16"), (1, "f16"), (2, "bf16"), (3, "bf16")])
def test_split_workloads(wid, io):
    d, o, fs = _check_all(inputs.make_workload(wid, io=io))
    if wid == 1:
        # the one-launch kernel on the same inputs: both within the bar of the exact result
        og, fg = gdn.prefill(*_args(d))
        torch.cuda.synchronize()
        check_pair("split vs gdn_prefill o", to_f64(o), to_f64(og), io)
        check_pair("split vs gdn_prefill state", to_f64(fs), to_f64(fg), io, stored=False)


def test_split_state_passing_workspace_reuse_and_determinism():
    x = inputs.make_custom(5200, [333], 1, 2, io="bf16", init_std=0.1)
    d = to_device(x, DEV)
    ws = torch.empty(gdn.prefill_split_workspace_size(1, 333, 2), dtype=torch.uint8, device=DEV)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o_all, f_all = gdn.prefill_split(*args, d["initial_state"], workspace=ws)
    o_again, f_again = gdn.prefill_split(*args, d["initial_state"], workspace=ws)
    cut = 128   # chunk-aligned: the two-call split runs the same chunks
    sl = lambda t, a, b: t[a:b].contiguous()  # noqa: E731
    o1, f1 = gdn.prefill_split(*(sl(t, 0, cut) for t in args), d["initial_state"], workspace=ws)
    o2, f2 = gdn.prefill_split(*(sl(t, cut, 333) for t in args), f1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_all, o_again) and torch.equal(f_all, f_again)
    assert torch.equal(torch.cat([o1, o2]), o_all)
    assert torch.equal(f2, f_all)


def test_split_empty_and_in_place():
    x = inputs.make_custom(5300, [0, 0], 1, 2, io="bf16", init_std=0.3)
    d = to_device(x, DEV)
    o, fs = gdn.prefill_split(*_args(d))
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(fs.cpu(), torch.from_numpy(x.initial_state))
    x = inputs.make_custom(5301, [150, 70], 2, 2, io="f16", init_std=0.2)
    d = to_device(x, DEV)
    o_ref, f_ref = gdn.prefill_split(*_args(d))
    st = d["initial_state"].clone()
    o2, _ = gdn.prefill_split(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu_seqlens"], final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o2) and torch.equal(f_ref, st)


def test_split_rejects_fp32_io():
    x = inputs.make_custom(5400, [10], 1, 1, io="f32")
    d = to_device(x, DEV)
    with pytest.raises(gdn.GDNError):
        gdn.prefill_split(d["q"], d["k"], d["v"], d["g"], d["beta"])


def test_split_many_tiny_sequences_and_many_heads():
    rng = np.random.default_rng(5454)
    lengths = rng.integers(0, 6, size=3000)
    _check_all(inputs.make_custom(5500, lengths, 1, 2, io="bf16", init_std=0.2, name="split_tiny3000"))
    _check_all(inputs.make_custom(5501, [130], 8, 64, io="f16", name="split_H64"))


def test_split_in_a_hip_graph():
    # both kernels captured from one call; every replay, with eager work and
    # synchronisations between replays, gives the eager call's bits
    x = inputs.make_workload(1)
    d = to_device(x, DEV)
    ws = torch.empty(gdn.prefill_split_workspace_size(x.N, x.T_tot, x.Hv), dtype=torch.uint8, device=DEV)
    o = torch.empty((x.T_tot, x.Hv, x.Dv), dtype=torch.bfloat16, device=DEV)
    fs = torch.empty((x.N, x.Hv, x.Dv, x.Dk), dtype=torch.float32, device=DEV)
    call = lambda: gdn.prefill_split(*_args(d), out=o, final_state=fs, workspace=ws)  # noqa: E731
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


@pytest.mark.parametrize("chunk", [32, 128])
@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_split_other_chunk_sizes_small(chunk, io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    _check_all(inputs.make_custom(5700 + case, lengths, Hk, Hv, io=io, init_std=init_std,
                                  g_shift=0.5 * (case % 3), name=f"split_c{chunk}_small{case}"), chunk)


@pytest.mark.parametrize("chunk", [32, 128])
def test_split_other_chunk_sizes_ragged_decay_and_workloads(chunk):
    # lengths around the chunk boundaries of every size, strong decay, and the headline and
    # varlen workloads; the three chunk sizes agree within twice the bar
    _check_all(inputs.make_custom(5800, [31, 32, 33, 127, 128, 129, 255, 0, 1], 2, 4, io="bf16", init_std=0.2,
                                  g_shift=1.0, name=f"split_c{chunk}_ragged"), chunk)
    _check_all(inputs.make_custom(5801, [300, 5], 1, 2, io="bf16", g_shift=4.0, init_std=0.5,
                                  name=f"split_c{chunk}_decay"), chunk)
    for wid in (1, 3):
        x = inputs.make_workload(wid)
        d, o, fs = _check_all(x, chunk)
        o64, f64 = gdn.prefill_split(*_args(d), chunk_size=64)
        torch.cuda.synchronize()
        check_pair(f"chunk {chunk} vs 64 o", to_f64(o), to_f64(o64), x.io)
        check_pair(f"chunk {chunk} vs 64 state", to_f64(fs), to_f64(f64), x.io, stored=False)
