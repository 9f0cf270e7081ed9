"""HIP path vs the fp64 CPU oracle, element by element, through the C-ABI.

Every workload is compared at its full size (the oracle finishes all of them in
seconds on the host cores), plus small ragged/edge shapes that span several chunks
and short tails, with fp32, bf16 and fp16 storage of q, k, v, o.  Bar: fp32 I/O max
abs <= 1e-3; 16-bit I/O max abs / rms <= 2e-2 beside the outputs' storage rounding,
outputs and final states separately.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import TORCH_IO, check, to_device, to_f64
from linear_attention_chunked_gdn_amd import gdn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    gdn.load_library()   # fails loudly when the HIP library is not built
    yield


def _run(x, **kw):
    d = to_device(x, DEV)
    o, fs = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                        d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, fs


def _oracle(x):
    return oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)


@pytest.mark.parametrize("wid,io", [(0, None), (1, None), (2, None), (3, None),
                                    (0, "f16"), (1, "f16"), (3, "f16")])
def test_workload_prefill(wid, io):
    x = inputs.make_workload(wid, io=io)
    print(f"\nworkload {wid} {x.name}: N={x.N} T={x.T_tot} Hk={x.Hk} Hv={x.Hv} io={x.io}", flush=True)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_workload_long_prefill_then_decode(io):
    x = inputs.make_workload(4, io=io, decode_steps=None if io == "bf16" else 64)
    print(f"\nworkload 4 {x.name}: T={x.T_tot} H={x.Hv}, then {x.decode['steps']} decode steps",
          flush=True)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, x.io)
    check("state after prefill", to_f64(fs), rf, x.io)
    del o
    dec = x.decode
    dq, dk, dv = (torch.from_numpy(dec[n]).to(DEV, TORCH_IO[x.io]) for n in ("q", "k", "v"))
    dg, db = (torch.from_numpy(dec[n]).to(DEV, torch.float32) for n in ("g", "beta"))
    state = fs
    st_ref = rf
    outs, refs = [], []
    for i in range(dec["steps"]):
        oi = gdn.decode_step(dq[i:i + 1], dk[i:i + 1], dv[i:i + 1], dg[i:i + 1], db[i:i + 1], state)
        outs.append(oi)
        r, st_ref = oracle.decode_step(dec["q"][i:i + 1], dec["k"][i:i + 1], dec["v"][i:i + 1],
                                       dec["g"][i:i + 1], dec["beta"][i:i + 1], st_ref)
        refs.append(r)
    torch.cuda.synchronize()
    check("decode outputs (all steps)", to_f64(torch.cat(outs)), np.concatenate(refs), x.io)
    check("state after decode", to_f64(state), st_ref, x.io)


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


@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes(io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    x = inputs.make_custom(1000 + case, lengths, Hk, Hv, io=io, init_std=init_std,
                           g_shift=0.5 * (case % 3))
    print(f"\nlengths={lengths} Hk={Hk} Hv={Hv} io={io} init={init_std}", flush=True)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, io)
    check("final_state", to_f64(fs), rf, io)


@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
def test_strong_decay_long_chunks(io):
    # g = -softplus(N(0,1) + 4): the cumulative gate reaches about -270 inside one chunk,
    # far past fp32's exponent range, so decays must only be formed as masked differences
    x = inputs.make_custom(77, [300, 5], 1, 2, io=io, g_shift=4.0, init_std=0.5)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, io)
    check("final_state", to_f64(fs), rf, io)


def test_empty_batch_copies_initial_state():
    x = inputs.make_custom(5, [0, 0], 1, 2, io="bf16", init_std=0.3)
    o, fs = _run(x)
    assert o.shape[0] == 0
    assert torch.equal(fs.cpu(), torch.from_numpy(x.initial_state))


def test_zero_initial_state_when_null():
    x = inputs.make_custom(6, [0, 3], 1, 1, io="bf16")
    o, fs = _run(x)
    ro, rf = _oracle(x)
    assert torch.count_nonzero(fs[0]) == 0
    check("final_state", to_f64(fs), rf, "bf16")


def test_in_place_state_and_no_final_state():
    x = inputs.make_custom(7, [150, 70], 2, 2, io="bf16", init_std=0.2)
    d = to_device(x, DEV)
    o_ref, f_ref = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                               d["cu_seqlens"])
    st = d["initial_state"].clone()
    o2, f2 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu_seqlens"],
                         final_state=st)
    o3, f3 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                         d["cu_seqlens"], output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None
    assert torch.equal(o_ref, o2) and torch.equal(o_ref, o3)
    assert torch.equal(f_ref, st)


def test_state_passing_matches_one_call():
    x = inputs.make_custom(8, [333], 1, 2, io="bf16", init_std=0.1)
    d = to_device(x, DEV)
    o_all, f_all = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    cut = 128   # chunk-aligned cut: the two-call split then runs the same chunks
    sl = lambda t, a, b: t[a:b].contiguous()  # noqa: E731
    o1, f1 = gdn.prefill(*(sl(d[n], 0, cut) for n in ("q", "k", "v", "g", "beta")), d["initial_state"])
    o2, f2 = gdn.prefill(*(sl(d[n], cut, 333) for n in ("q", "k", "v", "g", "beta")), f1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2]), o_all)
    assert torch.equal(f2, f_all)


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_deterministic(io):
    x = inputs.make_workload(1, io=io)
    d = to_device(x, DEV)
    a = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    b = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_f16_values_near_the_top_of_its_range():
    # fp16 has 5 exponent bits: v scaled to |v| ~ 1e3 keeps outputs and the state's fp16
    # copy far above the subnormal range and far below 65504
    x = inputs.make_custom(11, [130, 64], 1, 2, io="f16", init_std=50.0)
    x.v = inputs.round_to_f16(x.v * np.float32(1000.0))
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, "f16")
    check("final_state", to_f64(fs), rf, "f16")


def test_decode_step_small_fp32_and_gqa():
    for io in ("f32", "bf16", "f16"):
        x = inputs.make_custom(9, [1, 1, 1], 2, 4, io=io, init_std=0.3)
        d = to_device(x, DEV)
        st = d["initial_state"].clone()
        o = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st)
        torch.cuda.synchronize()
        ro, rs = oracle.decode_step(x.q, x.k, x.v, x.g, x.beta, x.initial_state)
        check(f"decode o ({io})", to_f64(o), ro, io)
        check(f"decode state ({io})", to_f64(st), rs, io)


def test_errors_raise():
    x = inputs.make_custom(10, [10], 1, 1, io="bf16")
    d = to_device(x, DEV)
    with pytest.raises(gdn.GDNError):
        gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=32)


@pytest.mark.parametrize("dvs", ["16", "32"])
def test_phase_by_phase_kernel_bf16(monkeypatch, dvs):
    # the bf16 path of the phase-by-phase kernel (the fp32 kernel's schedule), kept as a
    # cross-check of the pipelined kernel
    monkeypatch.setenv("GDN_KERNEL", "v1")
    monkeypatch.setenv("GDN_DVS", dvs)
    for x in (inputs.make_custom(40, [300, 0, 77], 2, 4, io="bf16", init_std=0.1),
              inputs.make_workload(1)):
        o, fs = _run(x)
        ro, rf = _oracle(x)
        check("o", to_f64(o), ro, x.io)
        check("final_state", to_f64(fs), rf, x.io)


def test_many_tiny_sequences_and_many_heads():
    # 3000 packed sequences of 0-5 tokens (a grid of 3000 x Hv x 8 workgroups, most of
    # them one short chunk), and a 64-head shape
    rng = np.random.default_rng(4242)
    lengths = rng.integers(0, 6, size=3000)
    x = inputs.make_custom(4300, lengths, 1, 2, io="bf16", init_std=0.2)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)
    x = inputs.make_custom(4301, [130], 8, 64, io="f16")
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o (64 heads)", to_f64(o), ro, x.io)
    check("final_state (64 heads)", to_f64(fs), rf, x.io)
