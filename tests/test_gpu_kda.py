"""Per-key-channel decay (KDA) on the GPU vs the fp64 CPU oracle, through the C-ABI.

Same bar as the scalar-gate path: 16-bit I/O, error / rms <= 2e-2 beside the stored
outputs' rounding, outputs and final states separately.  Shapes span several chunks with
ragged tails, empty sequences, GQA and initial states; the gate recipes include decays
far past exp's range inside one chunk and channels that forget at once next to channels
that never decay.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import TORCH_IO, check, check_pair, to_device, to_f64
from linear_attention_chunked_gdn_amd import gdn, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    gdn.load_library()
    yield


def _run(x, **kw):
    d = to_device(x, DEV)
    o, fs = gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                            d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, fs


def _oracle(x):
    return oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)


def _check_all(x):
    print(f"\n{x.name}: lengths={x.seq_lengths().tolist()[:10]} Hk={x.Hk} Hv={x.Hv} io={x.io}", flush=True)
    o, fs = _run(x)
    ro, rf = _oracle(x)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)
    return o, fs


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
]


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_kda_small_shapes(io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    x = inputs.make_custom(2000 + case, lengths, Hk, Hv, io=io, init_std=init_std,
                           g_shift=0.5 * (case % 3), per_channel=True, name=f"kda_small{case}")
    _check_all(x)


@pytest.mark.parametrize("shift", [2.0, 4.0])
def test_kda_strong_decay(shift):
    # mean decay about -2.2 and -4.0 per token and channel: Gamma reaches -140 / -260
    # inside one chunk, so only masked differences and products of decays <= 1 survive
    x = inputs.make_custom(2100 + int(shift), [300, 5], 1, 2, io="bf16", g_shift=shift,
                           init_std=0.5, per_channel=True, name=f"kda_decay{shift}")
    _check_all(x)


def test_kda_mixed_channels():
    # per channel: some forget at once (g = -30), some never decay (g = 0), the rest random
    x = inputs.make_custom(2200, [190, 64], 2, 2, io="bf16", init_std=0.3, per_channel=True,
                           name="kda_mixed")
    x.g[:, :, 0::7] = -30.0
    x.g[:, :, 3::11] = 0.0
    _check_all(x)


def test_kda_uniform_gate_matches_scalar_gate_path():
    # a per-channel gate equal on every channel is the scalar gate: both paths meet the
    # bar against the oracle, so they agree with each other within twice the tolerance
    x = inputs.make_custom(2300, [150, 70], 2, 2, io="bf16", init_std=0.2, name="uniform")
    xk = inputs.GDNInputs("kda_uniform", x.io, x.q, x.k, x.v, np.repeat(x.g[:, :, None], 128, axis=2),
                          x.beta, x.cu_seqlens, x.initial_state)
    ok_, fk = _check_all(xk)
    d = to_device(x, DEV)
    og, fg = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
    torch.cuda.synchronize()
    check_pair("kda vs scalar-gate o", to_f64(ok_), to_f64(og), "bf16")
    check_pair("kda vs scalar-gate state", to_f64(fk), to_f64(fg), "bf16", stored=False)


@pytest.mark.parametrize("wid,io", [(1, "bf16"), (1, "f16"), (2, "bf16"), (3, "bf16")])
def test_kda_workloads(wid, io):
    x = inputs.make_workload(wid, io=io, per_channel=True)
    _check_all(x)


def test_kda_long_prefill_then_decode():
    x = inputs.make_workload(4, per_channel=True, decode_steps=64)
    o, fs = _check_all(x)
    del o
    dec = x.decode
    dq, dk, dv = (torch.from_numpy(dec[n]).to(DEV, TORCH_IO[x.io]) for n in ("q", "k", "v"))
    dg, db = (torch.from_numpy(np.ascontiguousarray(dec[n])).to(DEV, torch.float32) for n in ("g", "beta"))
    state = fs
    _, st_ref = _oracle(x)
    outs, refs = [], []
    for i in range(dec["steps"]):
        outs.append(gdn.kda_decode_step(dq[i:i + 1], dk[i:i + 1], dv[i:i + 1], dg[i:i + 1], db[i:i + 1], state))
        r, st_ref = oracle.decode_step(dec["q"][i:i + 1], dec["k"][i:i + 1], dec["v"][i:i + 1],
                                       dec["g"][i:i + 1], dec["beta"][i:i + 1], st_ref)
        refs.append(r)
    torch.cuda.synchronize()
    check("decode outputs (all steps)", to_f64(torch.cat(outs)), np.concatenate(refs), x.io)
    check("state after decode", to_f64(state), st_ref, x.io)


def test_kda_decode_step_all_dtypes_and_gqa():
    for io in ("f32", "bf16", "f16"):
        x = inputs.make_custom(2400, [1, 1, 1], 2, 4, io=io, init_std=0.3, per_channel=True)
        d = to_device(x, DEV)
        st = d["initial_state"].clone()
        o = gdn.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st)
        torch.cuda.synchronize()
        ro, rs = oracle.decode_step(x.q, x.k, x.v, x.g, x.beta, x.initial_state)
        check(f"kda decode o ({io})", to_f64(o), ro, io)
        check(f"kda decode state ({io})", to_f64(st), rs, io)


def test_kda_state_passing_workspace_reuse_and_determinism():
    x = inputs.make_custom(2500, [333], 1, 2, io="bf16", init_std=0.1, per_channel=True)
    d = to_device(x, DEV)
    ws = torch.empty(gdn.kda_workspace_size(1, 333, 2), dtype=torch.uint8, device=DEV)
    o_all, f_all = gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], workspace=ws)
    o_again, f_again = gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                                       workspace=ws)
    cut = 128   # chunk-aligned: the two-call split runs the same chunks
    sl = lambda t, a, b: t[a:b].contiguous()  # noqa: E731
    o1, f1 = gdn.kda_prefill(*(sl(d[n], 0, cut) for n in ("q", "k", "v", "g", "beta")), d["initial_state"],
                             workspace=ws)
    o2, f2 = gdn.kda_prefill(*(sl(d[n], cut, 333) for n in ("q", "k", "v", "g", "beta")), f1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_all, o_again) and torch.equal(f_all, f_again)
    assert torch.equal(torch.cat([o1, o2]), o_all)
    assert torch.equal(f2, f_all)


def test_kda_empty_and_in_place():
    x = inputs.make_custom(2600, [0, 0], 1, 2, io="bf16", init_std=0.3, per_channel=True)
    o, fs = _run(x)
    assert o.shape[0] == 0
    assert torch.equal(fs.cpu(), torch.from_numpy(x.initial_state))
    x = inputs.make_custom(2601, [150, 70], 2, 2, io="f16", init_std=0.2, per_channel=True)
    d = to_device(x, DEV)
    o_ref, f_ref = gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
    st = d["initial_state"].clone()
    o2, _ = gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu_seqlens"], final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o2) and torch.equal(f_ref, st)


def test_kda_rejects_fp32_io():
    x = inputs.make_custom(2700, [10], 1, 1, io="f32", per_channel=True)
    d = to_device(x, DEV)
    with pytest.raises(gdn.GDNError):
        gdn.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])


def test_kda_many_tiny_sequences_and_many_heads():
    # 3000 packed sequences of 0-5 tokens: 3000 + T/64 chunk slots, most unused, found by
    # the map kernel's binary search over cu_seqlens; and a 64-head shape
    rng = np.random.default_rng(4343)
    lengths = rng.integers(0, 6, size=3000)
    _check_all(inputs.make_custom(4400, lengths, 1, 2, io="bf16", init_std=0.2, per_channel=True,
                                  name="kda_tiny3000"))
    _check_all(inputs.make_custom(4401, [130], 8, 64, io="f16", per_channel=True, name="kda_H64"))
