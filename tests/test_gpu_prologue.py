"""The fused input prologue on the GPU (gdn_prefill_fused, gdn_decode_step_fused) vs the
fp64 oracle applying the same steps (oracle.prologue) to the same stored inputs.

Inputs are the generator's raw draws (q, k not normalised, beta and g as logits).  For a
subset of the steps, the others are applied on the host first and the result, rounded to
the storage types, is what both sides read.  Same bar as the plain path.
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
    gdn.load_library()
    yield


def _round(x, io):
    if io == "bf16":
        return inputs.round_to_bf16(x)
    if io == "f16":
        return inputs.round_to_f16(x)
    return np.asarray(x, np.float32)


def _host_steps(x, flags):
    """Apply on the host the prologue steps NOT in flags (rounded to the storage types)."""
    rest = oracle.PROLOGUE_QK_L2NORM | oracle.PROLOGUE_BETA_SIGMOID | oracle.PROLOGUE_G_SOFTPLUS
    q, k, g, b = oracle.prologue(x.q, x.k, x.g, x.beta, rest & ~flags)
    return inputs.GDNInputs(x.name, x.io, _round(q, x.io), _round(k, x.io), x.v, g.astype(np.float32),
                            b.astype(np.float32), x.cu_seqlens, x.initial_state)


def _oracle(x, flags):
    q, k, g, b = oracle.prologue(x.q, x.k, x.g, x.beta, flags)
    return oracle.recurrent(q, k, x.v, g, b, x.initial_state, x.cu_seqlens)


def _run(x, flags, split=False):
    d = to_device(x, DEV)
    fn = gdn.prefill_split if split else gdn.prefill
    o, fs = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"], prologue=flags)
    torch.cuda.synchronize()
    return o, fs


SMALL = [([1], 1, 1, None), ([65], 1, 2, None), ([200], 2, 4, 0.1), ([0, 130, 1, 64, 77], 1, 2, 0.1)]


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prologue_all_steps_small_shapes(io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    x = inputs.make_custom(3000 + case, lengths, Hk, Hv, io=io, init_std=init_std, g_shift=0.5, raw=True)
    print(f"\nlengths={lengths} Hk={Hk} Hv={Hv} io={io}", flush=True)
    o, fs = _run(x, gdn.PROLOGUE_ALL)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, io)
    check("final_state", to_f64(fs), rf, io)


@pytest.mark.parametrize("flags", [1, 2, 4, 3, 6])
def test_prologue_flag_subsets(flags):
    raw = inputs.make_custom(3100 + flags, [150, 70], 2, 2, io="bf16", init_std=0.2, g_shift=1.0, raw=True)
    x = _host_steps(raw, flags)
    o, fs = _run(x, flags)
    ro, rf = _oracle(x, flags)
    check("o", to_f64(o), ro, "bf16")
    check("final_state", to_f64(fs), rf, "bf16")


def test_prologue_unnormalised_scale_and_strong_decay():
    # rows far from unit norm (x 40) and decay logits shifted to about -4.0 per token
    x = inputs.make_custom(3200, [300, 5], 1, 2, io="bf16", init_std=0.5, g_shift=4.0, raw=True)
    x.q = inputs.round_to_bf16(x.q * np.float32(40.0))
    x.k = inputs.round_to_bf16(x.k * np.float32(0.05))
    o, fs = _run(x, gdn.PROLOGUE_ALL)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, "bf16")
    check("final_state", to_f64(fs), rf, "bf16")


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_prologue_headline_shape(io):
    x = inputs.make_custom(3300, [4096], 16, 16, io=io, raw=True, name="raw_H16_T4096")
    o, fs = _run(x, gdn.PROLOGUE_ALL)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, io)
    check("final_state", to_f64(fs), rf, io)


def test_prologue_off_is_the_plain_kernel():
    x = inputs.make_custom(3400, [129], 1, 2, io="bf16", init_std=0.1)
    d = to_device(x, DEV)
    a = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    b = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], prologue=0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
def test_decode_prologue(io):
    x = inputs.make_custom(3500, [1, 1, 1], 2, 4, io=io, init_std=0.3, raw=True)
    d = to_device(x, DEV)
    st = d["initial_state"].clone()
    o = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, prologue=gdn.PROLOGUE_ALL)
    torch.cuda.synchronize()
    q, k, g, b = oracle.prologue(x.q, x.k, x.g, x.beta, gdn.PROLOGUE_ALL)
    ro, rs = oracle.decode_step(q, k, x.v, g, b, x.initial_state)
    check(f"decode o ({io})", to_f64(o), ro, io)
    check(f"decode state ({io})", to_f64(st), rs, io)


# the same steps in the two-launch path's map kernel (gdn_prefill_split_fused)

@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_split_prologue_all_steps_small_shapes(io, case):
    lengths, Hk, Hv, init_std = SMALL[case]
    x = inputs.make_custom(3400 + case, lengths, Hk, Hv, io=io, init_std=init_std, g_shift=0.5, raw=True)
    print(f"\nsplit: lengths={lengths} Hk={Hk} Hv={Hv} io={io}", flush=True)
    o, fs = _run(x, gdn.PROLOGUE_ALL, split=True)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, io)
    check("final_state", to_f64(fs), rf, io)


@pytest.mark.parametrize("flags", [1, 2, 4, 3, 6])
def test_split_prologue_flag_subsets(flags):
    raw = inputs.make_custom(3500 + flags, [150, 70], 2, 2, io="bf16", init_std=0.2, g_shift=1.0, raw=True)
    x = _host_steps(raw, flags)
    o, fs = _run(x, flags, split=True)
    ro, rf = _oracle(x, flags)
    check("o", to_f64(o), ro, "bf16")
    check("final_state", to_f64(fs), rf, "bf16")


@pytest.mark.parametrize("chunk", [32, 128])
def test_split_prologue_other_chunk_sizes(chunk):
    x = inputs.make_custom(3600 + chunk, [200, 0, 129], 2, 4, io="bf16", init_std=0.1, g_shift=0.5, raw=True)
    d = to_device(x, DEV)
    o, fs = gdn.prefill_split(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"],
                              chunk_size=chunk, prologue=gdn.PROLOGUE_ALL)
    torch.cuda.synchronize()
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, "bf16")
    check("final_state", to_f64(fs), rf, "bf16")


def test_split_prologue_headline_workload():
    x = inputs.make_workload(1, raw=True)
    o, fs = _run(x, gdn.PROLOGUE_ALL, split=True)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)


def test_split_prologue_unnormalised_scale_and_strong_decay():
    x = inputs.make_custom(3700, [300, 5], 1, 2, io="bf16", init_std=0.5, g_shift=4.0, raw=True)
    x.q = inputs.round_to_bf16(x.q * np.float32(40.0))
    x.k = inputs.round_to_bf16(x.k * np.float32(0.05))
    o, fs = _run(x, gdn.PROLOGUE_ALL, split=True)
    ro, rf = _oracle(x, gdn.PROLOGUE_ALL)
    check("o", to_f64(o), ro, "bf16")
    check("final_state", to_f64(fs), rf, "bf16")


def test_split_prologue_off_is_the_split_path():
    x = inputs.make_custom(3800, [129], 1, 2, io="bf16", init_std=0.1)
    d = to_device(x, DEV)
    a = gdn.prefill_split(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    b = gdn.prefill_split(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], prologue=0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
