"""Library-level behaviour on the GPU, through the C-ABI: gdn_prefill_auto (the library's
own choice among the prefill paths) against the entry point it chose, the GDN_CHECK
read-back of cu_seqlens, and every 16-bit prefill path with values near the top of
fp16's range (the precondition the header states for bf16 and fp16 I/O).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import check, to_device, to_f64
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


# ---- gdn_prefill_auto ------------------------------------------------------------------

AUTO = [
    # (inputs, expected path): the two-launch recurrence while its workgroups (at least 4
    # per head) fit the 256 CUs in one round, segmented when three or more segments fit
    # (4 heads of a long sequence; 16 heads fit only two); 80 heads take the one-launch
    # kernel; packed batches take the two-launch map; fp32 has one path
    (lambda: inputs.make_workload(1), "split"),
    (lambda: inputs.make_custom(7700, [8192], 2, 4, io="bf16", init_std=0.1, name="auto_H4_T8192"), "seg"),
    (lambda: inputs.make_custom(7701, [1000], 16, 32, io="f16", name="auto_H32_T1000"), "split"),
    (lambda: inputs.make_custom(7704, [300], 80, 80, io="bf16", name="auto_H80_T300"), "one_launch"),
    (lambda: inputs.make_custom(7702, [100, 0, 700, 65], 2, 16, io="bf16", init_std=0.2, name="auto_packed"),
     "split"),
    (lambda: inputs.make_workload(0), "one_launch"),
]


def _chosen(path, d, plan):
    if path == "split":
        return gdn.prefill_split(*_args(d))
    if path == "seg":
        return gdn.prefill_seg(*_args(d), segments=plan["segments"])
    return gdn.prefill(*_args(d))


@pytest.mark.parametrize("case", range(len(AUTO)))
def test_auto_runs_the_planned_path(case):
    make, want = AUTO[case]
    x = make()
    io = {"f32": gdn.GDN_F32, "bf16": gdn.GDN_BF16, "f16": gdn.GDN_F16}[x.io]
    plan = gdn.prefill_auto_plan(x.N, x.T_tot, x.Hv, io)
    print(f"\n{x.name}: plan {plan}", flush=True)
    assert plan["path"] == want
    d = to_device(x, DEV)
    o, fs = gdn.prefill_auto(*_args(d))
    o2, f2 = _chosen(want, d, plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fs, f2)
    if x.T_tot * x.Hv <= 20000:
        ro, rf = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)
        check("o", to_f64(o), ro, x.io)
        check("final_state", to_f64(fs), rf, x.io)


def test_auto_with_the_prologue():
    # the headline shape with raw inputs: the fused two-launch path
    x = inputs.make_workload(1, raw=True)
    plan = gdn.prefill_auto_plan(x.N, x.T_tot, x.Hv, gdn.GDN_BF16, gdn.PROLOGUE_ALL)
    assert plan["path"] == "split"
    d = to_device(x, DEV)
    o, fs = gdn.prefill_auto(*_args(d), prologue=gdn.PROLOGUE_ALL)
    o2, f2 = gdn.prefill_split(*_args(d), prologue=gdn.PROLOGUE_ALL)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fs, f2)


def test_auto_rejects_a_short_workspace():
    x = inputs.make_custom(7703, [300], 1, 2, io="bf16")
    d = to_device(x, DEV)
    need = gdn.prefill_auto_plan(x.N, x.T_tot, x.Hv, gdn.GDN_BF16)["workspace_bytes"]
    assert need > 0
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(gdn.GDNError, match="smaller than"):
        gdn.prefill_auto(*_args(d), workspace=ws)


# ---- GDN_CHECK -------------------------------------------------------------------------

# malformed packings of T_tot = 10 tokens: the check returns before any launch
BAD_CU = [([2, 10], "cu_seqlens\\[0\\] = 2"),
          ([0, 6, 4, 10], "decreases at 2"),
          ([0, 3, 8], "cu_seqlens\\[2\\] = 8, not T_tot = 10")]

ENTRY = {
    "prefill": lambda a, cu: gdn.prefill(*a, cu_seqlens=cu),
    "prefill_split": lambda a, cu: gdn.prefill_split(*a, cu_seqlens=cu),
    "prefill_seg": lambda a, cu: gdn.prefill_seg(*a, cu_seqlens=cu, segments=2),
    "prefill_split_noalloc": lambda a, cu: gdn.prefill_split_noalloc(*a, cu_seqlens=cu),
    "prefill_auto": lambda a, cu: gdn.prefill_auto(*a, cu_seqlens=cu),
}


@pytest.mark.parametrize("entry", sorted(ENTRY))
def test_gdn_check_rejects_malformed_cu_seqlens(entry, monkeypatch):
    x = inputs.make_custom(7800, [10], 1, 2, io="bf16")
    d = to_device(x, DEV)
    a = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    monkeypatch.setenv("GDN_CHECK", "1")
    for cu, msg in BAD_CU:
        c = torch.tensor(cu, dtype=torch.int32, device=DEV)
        with pytest.raises(gdn.GDNError, match=msg):
            ENTRY[entry](a, c)
    # a valid packing passes the check and gives the unchecked call's results
    good = torch.tensor([0, 4, 4, 10], dtype=torch.int32, device=DEV)
    o1, f1 = ENTRY[entry](a, good)
    monkeypatch.setenv("GDN_CHECK", "0")
    o2, f2 = ENTRY[entry](a, good)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_gdn_check_kda(monkeypatch):
    x = inputs.make_custom(7801, [10], 1, 2, io="bf16", per_channel=True)
    d = to_device(x, DEV)
    monkeypatch.setenv("GDN_CHECK", "1")
    c = torch.tensor([0, 3, 8], dtype=torch.int32, device=DEV)
    for fn in (gdn.kda_prefill, gdn.kda_prefill_seg):
        with pytest.raises(gdn.GDNError, match="not T_tot = 10"):
            fn(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=c)


# ---- values near the top of fp16's range -----------------------------------------------

def _near_range(seed, per_channel):
    # states up to ~4e4 from the first token to the last (initial states N(0, 9000^2), a
    # decay of ~0.9997 per token), values up to ~1.9e4, outputs up to ~3.6e4 at an rms of
    # ~6.7e3: within a factor 2 of fp16's largest finite value (65504) in the state's
    # 16-bit copy throughout
    x = inputs.make_custom(seed, [300, 77], 1, 2, io="bf16", init_std=9000.0, g_shift=-8.0,
                           per_channel=per_channel, name="near_fp16_range")
    x.v = inputs.round_to_bf16(x.v * np.float32(4000.0))
    return x


NEAR = {
    "prefill": (False, lambda a: gdn.prefill(*a)),
    "prefill_split": (False, lambda a: gdn.prefill_split(*a)),
    "prefill_seg": (False, lambda a: gdn.prefill_seg(*a, segments=3)),
    "kda_prefill": (True, lambda a: gdn.kda_prefill(*a)),
    "kda_prefill_seg": (True, lambda a: gdn.kda_prefill_seg(*a, segments=3)),
}


@pytest.mark.parametrize("entry", sorted(NEAR))
def test_bf16_values_near_the_fp16_range(entry):
    per_channel, fn = NEAR[entry]
    x = _near_range(7900, per_channel)
    ro, rf = oracle.recurrent(x.q, x.k, x.v, x.g, x.beta, x.initial_state, x.cu_seqlens)
    assert 3e4 < np.abs(x.initial_state).max() < 65504 and np.abs(ro).max() > 3e4 and np.abs(rf).max() > 2e4
    d = to_device(x, DEV)
    o, fs = fn(_args(d))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(fs).all()
    check("o", to_f64(o), ro, x.io)
    check("final_state", to_f64(fs), rf, x.io)


# ---- HIP graph capture ---------------------------------------------------------------

GRAPH_CASES = [
    # (inputs, entry point, expected gdn_prefill_auto path or None): the headline shape
    # (split), one GPU's share of the long workload (segmented), 80 heads (the one-launch
    # kernel, no workspace), and the per-key-channel prefill
    (lambda: inputs.make_workload(1), "auto", "split"),
    (lambda: inputs.head_shard(inputs.make_workload(4), 8), "auto", "seg"),
    (lambda: inputs.make_custom(7951, [300], 80, 80, io="bf16", init_std=0.1), "auto", "one_launch"),
    (lambda: inputs.make_custom(7952, [1000, 333], 8, 16, io="bf16", init_std=0.1, per_channel=True), "kda", None),
]


@pytest.mark.parametrize("case", range(len(GRAPH_CASES)))
def test_graph_replays_match_eager(case):
    # a prefill call captured in a HIP graph, replayed three times with eager calls on
    # other inputs between the replays; every replay gives the eager call's bits
    make, entry, path = GRAPH_CASES[case]
    x = make()
    d = to_device(x, DEV)
    if entry == "auto":
        plan = gdn.prefill_auto_plan(x.N, x.T_tot, x.Hv, gdn.GDN_BF16)
        assert plan["path"] == path
        nbytes = plan["workspace_bytes"]
        call = gdn.prefill_auto
        y = inputs.make_custom(7950, [300, 77], 1, x.Hv, io="bf16", init_std=0.1)
    else:
        nbytes = gdn.kda_workspace_size(x.N, x.T_tot, x.Hv)
        call = gdn.kda_prefill
        y = inputs.make_custom(7953, [300, 77], 1, x.Hv, io="bf16", init_std=0.1, per_channel=True)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    o_ref, f_ref = call(*_args(d), workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(o_ref)
    fs = torch.empty_like(f_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(*_args(d), out=out, final_state=fs, workspace=ws)
    dy = to_device(y, DEV)
    for rep in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(fs, f_ref), f"replay {rep}"
        call(*_args(dy))   # eager work between the replays, sharing the workspace's device
        torch.cuda.synchronize()
