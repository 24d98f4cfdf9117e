"""GPU parity: the HIP library against the CPU fp64 oracle, element by element.

Bar (floating point): every output element satisfies
    |gpu - oracle| <= 1e-2 + 1e-2 * |oracle|
(max-abs 1e-2 and max-relative 1e-2, in fp32 output against bf16 inputs).
Both sides always receive the same bf16 tensors (the GPU copy is moved to the
host for the oracle); padding beyond each sequence's length is poisoned with
NaN so a read of it shows.

Small cases cover several tiles, ragged tails, every head size, both kernel
families, forced split sizes (so the combine kernel runs) and edge cases.  The
five full-size workloads run in the launch configuration the benchmark uses,
every sequence against the oracle.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gqa_decode_attention_mqa_amd import binding
from gqa_decode_attention_mqa_amd.workloads import (WORKLOADS, Workload, make_inputs, make_prefill_inputs,
                                                    make_multi_inputs, page_contiguous_cache, page_quant_cache,
                                                    poison_positions_below_, quantize_cache)

pytestmark = pytest.mark.gpu

ATOL = 1e-2
RTOL = 1e-2
DEV = "cuda:0"


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def check_close(gpu, ref, what=""):
    g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) else gpu
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements out of tolerance, max abs err %.3g" % (what, int(bad.sum()), err.max())
    return float(err.max())


def run_case(w: Workload, variant=None, chunk=None, seq_lens=None, poison=True, combine=None):
    inp = to_dev(make_inputs(w, poison_padding=poison, seq_lens=seq_lens))
    out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], variant=variant, chunk=chunk,
                         combine=combine)
    torch.cuda.synchronize()
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    return check_close(out, ref, "%s variant=%s chunk=%s combine=%s" % (w, variant, chunk, combine))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield
    binding.release_workspaces()


def test_tiny_workload_full():
    print("case tiny", flush=True)
    run_case(WORKLOADS["tiny"])


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G,Hkv,B", [(1, 2, 3), (2, 3, 5), (3, 1, 3), (4, 2, 4), (8, 1, 3), (16, 1, 8), (48, 1, 3),
                                     (20, 2, 3), (64, 1, 3), (80, 1, 3), (96, 1, 2), (112, 1, 2)])
def test_small_shapes(variant, D, G, Hkv, B):
    seed = 1000 + D + 7 * G + Hkv + (0 if variant == "mfma" else 1)
    w = Workload("small", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=700, seed=seed, len_lo=1, len_hi=700)
    print("case small", variant, D, G, Hkv, B, flush=True)
    # planner's chunk, then forced 128-position chunks merged by the fused
    # combine and by the separate combine kernel, all on the same inputs
    run_case(w, variant=variant)
    run_case(w, variant=variant, chunk=128)
    run_case(w, variant=variant, chunk=128, combine="fused")


def _random_shapes(n, seed):
    """Seeded random decode shapes: B <= 8, G in {1, 2, 4, 8, 16, 48}, D in {64, 128, 256}, lengths 0..3000."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16, 48]))
        Hkv = int(rng.choice([1, 2, 4])) if G <= 16 else 1
        D = int(rng.choice([64, 128, 256]))
        B = int(rng.integers(1, 9))
        Lmax = int(rng.integers(1, 3001))
        shapes.append((B, G * Hkv, Hkv, D, Lmax, 5000 + 17 * seed + i))
    return shapes


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax,seed", _random_shapes(12, 1))
def test_random_shapes(B, Hq, Hkv, D, Lmax, seed):
    w = Workload("rand", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=seed, len_lo=0, len_hi=Lmax)
    print("case random", B, Hq, Hkv, D, Lmax, seed, flush=True)
    run_case(w)                  # the planner's choice
    run_case(w, chunk=128)       # many chunks, both combine kernels


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_edge_lengths(variant):
    w = Workload("edges", B=8, Hq=16, Hkv=2, D=128, Lmax=300, seed=77)
    lens = [0, 1, 2, 63, 64, 65, 299, 300]
    print("case edges", variant, flush=True)
    run_case(w, variant=variant, seq_lens=lens)
    run_case(w, variant=variant, chunk=128, seq_lens=lens)
    run_case(w, variant=variant, chunk=128, seq_lens=lens, combine="fused")


@pytest.mark.parametrize("combine", ["fused", "separate"])
def test_many_chunks_and_shape_changes_reuse_the_workspace(combine):
    """The fused combine's counters must be back at zero after every call, whatever the shape."""
    cases = [Workload("ws1", B=8, Hq=48, Hkv=1, D=256, Lmax=2000, seed=90, len_lo=1, len_hi=2000),
             Workload("ws2", B=16, Hq=16, Hkv=2, D=128, Lmax=1900, seed=91, len_lo=1000, len_hi=1900),
             Workload("ws3", B=8, Hq=48, Hkv=1, D=256, Lmax=2000, seed=92, len_lo=1, len_hi=2000)]
    for w in cases:
        for variant in ("mfma", "valu"):
            print("case ws", w.name, combine, variant, flush=True)
            # the fused merge takes at most 8 chunks per sequence
            run_case(w, variant=variant, chunk=128 if combine == "separate" else 256, combine=combine)


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_fused_combine_reads_this_calls_partials(variant):
    """The fused combine's workgroups read each other's partials through device-coherent loads:
    two different input sets alternate through the same cached workspace, so a stale read (the
    previous call's partials) would show as a wrong result."""
    ws = [Workload("fz%d" % i, B=8, Hq=48, Hkv=1, D=256, Lmax=1536, seed=1200 + i, len_lo=700, len_hi=1536)
          for i in range(2)]
    cases = []
    for w in ws:
        inp = make_inputs(w, poison_padding=True)
        ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
        cases.append((to_dev(inp), ref))
    for it in range(12):
        dev, ref = cases[it % 2]
        print("case fused alternate", variant, it, flush=True)
        out = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant, chunk=256,
                             combine="fused")
        torch.cuda.synchronize()
        check_close(out, ref, "fused alternate %s iteration %d" % (variant, it))


@pytest.mark.parametrize("hint", ["uniform", "ragged", "wrong"])
def test_host_lengths_hint_changes_the_plan_not_the_result(hint):
    """The host copy of the lengths only picks the chunk size.  A uniform batch gets whole-sequence
    chunks, a ragged one short chunks; a hint that claims a uniform batch of short sequences while
    the device lengths are ragged up to Lmax must still give every position (chunks cover Lmax)."""
    w = Workload("hint", B=16, Hq=32, Hkv=4, D=128, Lmax=3000, seed=1700, len_lo=1, len_hi=3000)
    lens = {"uniform": [3000] * 16, "ragged": None, "wrong": None}[hint]
    inp = make_inputs(w, poison_padding=True,
                      seq_lens=None if lens is None else torch.tensor(lens, dtype=torch.int32))
    host = inp["seq_lens"].clone() if hint != "wrong" else torch.full((16,), 200, dtype=torch.int32)
    ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    dev = to_dev(inp)
    plan = binding.plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, inp["scale"], host_seq_lens=host)
    assert plan["chunk"] * plan["max_splits"] >= w.Lmax
    print("case host lengths hint", hint, plan["chunk"], flush=True)
    out = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], host_seq_lens=host)
    torch.cuda.synchronize()
    check_close(out, ref, "host lengths hint %s" % hint)


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_fused_combine_with_timed_out_waits(variant):
    """The fused combine's bounded wait, forced to time out at once (MQA_FUSED_WAIT_TICKS=0, read
    by the library on every call): workgroups that give up their part of the merge either merge it
    themselves (the last chunk came meanwhile) or leave it to the last one.  Every call must still
    give the separate merge's bits, and so must ordinary fused calls afterwards (a part left
    recorded in the counters only makes a later call merge it twice)."""
    ws = [Workload("fw%d" % i, B=8, Hq=48, Hkv=1, D=256, Lmax=1024, seed=1230 + i, len_lo=300, len_hi=1024)
          for i in range(2)]
    cases = []
    for w in ws:
        dev = to_dev(make_inputs(w, poison_padding=True))
        ref = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant,
                             chunk=128, combine="separate")
        cases.append((dev, ref))
    torch.cuda.synchronize()
    old = os.environ.get("MQA_FUSED_WAIT_TICKS")
    try:
        for it in range(16):
            if it < 8:
                os.environ["MQA_FUSED_WAIT_TICKS"] = "0"
            else:  # the default wait
                os.environ.pop("MQA_FUSED_WAIT_TICKS", None)
            dev, ref = cases[it % 2]
            print("case fused timed-out waits", variant, it, flush=True)
            out = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant,
                                 chunk=128, combine="fused")
            torch.cuda.synchronize()
            assert torch.equal(out, ref), "fused merge with timed-out waits, %s iteration %d" % (variant, it)
    finally:
        if old is None:
            os.environ.pop("MQA_FUSED_WAIT_TICKS", None)
        else:
            os.environ["MQA_FUSED_WAIT_TICKS"] = old


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [None, 128, 256])
def test_fused_and_separate_merges_give_the_same_bits(variant, chunk):
    """Both merge forms run the same arithmetic over the same partials in the same order."""
    w = Workload("fz-eq", B=6, Hq=48, Hkv=1, D=256, Lmax=1000, seed=1210, len_lo=0, len_hi=1000)
    dev = to_dev(make_inputs(w, poison_padding=True))
    print("case fused == separate", variant, chunk, flush=True)
    a = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant, chunk=chunk,
                       combine="separate")
    b = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant, chunk=chunk,
                       combine="fused")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("vscale", [2.0 ** 20, 2.0 ** -20])
def test_split_partials_keep_range_and_precision(variant, vscale):
    """Split chunks store fp16 partials scaled per (chunk, head); V far outside the fp16 range
    (and far below it) must come back exact up to that rounding.  Attention is linear in V, so
    the output is compared after dividing by the (power-of-two, hence exact) scale."""
    w = Workload("range", B=3, Hq=8, Hkv=2, D=128, Lmax=900, seed=84, len_lo=300, len_hi=900)
    inp = to_dev(make_inputs(w))
    inp["v"] = (inp["v"].float() * vscale).to(torch.bfloat16)
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    for combine in ("separate", "fused"):
        print("case range", variant, vscale, combine, flush=True)
        out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], variant=variant,
                             chunk=128, combine=combine)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        err = check_close(out.double() / vscale, ref / vscale, "range %s %g %s" % (variant, vscale, combine))
        assert err <= 2e-3 * float(np.abs(ref / vscale).max()) + 1e-3


def test_lengths_outside_the_cache_are_clamped():
    w = Workload("clamp", B=3, Hq=8, Hkv=1, D=64, Lmax=200, seed=78)
    inp = to_dev(make_inputs(w, seq_lens=[-5, 200, 200]))
    inp["seq_lens"][2] = 10_000
    out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), [0, 200, 200], inp["scale"])
    check_close(out, ref, "clamp")


def test_empty_batch_and_empty_cache():
    q = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((0, 16, 1, 64), dtype=torch.bfloat16, device=DEV)
    out = binding.decode(q, kv, kv, torch.zeros((0,), dtype=torch.int32, device=DEV))
    assert out.shape == (0, 8, 64)
    q = torch.randn((2, 8, 64), device=DEV).to(torch.bfloat16)
    kv = torch.zeros((2, 0, 1, 64), dtype=torch.bfloat16, device=DEV)
    out = binding.decode(q, kv, kv, torch.zeros((2,), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.zeros((2, 8, 64)))


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_bitwise_deterministic(variant):
    w = Workload("det", B=4, Hq=48, Hkv=1, D=256, Lmax=1500, seed=79)
    inp = to_dev(make_inputs(w))
    outs = [binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], variant=variant, chunk=256)
            .clone() for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
def test_bitwise_deterministic_8bit(kv_format):
    """The 8-bit kernel at D = 256 (two waves per 16-head tile, merged in a fixed order), repeated."""
    w = Workload("det8", B=4, Hq=48, Hkv=1, D=256, Lmax=1500, seed=81, len_lo=1, len_hi=1500)
    dev, qc, _ = quant_case(w, kv_format)
    outs = [binding.decode_quant(dev["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                                 dev["seq_lens"], kv_format, dev["scale"], chunk=256).clone() for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_identical_keys_give_mean_of_values():
    w = Workload("same-k", B=2, Hq=48, Hkv=1, D=256, Lmax=1000, seed=80, len_lo=500, len_hi=1000)
    inp = to_dev(make_inputs(w))
    inp["k"][:] = inp["k"][:, :1].clone()
    out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"]).cpu().double()
    for b in range(w.B):
        n = int(inp["seq_lens"][b])
        mean = inp["v"][b, :n].double().mean(dim=0).cpu()          # [1, D]
        err = (out[b] - mean).abs().max().item()
        assert err <= ATOL, err


def test_dominant_logit_selects_its_value_row():
    w = Workload("dom", B=1, Hq=16, Hkv=16, D=128, Lmax=2000, seed=81)
    inp = make_inputs(w)
    stars = [(h * 97 + 13) % 2000 for h in range(16)]
    for h, js in enumerate(stars):
        inp["k"][0, js, h] = (inp["q"][0, h].float() * 8.0).to(torch.bfloat16)
    inp = to_dev(inp)
    out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"]).cpu().double()
    for h, js in enumerate(stars):
        err = (out[0, h] - inp["v"][0, js, h].cpu().double()).abs().max().item()
        assert err <= ATOL, (h, err)


def test_runs_on_a_side_stream():
    w = Workload("stream", B=4, Hq=8, Hkv=1, D=128, Lmax=900, seed=82)
    inp = to_dev(make_inputs(w))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], chunk=128)
    s.synchronize()
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    check_close(out, ref, "side stream")


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax", [(2, 8, 1, 64, 150), (2, 48, 1, 256, 130), (3, 16, 4, 128, 97)])
def test_prefill_matches_oracle_causal_attention(B, Hq, Hkv, D, Lmax):
    w = Workload("pf", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=83 + D, len_lo=1, len_hi=Lmax)
    inp = to_dev(make_prefill_inputs(w, poison_padding=True))
    print("case prefill", B, Hq, Hkv, D, Lmax, flush=True)
    out = binding.prefill(inp["q_seq"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    torch.cuda.synchronize()
    ref = oracle.causal_prefill(inp["q_seq"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(),
                                inp["scale"])
    check_close(out, ref, "prefill")
    # decode at each sequence's full length equals the last prefill row
    lens = inp["seq_lens"].cpu()
    q_last = torch.stack([inp["q_seq"][b, int(lens[b]) - 1] for b in range(B)]).contiguous()
    dec = binding.decode(q_last, inp["k"], inp["v"], inp["seq_lens"], inp["scale"]).cpu()
    last = torch.stack([out[b, int(lens[b]) - 1].cpu() for b in range(B)])
    assert (dec - last).abs().max().item() <= ATOL


@pytest.mark.parametrize("G,Hkv,D,Lmax,B", [(1, 2, 64, 700, 2), (2, 3, 128, 333, 3), (4, 2, 128, 500, 2),
                                           (8, 1, 256, 420, 2), (48, 1, 256, 300, 2), (64, 1, 128, 200, 2),
                                           (80, 1, 64, 150, 2), (96, 1, 128, 130, 1), (112, 1, 64, 100, 2),
                                           (3, 2, 256, 257, 2), (20, 2, 128, 97, 3)])
def test_prefill_shapes(G, Hkv, D, Lmax, B):
    """The prefill kernel at several tiles per prefix, row blocks of (position, head) rows that
    split a position's heads or do not divide Lmax * G, ragged lengths (0, 1 and Lmax among them),
    NaN padding past each length, several kv heads, every head size."""
    Hq = G * Hkv
    w = Workload("pf-blk", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=1400 + G + D + Lmax)
    inp = make_prefill_inputs(w)
    lens = torch.tensor(([0, Lmax, 1] + [Lmax // 2 + 7])[:B] if B > 1 else [Lmax - 3], dtype=torch.int32)
    from gqa_decode_attention_mqa_amd.workloads import poison_padding_
    poison_padding_(inp["k"], lens)
    poison_padding_(inp["v"], lens)
    plan = binding.prefill_plan(B, Hq, Hkv, D, Lmax, inp["scale"])
    rows = plan["rows_per_block"]
    assert rows % 16 == 0 and 64 <= rows <= 256 and plan["combine"] == 0 and plan["workspace_bytes"] == 0
    assert plan["grid_main"] == B * Hkv * -(-Lmax * G // rows) and plan["block_main"] in (256, 512, 1024)
    ref = oracle.causal_prefill(inp["q_seq"], inp["k"], inp["v"], lens, inp["scale"])
    dev = to_dev(inp)
    print("case prefill shapes", G, Hkv, D, Lmax, B, flush=True)
    out = torch.full((B, Lmax, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    binding.prefill(dev["q_seq"], dev["k"], dev["v"], lens.to(DEV), dev["scale"], out=out)
    torch.cuda.synchronize()
    check_close(out, ref, "prefill G %d D %d Lmax %d" % (G, D, Lmax))
    for b in range(B):  # rows at or past the length are zeros
        assert torch.equal(out[b, int(lens[b]):].cpu(), torch.zeros_like(out[b, int(lens[b]):].cpu()))


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.37])
def test_prefill_scale_signs(scale):
    """The prefill kernel folds the scale into each weight's exponent: a negative scale flips q,
    a zero scale gives equal weights over each prefix (masked positions still excluded)."""
    w = Workload("pf-scale", B=2, Hq=8, Hkv=2, D=128, Lmax=300, seed=1500)
    inp = make_prefill_inputs(w, poison_padding=True)
    ref = oracle.causal_prefill(inp["q_seq"], inp["k"], inp["v"], inp["seq_lens"], scale)
    dev = to_dev(inp)
    print("case prefill scale", scale, flush=True)
    out = binding.prefill(dev["q_seq"], dev["k"], dev["v"], dev["seq_lens"], scale)
    torch.cuda.synchronize()
    check_close(out, ref, "prefill scale %g" % scale)


@pytest.mark.parametrize("name", ["palm", "gqa70b"])
def test_prefill_full_size_rows(name):
    """Prefill of a full-size batch's sequences (the first four of the workload's B, every
    position of their Lmax), checked on sampled rows against the oracle's decode at length t + 1
    (a causal row t is the decode step at that length, pinned in the oracle's tests)."""
    w = WORKLOADS[name].with_(B=4)
    inp = make_prefill_inputs(w, device=DEV)
    print("case full prefill", name, binding.prefill_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax), flush=True)
    out = binding.prefill(inp["q_seq"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(77)
    worst = 0.0
    for b in range(w.B):
        n = int(inp["seq_lens"][b])
        rows = sorted(set([0, 1, n - 1] + torch.randint(0, n, (13,), generator=g).tolist()))
        q = torch.stack([inp["q_seq"][b, t] for t in rows]).contiguous().cpu()
        kk = inp["k"][b:b + 1].cpu().expand(len(rows), -1, -1, -1).contiguous()
        vv = inp["v"][b:b + 1].cpu().expand(len(rows), -1, -1, -1).contiguous()
        ref = oracle.decode(q, kk, vv, torch.tensor([t + 1 for t in rows], dtype=torch.int32), inp["scale"])
        worst = max(worst, check_close(out[b, rows], ref, "%s prefill rows of sequence %d" % (name, b)))
    print("full prefill %s: %d sampled rows per sequence, max abs err %.3g" % (name, 16, worst), flush=True)


# ------------------------------------------------------------ paged cache


def paged_inputs(w: Workload, page_size: int, seed: int, spare_pages: int = 3):
    """Seeded paged pool (NaN padding and spare pages) built on the CPU, then moved to the GPU."""
    inp = make_inputs(w, poison_padding=True)
    pg = page_contiguous_cache(inp, page_size, seed=seed, spare_pages=spare_pages)
    return pg, to_dev(pg)


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("page_size", [32, 64, 128, 256])
@pytest.mark.parametrize("G,Hkv,D", [(8, 2, 128), (4, 2, 64), (48, 1, 256)])
def test_paged_matches_paged_oracle(variant, page_size, G, Hkv, D):
    w = Workload("paged", B=5, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=1000, seed=400 + page_size + D + G,
                 len_lo=0, len_hi=1000)
    pg, dev = paged_inputs(w, page_size, seed=page_size + G)
    ref = oracle.decode_paged(pg["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], pg["seq_lens"], pg["scale"])
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case paged", variant, page_size, G, Hkv, D, chunk, combine, flush=True)
        out = binding.decode_paged(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["seq_lens"],
                                   dev["scale"], variant=variant, chunk=chunk, combine=combine)
        torch.cuda.synchronize()
        check_close(out, ref, "paged %s page %d G %d D %d chunk %s %s" % (variant, page_size, G, D, chunk, combine))


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_paged_equals_contiguous_bitwise(variant):
    """Same data, same plan (max_blocks * page_size == Lmax): the paged kernels read the same
    tiles through the block table and must produce identical bits."""
    w = Workload("pgeq", B=6, Hq=16, Hkv=2, D=128, Lmax=1024, seed=450, len_lo=1, len_hi=1024)
    pg, dev = paged_inputs(w, 64, seed=3)
    for chunk in (None, 128):
        a = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant, chunk=chunk)
        b = binding.decode_paged(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["seq_lens"],
                                 dev["scale"], variant=variant, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_paged_shared_prefix():
    """Two sequences whose block tables point at the same pages, with the same query, agree exactly."""
    w = Workload("pgsh", B=2, Hq=48, Hkv=1, D=256, Lmax=512, seed=451)
    pg, dev = paged_inputs(w, 128, seed=4, spare_pages=0)
    table = dev["block_table"].clone()
    table[1] = table[0]
    q = dev["q"].clone()
    q[1] = q[0]
    out = binding.decode_paged(q, dev["k_pages"], dev["v_pages"], table, dev["seq_lens"], dev["scale"], chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])
    ref = oracle.decode_paged(q.cpu(), pg["k_pages"], pg["v_pages"], table.cpu(), pg["seq_lens"], pg["scale"])
    check_close(out, ref, "shared prefix")


def test_paged_full_size_ragged():
    """The ragged workload on a page pool of 64-position pages (pool = the used pages only),
    every sequence against the paged oracle."""
    w = WORKLOADS["ragged"]
    print("case full paged ragged", flush=True)
    inp = make_inputs(w, device=DEV)
    pg = page_contiguous_cache(inp, 64, seed=5)
    del inp["k"], inp["v"]
    out = binding.decode_paged(pg["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], pg["seq_lens"], pg["scale"])
    torch.cuda.synchronize()
    ref = oracle.decode_paged(pg["q"].cpu(), pg["k_pages"].cpu(), pg["v_pages"].cpu(), pg["block_table"].cpu(),
                              pg["seq_lens"].cpu(), pg["scale"])
    err = check_close(out, ref, "paged ragged")
    print("full paged ragged: all %d sequences checked, max abs err %.3g" % (w.B, err), flush=True)


# ------------------------------------------------------ sliding window (local attention)

def window_inputs(w: Workload, window: int):
    """Seeded inputs whose positions before each sequence's window (and past its end) hold NaN."""
    inp = make_inputs(w, poison_padding=True)
    lo = torch.clamp(inp["seq_lens"].to(torch.int64) - window, min=0).to(torch.int32)
    poison_positions_below_(inp["k"], lo)
    poison_positions_below_(inp["v"], lo)
    return inp


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("window", [1, 31, 32, 33, 100, 333, 999])
@pytest.mark.parametrize("G,Hkv,D", [(8, 2, 128), (4, 2, 64), (48, 1, 256), (2, 3, 128)])
def test_window_matches_window_oracle(variant, window, G, Hkv, D):
    w = Workload("win", B=6, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=1000, seed=500 + window + D + G,
                 len_lo=0, len_hi=1000)
    inp = window_inputs(w, window)
    ref = oracle.decode_window(inp["q"], inp["k"], inp["v"], inp["seq_lens"], window, inp["scale"])
    dev = to_dev(inp)
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case window", variant, window, G, Hkv, D, chunk, combine, flush=True)
        out = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant,
                             chunk=chunk, combine=combine, window=window)
        torch.cuda.synchronize()
        check_close(out, ref, "window %d %s G %d D %d chunk %s %s" % (window, variant, G, D, chunk, combine))


def test_window_entry_point_and_wide_window():
    """mqa_decode_attention_window agrees with the option form bit for bit, and a
    window of at least Lmax gives the plain decode step's bits."""
    w = Workload("win-ep", B=5, Hq=32, Hkv=8, D=128, Lmax=900, seed=520, len_lo=0, len_hi=900)
    dev = to_dev(make_inputs(w, poison_padding=True))
    a = binding.decode_window(dev["q"], dev["k"], dev["v"], dev["seq_lens"], 257, dev["scale"])
    b = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], window=257)
    full = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"])
    wide = binding.decode_window(dev["q"], dev["k"], dev["v"], dev["seq_lens"], 900, dev["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(full, wide)
    ref = oracle.decode_window(dev["q"].cpu(), dev["k"].cpu(), dev["v"].cpu(), dev["seq_lens"].cpu(), 257,
                               dev["scale"])
    check_close(a, ref, "window entry point")


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("page_size,window", [(32, 45), (64, 64), (128, 500)])
def test_window_on_a_paged_cache(variant, page_size, window):
    w = Workload("win-pg", B=5, Hq=16, Hkv=2, D=128, Lmax=1000, seed=530 + page_size, len_lo=0, len_hi=1000)
    inp = window_inputs(w, window)
    ref = oracle.decode_window(inp["q"], inp["k"], inp["v"], inp["seq_lens"], window, inp["scale"])
    pg = to_dev(page_contiguous_cache(inp, page_size, seed=page_size, spare_pages=2))
    for chunk in (None, 128):
        print("case window paged", variant, page_size, window, chunk, flush=True)
        out = binding.decode_paged(pg["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], pg["seq_lens"],
                                   pg["scale"], variant=variant, chunk=chunk, window=window)
        torch.cuda.synchronize()
        check_close(out, ref, "window paged %s page %d W %d chunk %s" % (variant, page_size, window, chunk))


@pytest.mark.parametrize("name,window", [("ragged", 4096), ("palm", 1024), ("long", 8192)])
def test_window_full_size(name, window):
    w = WORKLOADS[name]
    print("case full window", name, window, flush=True)
    inp = make_inputs(w, device=DEV, poison_padding=w.ragged)
    lo = torch.clamp(inp["seq_lens"].to(torch.int64) - window, min=0).to(torch.int32)
    poison_positions_below_(inp["k"], lo)
    poison_positions_below_(inp["v"], lo)
    out = binding.decode_window(inp["q"], inp["k"], inp["v"], inp["seq_lens"], window, inp["scale"])
    torch.cuda.synchronize()
    ref = oracle.decode_window(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), window,
                               inp["scale"])
    err = check_close(out, ref, "%s window %d" % (name, window))
    print("full %s window %d: all %d sequences checked, max abs err %.3g" % (name, window, w.B, err), flush=True)


# ------------------------------------------------------ 8-bit KV cache

def quant_case(w: Workload, kv_format: str):
    """Seeded bf16 inputs, their 8-bit cache (NaN codes and scales past each length) and the oracle."""
    inp = make_inputs(w, poison_padding=True)
    qc = quantize_cache(inp, kv_format)
    ref = oracle.decode_quant(inp["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                              inp["seq_lens"], kv_format, inp["scale"])
    return to_dev(inp), to_dev(qc), ref


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G,Hkv,B", [(1, 2, 3), (4, 2, 4), (8, 1, 3), (48, 1, 3), (20, 2, 3)])
def test_quant_small_shapes(kv_format, variant, D, G, Hkv, B):
    w = Workload("q8", B=B, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=700, seed=700 + D + 7 * G + Hkv,
                 len_lo=0, len_hi=700)
    dev, qc, ref = quant_case(w, kv_format)
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case quant", kv_format, variant, D, G, Hkv, B, chunk, combine, flush=True)
        out = binding.decode_quant(dev["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                                   dev["seq_lens"], kv_format, dev["scale"], variant=variant, chunk=chunk,
                                   combine=combine)
        torch.cuda.synchronize()
        check_close(out, ref, "quant %s %s D %d G %d chunk %s %s" % (kv_format, variant, D, G, chunk, combine))


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("page_size", [32, 128])
def test_quant_paged(kv_format, variant, page_size):
    w = Workload("q8pg", B=5, Hq=16, Hkv=2, D=128, Lmax=1000, seed=760 + page_size, len_lo=0, len_hi=1000)
    inp = make_inputs(w, poison_padding=True)
    qc = quantize_cache(inp, kv_format)
    ref = oracle.decode_quant(inp["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                              inp["seq_lens"], kv_format, inp["scale"])
    pg = to_dev(page_quant_cache(inp, qc, page_size, seed=page_size, spare_pages=2))
    dev = to_dev(inp)
    for chunk in (None, 128):
        print("case quant paged", kv_format, variant, page_size, chunk, flush=True)
        out = binding.decode_paged(dev["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], dev["seq_lens"],
                                   dev["scale"], variant=variant, chunk=chunk, kv_format=kv_format,
                                   k_scale=pg["k_scale_pages"], v_scale=pg["v_scale_pages"])
        torch.cuda.synchronize()
        check_close(out, ref, "quant paged %s %s page %d chunk %s" % (kv_format, variant, page_size, chunk))


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("window", [1, 45, 300])
def test_quant_window(variant, window):
    """fp8 cache with a sliding window, against the oracle run on the window's rows moved to the front."""
    w = Workload("q8win", B=5, Hq=16, Hkv=2, D=128, Lmax=900, seed=780 + window, len_lo=0, len_hi=900)
    inp = make_inputs(w, poison_padding=True)
    qc = quantize_cache(inp, "fp8")
    lens = inp["seq_lens"]
    lo = torch.clamp(lens.to(torch.int64) - window, min=0)
    shifted = {key: torch.full_like(qc[key], 0x7F) for key in ("k_codes", "v_codes")}
    shifted.update({key: torch.full_like(qc[key], float("nan")) for key in ("k_scale", "v_scale")})
    for b in range(w.B):
        n, a0 = int(lens[b]), int(lo[b])
        for key in ("k_codes", "v_codes"):
            shifted[key][b, :n - a0] = qc[key][b, a0:n]
            qc[key][b, :a0] = 0x7F                       # positions before the window: NaN codes
        for key in ("k_scale", "v_scale"):
            shifted[key][b, :, :n - a0] = qc[key][b, :, a0:n]
            qc[key][b, :, :a0] = float("nan")
    ref = oracle.decode_quant(inp["q"], shifted["k_codes"], shifted["v_codes"], shifted["k_scale"],
                              shifted["v_scale"], (lens - lo).to(torch.int32), "fp8", inp["scale"])
    dev, dq = to_dev(inp), to_dev(qc)
    print("case quant window", variant, window, flush=True)
    out = binding.decode_quant(dev["q"], dq["k_codes"], dq["v_codes"], dq["k_scale"], dq["v_scale"],
                               dev["seq_lens"], "fp8", dev["scale"], variant=variant, window=window)
    torch.cuda.synchronize()
    check_close(out, ref, "quant window %s W %d" % (variant, window))


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("page_size,window", [(32, 45), (64, 300)])
def test_quant_paged_window(kv_format, variant, page_size, window):
    """8-bit codes in a paged pool with a sliding window: the oracle sees the window's rows moved to
    the front of a contiguous 8-bit cache; the pool holds the unshifted cache, whose positions before
    the window carry NaN codes and scales."""
    w = Workload("q8pgwin", B=5, Hq=16, Hkv=2, D=128, Lmax=900, seed=1100 + window + page_size, len_lo=0, len_hi=900)
    inp = make_inputs(w, poison_padding=True)
    qc = quantize_cache(inp, kv_format)
    lens = inp["seq_lens"]
    lo = torch.clamp(lens.to(torch.int64) - window, min=0)
    bad_code = 0x7F if kv_format == "fp8" else 0
    shifted = {key: torch.full_like(qc[key], bad_code) for key in ("k_codes", "v_codes")}
    shifted.update({key: torch.full_like(qc[key], float("nan")) for key in ("k_scale", "v_scale")})
    for b in range(w.B):
        n, a0 = int(lens[b]), int(lo[b])
        for key in ("k_codes", "v_codes"):
            shifted[key][b, :n - a0] = qc[key][b, a0:n]
            qc[key][b, :a0] = bad_code
        for key in ("k_scale", "v_scale"):
            shifted[key][b, :, :n - a0] = qc[key][b, :, a0:n]
            qc[key][b, :, :a0] = float("nan")       # positions before the window: NaN scales
    ref = oracle.decode_quant(inp["q"], shifted["k_codes"], shifted["v_codes"], shifted["k_scale"],
                              shifted["v_scale"], (lens - lo).to(torch.int32), kv_format, inp["scale"])
    pg = to_dev(page_quant_cache(inp, qc, page_size, seed=page_size + window, spare_pages=2))
    dev = to_dev(inp)
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case quant paged window", kv_format, variant, page_size, window, chunk, combine, flush=True)
        out = binding.decode_paged(dev["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], dev["seq_lens"],
                                   dev["scale"], variant=variant, chunk=chunk, combine=combine, window=window,
                                   kv_format=kv_format, k_scale=pg["k_scale_pages"], v_scale=pg["v_scale_pages"])
        torch.cuda.synchronize()
        check_close(out, ref, "quant paged window %s %s page %d W %d chunk %s %s"
                    % (kv_format, variant, page_size, window, chunk, combine))


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax,seed", _random_shapes(10, 2))
def test_quant_random_shapes(B, Hq, Hkv, D, Lmax, seed):
    """Seeded random shapes (groups 1..48, D 64..256, lengths 0..Lmax) on both 8-bit formats, with
    the planner's chunk, 128-position chunks and the fused merge (at most 8 chunks per sequence)."""
    kv_format = ("fp8", "int8")[seed % 2]
    w = Workload("q8rand", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=seed, len_lo=0, len_hi=Lmax)
    dev, qc, ref = quant_case(w, kv_format)
    fused_chunk = 128 * -(-Lmax // (8 * 128))
    for chunk, combine in ((None, None), (128, "separate"), (fused_chunk, "fused")):
        print("case quant random", kv_format, B, Hq, Hkv, D, Lmax, seed, chunk, combine, flush=True)
        out = binding.decode_quant(dev["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                                   dev["seq_lens"], kv_format, dev["scale"], chunk=chunk, combine=combine)
        torch.cuda.synchronize()
        check_close(out, ref, "quant random %s %s chunk %s %s" % (kv_format, (B, Hq, Hkv, D, Lmax), chunk, combine))


D256_LENS = [0, 1, 31, 32, 33, 63, 64, 65, 95, 129, 700]


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
@pytest.mark.parametrize("Hq", [16, 48, 64])
def test_quant_d256_steps_of_two_tiles(kv_format, Hq):
    """8-bit caches at D = 256: a compute step takes two 32-position tiles, and for up to 48 heads per
    block the two tiles go to two waves per 16-head tile whose softmax states merge after the loop
    (64 heads: one wave takes both).  Lengths sit on and around tile and step boundaries (a chunk of
    at most 32 positions, as in lengths 1, 32 and 129 with 128-position chunks, leaves the second
    wave nothing); the chunk is the default, or 128 positions with both merge forms; then a paged pool
    of 32-position pages (the two tiles of a step on different pages) with a window that is not a
    multiple of 32, and three query tokens per sequence."""
    w = Workload("q8d256", B=len(D256_LENS), Hq=Hq, Hkv=1, D=256, Lmax=704, seed=1200 + Hq)
    inp = make_inputs(w, seq_lens=D256_LENS, poison_padding=True)
    qc = quantize_cache(inp, kv_format)
    ref = oracle.decode_quant(inp["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                              inp["seq_lens"], kv_format, inp["scale"])
    dev, dq = to_dev(inp), to_dev(qc)
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case quant d256", kv_format, Hq, chunk, combine, flush=True)
        out = binding.decode_quant(dev["q"], dq["k_codes"], dq["v_codes"], dq["k_scale"], dq["v_scale"],
                                   dev["seq_lens"], kv_format, dev["scale"], variant="mfma", chunk=chunk,
                                   combine=combine)
        torch.cuda.synchronize()
        check_close(out, ref, "quant d256 %s Hq %d chunk %s %s" % (kv_format, Hq, chunk, combine))

    # paged pool of 32-position pages with a sliding window of 100 positions
    window = 100
    lens = inp["seq_lens"]
    lo = torch.clamp(lens.to(torch.int64) - window, min=0)
    bad_code = 0x7F if kv_format == "fp8" else 0
    shifted = {key: torch.full_like(qc[key], bad_code) for key in ("k_codes", "v_codes")}
    shifted.update({key: torch.full_like(qc[key], float("nan")) for key in ("k_scale", "v_scale")})
    wq = {key: qc[key].clone() for key in qc}
    for b in range(w.B):
        n, a0 = int(lens[b]), int(lo[b])
        for key in ("k_codes", "v_codes"):
            shifted[key][b, :n - a0] = qc[key][b, a0:n]
            wq[key][b, :a0] = bad_code
        for key in ("k_scale", "v_scale"):
            shifted[key][b, :, :n - a0] = qc[key][b, :, a0:n]
            wq[key][b, :, :a0] = float("nan")       # positions before the window: NaN scales
    ref_w = oracle.decode_quant(inp["q"], shifted["k_codes"], shifted["v_codes"], shifted["k_scale"],
                                shifted["v_scale"], (lens - lo).to(torch.int32), kv_format, inp["scale"])
    pg = to_dev(page_quant_cache(inp, wq, 32, seed=1200 + Hq, spare_pages=2))
    for chunk in (None, 128):
        print("case quant d256 paged window", kv_format, Hq, chunk, flush=True)
        out = binding.decode_paged(dev["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], dev["seq_lens"],
                                   dev["scale"], variant="mfma", chunk=chunk, window=window, kv_format=kv_format,
                                   k_scale=pg["k_scale_pages"], v_scale=pg["v_scale_pages"])
        torch.cuda.synchronize()
        check_close(out, ref_w, "quant d256 paged window %s Hq %d chunk %s" % (kv_format, Hq, chunk))

    # three query tokens per sequence, each an 8-bit decode with its own length
    T = 3
    wm = Workload("q8d256m", B=len(D256_LENS), Hq=Hq, Hkv=1, D=256, Lmax=704, seed=1250 + Hq)
    mi = make_multi_inputs(wm, T, seq_lens=D256_LENS, poison_padding=True)
    mq = quantize_cache(mi, kv_format)
    ml = mi["seq_lens"]
    ref_m = np.stack([oracle.decode_quant(mi["q"][:, i], mq["k_codes"], mq["v_codes"], mq["k_scale"], mq["v_scale"],
                                          torch.clamp(ml - T + 1 + i, min=0), kv_format, mi["scale"])
                      for i in range(T)], 1)
    md, mqd = to_dev(mi), to_dev(mq)
    for chunk in (None, 128):
        print("case quant d256 multi", kv_format, Hq, chunk, flush=True)
        out = binding.decode_multi(md["q"], mqd["k_codes"], mqd["v_codes"], md["seq_lens"], md["scale"],
                                   variant="mfma", chunk=chunk, kv_format=kv_format, k_scale=mqd["k_scale"],
                                   v_scale=mqd["v_scale"])
        torch.cuda.synchronize()
        check_close(out, ref_m, "quant d256 multi %s Hq %d chunk %s" % (kv_format, Hq, chunk))


@pytest.mark.parametrize("name,kv_format", [("palm", "fp8"), ("gqa70b", "fp8"), ("ragged", "fp8"), ("long", "fp8"),
                                            ("ragged", "int8"), ("palm", "int8"), ("long", "int8"), ("gqa70b", "int8")])
def test_quant_full_size(name, kv_format):
    w = WORKLOADS[name]
    print("case full quant", name, kv_format, flush=True)
    inp = make_inputs(w, device=DEV, poison_padding=w.ragged)
    qc = quantize_cache(inp, kv_format)
    del inp["k"], inp["v"]
    out = binding.decode_quant(inp["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                               inp["seq_lens"], kv_format, inp["scale"])
    torch.cuda.synchronize()
    ref = oracle.decode_quant(inp["q"].cpu(), qc["k_codes"].cpu(), qc["v_codes"].cpu(), qc["k_scale"].cpu(),
                              qc["v_scale"].cpu(), inp["seq_lens"].cpu(), kv_format, inp["scale"])
    err = check_close(out, ref, "%s %s" % (name, kv_format))
    print("full %s %s: all %d sequences checked, max abs err %.3g" % (name, kv_format, w.B, err), flush=True)


# ------------------------------------------------------ multi-token decode

@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("T,G,Hkv", [(2, 1, 2), (4, 4, 2), (8, 1, 1), (3, 8, 1), (2, 48, 1), (4, 20, 1)])
def test_multi_matches_multi_oracle(variant, D, T, G, Hkv):
    w = Workload("multi", B=4, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=600, seed=900 + D + 7 * G + T, len_lo=0, len_hi=600)
    inp = make_multi_inputs(w, T, poison_padding=True)
    ref = oracle.decode_multi(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    dev = to_dev(inp)
    for chunk, combine in ((None, None), (128, "separate"), (128, "fused")):
        print("case multi", variant, D, T, G, Hkv, chunk, combine, flush=True)
        out = binding.decode_multi(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], variant=variant,
                                   chunk=chunk, combine=combine)
        torch.cuda.synchronize()
        check_close(out, ref, "multi %s D %d T %d G %d chunk %s %s" % (variant, D, T, G, chunk, combine))


def test_multi_short_sequences_and_one_token():
    """Lengths below T (tokens before the start get zero rows), and T = 1 = the decode step bit for bit."""
    w = Workload("multi-short", B=6, Hq=16, Hkv=2, D=128, Lmax=300, seed=950)
    T = 6
    inp = make_multi_inputs(w, T)
    lens = torch.tensor([0, 1, 3, 5, 6, 300], dtype=torch.int32)
    from gqa_decode_attention_mqa_amd.workloads import poison_padding_
    poison_padding_(inp["k"], lens)
    poison_padding_(inp["v"], lens)
    ref = oracle.decode_multi(inp["q"], inp["k"], inp["v"], lens, inp["scale"])
    dev = to_dev(inp)
    dl = lens.to(DEV)
    for variant in ("mfma", "valu"):
        print("case multi short", variant, flush=True)
        out = binding.decode_multi(dev["q"], dev["k"], dev["v"], dl, dev["scale"], variant=variant, chunk=128)
        torch.cuda.synchronize()
        check_close(out, ref, "multi short %s" % variant)
        one = binding.decode_multi(dev["q"][:, :1].contiguous(), dev["k"], dev["v"], dl, dev["scale"], variant=variant)
        dec = binding.decode(dev["q"][:, 0].contiguous(), dev["k"], dev["v"], dl, dev["scale"], variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(one[:, 0], dec)


@pytest.mark.parametrize("variant", ["mfma", "valu"])
@pytest.mark.parametrize("combine", ["separate", "fused"])
def test_multi_tokens_before_the_start_of_a_split_sequence(variant, combine):
    """chunk < n < T: tokens i < T - n see no position in any of the sequence's chunks, so every chunk
    reports lse = -inf for them; the merge must write their rows as zeros (the oracle's and the
    header's contract), not NaN."""
    T = 600
    w = Workload("multi-split-short", B=3, Hq=8, Hkv=1, D=128, Lmax=1024, seed=970)
    inp = make_multi_inputs(w, T)
    lens = torch.tensor([500, 300, 1024], dtype=torch.int32)
    from gqa_decode_attention_mqa_amd.workloads import poison_padding_
    poison_padding_(inp["k"], lens)
    poison_padding_(inp["v"], lens)
    ref = oracle.decode_multi(inp["q"], inp["k"], inp["v"], lens, inp["scale"])
    assert (ref[0, :T - 500] == 0).all() and (ref[1, :T - 300] == 0).all()
    dev = to_dev(inp)
    print("case multi split short", variant, combine, flush=True)
    out = binding.decode_multi(dev["q"], dev["k"], dev["v"], lens.to(DEV), dev["scale"], variant=variant,
                               chunk=128, combine=combine)
    torch.cuda.synchronize()
    check_close(out, ref, "multi split short %s %s" % (variant, combine))
    assert torch.equal(out[0, :T - 500].cpu(), torch.zeros_like(out[0, :T - 500].cpu()))


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_multi_default_plan_with_tokens_before_the_start(variant):
    """The planner's own chunking (B=1, Hq=8, D=64, Lmax=2048, T=1500, n=1200 splits the sequence):
    tokens 0..299 have no visible position and must come back as zero rows."""
    T = 1500
    w = Workload("multi-plan-short", B=1, Hq=8, Hkv=1, D=64, Lmax=2048, seed=971)
    inp = make_multi_inputs(w, T)
    lens = torch.tensor([1200], dtype=torch.int32)
    from gqa_decode_attention_mqa_amd.workloads import poison_padding_
    poison_padding_(inp["k"], lens)
    poison_padding_(inp["v"], lens)
    plan = binding.plan(1, 8, 1, 64, 2048, inp["scale"], variant=variant, tokens=T)
    assert plan["max_splits"] > 1, plan
    ref = oracle.decode_multi(inp["q"], inp["k"], inp["v"], lens, inp["scale"])
    dev = to_dev(inp)
    print("case multi default plan short", variant, plan, flush=True)
    out = binding.decode_multi(dev["q"], dev["k"], dev["v"], lens.to(DEV), dev["scale"], variant=variant)
    torch.cuda.synchronize()
    check_close(out, ref, "multi default plan short %s" % variant)
    assert torch.equal(out[0, :300].cpu(), torch.zeros((300, 8, 64)))


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_multi_on_an_fp8_cache(variant):
    T = 4
    w = Workload("multi-q8", B=4, Hq=16, Hkv=4, D=128, Lmax=700, seed=960, len_lo=0, len_hi=700)
    inp = make_multi_inputs(w, T, poison_padding=True)
    qc = quantize_cache(inp, "fp8")
    # the oracle of several tokens on an 8-bit cache: each token is an 8-bit
    # decode with its own length (the pinned quantized decode)
    lens = inp["seq_lens"]
    ref = np.stack([oracle.decode_quant(inp["q"][:, i], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                                        torch.clamp(lens - T + 1 + i, min=0), "fp8", inp["scale"]) for i in range(T)], 1)
    dev, dq = to_dev(inp), to_dev(qc)
    print("case multi fp8", variant, flush=True)
    out = binding.decode_multi(dev["q"], dq["k_codes"], dq["v_codes"], dev["seq_lens"], dev["scale"], variant=variant,
                               kv_format="fp8", k_scale=dq["k_scale"], v_scale=dq["v_scale"])
    torch.cuda.synchronize()
    check_close(out, ref, "multi fp8 %s" % variant)


@pytest.mark.parametrize("name,T", [("ragged", 4), ("gqa70b", 4), ("palm", 2), ("long", 2)])
def test_multi_full_size(name, T):
    w = WORKLOADS[name]
    print("case full multi", name, T, flush=True)
    inp = make_multi_inputs(w, T, device=DEV, poison_padding=w.ragged)
    ref = oracle.decode_multi(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    # with the host copy of the lengths (the benchmark's plan) and without
    for h in (inp["seq_lens"].cpu(), None):
        out = binding.decode_multi(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], host_seq_lens=h)
        torch.cuda.synchronize()
        err = check_close(out, ref, "%s T=%d hint %s" % (name, T, h is not None))
        print("full %s T=%d hint %s: all %d sequences checked, max abs err %.3g" % (name, T, h is not None, w.B, err),
              flush=True)


# ------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("name,variant", [("tiny", None), ("palm", None), ("gqa70b", None), ("ragged", None),
                                          ("long", None), ("tiny", "valu"), ("gqa70b", "valu"), ("ragged", "valu")])
def test_full_size_workload(name, variant):
    """The five workloads at their full sizes, in the launch configuration the benchmark times
    (the planner's choice), every sequence against the oracle; the vector-ALU kernel also runs the
    small-group workloads (G = 8 and 4) at full size."""
    w = WORKLOADS[name]
    print("case full", name, variant, flush=True)
    inp = make_inputs(w, device=DEV, poison_padding=w.ragged)
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    # with the host copy of the lengths, as the benchmark plans it (a uniform
    # batch may then get other chunks), and without
    host = inp["seq_lens"].cpu()
    plans = {binding.plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, inp["scale"], variant, host_seq_lens=h)["chunk"]: h
             for h in (host, None)}
    for chunk, h in plans.items():
        out = binding.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"], variant=variant,
                             host_seq_lens=h)
        torch.cuda.synchronize()
        err = check_close(out, ref, "%s %s chunk %d" % (name, variant, chunk))
        print("full %s %s chunk %d: all %d sequences checked, max abs err %.3g" % (name, variant, chunk, w.B, err),
              flush=True)


@pytest.mark.parametrize("name", ["tiny", "palm", "ragged"])
def test_plain_entry_point(name):
    """mqa_decode_attention itself (no options): bit for bit the options form with NULL options,
    and within the bar of the oracle on every sequence."""
    w = WORKLOADS[name]
    print("case plain entry point", name, flush=True)
    inp = make_inputs(w, device=DEV, poison_padding=w.ragged)
    lib = binding.load_library()
    B, Hq, Hkv, D, Lmax = w.B, w.Hq, w.Hkv, w.D, w.Lmax
    plain = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ex = torch.empty_like(plain)
    sp = torch.cuda.current_stream(DEV).cuda_stream
    args = (inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(), inp["seq_lens"].data_ptr())
    st = lib.mqa_decode_attention(*args, plain.data_ptr(), B, Hq, Hkv, D, Lmax, inp["scale"], sp)
    assert st == 0, lib.mqa_last_error()
    st = lib.mqa_decode_attention_ex(*args, ex.data_ptr(), B, Hq, Hkv, D, Lmax, inp["scale"], sp, None)
    assert st == 0, lib.mqa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(plain, ex)
    ref = oracle.decode(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"])
    check_close(plain, ref, "plain entry point %s" % name)


# ------------------------------------------------------ persistent schedule

PERSIST_CASES = {
    # 40 sequences x 8 kv heads x 16 chunks of 128 = 5120 items: persistent by default
    "gqa": Workload("persist-gqa", B=40, Hq=32, Hkv=8, D=128, Lmax=2000, seed=1300, len_lo=0, len_hi=2000),
    # MQA at D = 256 (one workgroup per CU), forced persistent
    "mqa": Workload("persist-mqa", B=12, Hq=48, Hkv=1, D=256, Lmax=1500, seed=1301, len_lo=1, len_hi=1500),
}


@pytest.mark.parametrize("case", sorted(PERSIST_CASES))
def test_persistent_schedule_gives_the_per_item_bits(case):
    """Workgroups that take work items from a queue compute each item exactly as one workgroup per item
    does: bf16, an 8-bit cache, a paged pool, a window and two query tokens, each bit for bit, and the
    oracle's values; repeated calls find the queue back at zero."""
    w = PERSIST_CASES[case]
    inp = make_inputs(w, poison_padding=True)
    dev = to_dev(inp)
    ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    for rep in range(3):
        print("case persistent bf16", case, rep, flush=True)
        outs = {s: binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], chunk=128,
                                  schedule=s) for s in ("per_item", "persistent", None)}
        torch.cuda.synchronize()
        assert torch.equal(outs["persistent"], outs["per_item"]) and torch.equal(outs[None], outs["per_item"])
        check_close(outs["persistent"], ref, "persistent %s" % case)

    qc = quantize_cache(inp, "fp8")
    dq = to_dev(qc)
    ref8 = oracle.decode_quant(inp["q"], qc["k_codes"], qc["v_codes"], qc["k_scale"], qc["v_scale"],
                               inp["seq_lens"], "fp8", inp["scale"])
    print("case persistent fp8", case, flush=True)
    o8 = {s: binding.decode_quant(dev["q"], dq["k_codes"], dq["v_codes"], dq["k_scale"], dq["v_scale"],
                                  dev["seq_lens"], "fp8", dev["scale"], chunk=128, schedule=s)
          for s in ("per_item", "persistent")}
    torch.cuda.synchronize()
    assert torch.equal(o8["persistent"], o8["per_item"])
    check_close(o8["persistent"], ref8, "persistent fp8 %s" % case)

    pg = to_dev(page_contiguous_cache(inp, 64, seed=1302))
    print("case persistent paged window", case, flush=True)
    op = {s: binding.decode_paged(dev["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], dev["seq_lens"],
                                  dev["scale"], chunk=128, window=300, schedule=s) for s in ("per_item", "persistent")}
    ow = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], chunk=128, window=300,
                        schedule="per_item")
    torch.cuda.synchronize()
    assert torch.equal(op["persistent"], op["per_item"]) and torch.equal(op["persistent"], ow)

    T = 2
    mi = make_multi_inputs(w, T, seed=1303, poison_padding=True)
    md = to_dev(mi)
    refm = oracle.decode_multi(mi["q"], mi["k"], mi["v"], mi["seq_lens"], mi["scale"])
    print("case persistent multi", case, flush=True)
    om = {s: binding.decode_multi(md["q"], md["k"], md["v"], md["seq_lens"], md["scale"], chunk=128, schedule=s)
          for s in ("per_item", "persistent")}
    torch.cuda.synchronize()
    assert torch.equal(om["persistent"], om["per_item"])
    check_close(om["persistent"], refm, "persistent multi %s" % case)


def test_persistent_schedule_with_fewer_items_than_workgroups_and_a_larger_grid_after():
    """Two items (fewer than the resident workgroups), then a grid of thousands: the queue left by
    each call is back at zero for the next."""
    small = Workload("persist-small", B=1, Hq=8, Hkv=2, D=64, Lmax=100, seed=1304, len_lo=1, len_hi=100)
    big = PERSIST_CASES["gqa"]
    for w in (small, big, small, big):
        inp = make_inputs(w, poison_padding=True)
        dev = to_dev(inp)
        print("case persistent sequence", w.name, flush=True)
        out = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], chunk=128,
                             schedule="persistent")
        torch.cuda.synchronize()
        ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
        check_close(out, ref, "persistent %s" % w.name)


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax,seed", _random_shapes(10, 3))
def test_random_shapes_persistent(B, Hq, Hkv, D, Lmax, seed):
    """Seeded random shapes run persistent (forced: most of them have fewer items than resident
    workgroups), bit for bit the per-item result, and within the oracle's tolerance."""
    w = Workload("rand-persist", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, seed=seed, len_lo=0, len_hi=Lmax)
    inp = make_inputs(w, poison_padding=True)
    dev = to_dev(inp)
    ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    for chunk in (None, 128):
        print("case random persistent", B, Hq, Hkv, D, Lmax, seed, chunk, flush=True)
        outs = [binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], chunk=chunk,
                               variant="mfma", schedule=s) for s in ("per_item", "persistent")]
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        check_close(outs[1], ref, "random persistent chunk %s" % chunk)


def test_persistent_schedule_with_several_head_blocks():
    """Items cover head blocks too (item = head block * grid_x + x): 128 heads per kv head take two
    blocks of 96 and 32 rows, and two query tokens of 64 heads the same."""
    w = Workload("persist-hb", B=3, Hq=128, Hkv=1, D=128, Lmax=1000, seed=1310, len_lo=1, len_hi=1000)
    assert binding.plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, chunk=128, schedule="persistent")["head_blocks"] == 2
    inp = make_inputs(w, poison_padding=True)
    dev = to_dev(inp)
    ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["scale"])
    print("case persistent head blocks", flush=True)
    outs = [binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"], chunk=128, schedule=s)
            for s in ("per_item", "persistent")]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    check_close(outs[1], ref, "persistent head blocks")
    wm = Workload("persist-hb-multi", B=3, Hq=64, Hkv=1, D=128, Lmax=1000, seed=1311, len_lo=1, len_hi=1000)
    mi = make_multi_inputs(wm, 2, poison_padding=True)
    md = to_dev(mi)
    refm = oracle.decode_multi(mi["q"], mi["k"], mi["v"], mi["seq_lens"], mi["scale"])
    print("case persistent head blocks multi", flush=True)
    om = [binding.decode_multi(md["q"], md["k"], md["v"], md["seq_lens"], md["scale"], chunk=128, schedule=s)
          for s in ("per_item", "persistent")]
    torch.cuda.synchronize()
    assert torch.equal(om[0], om[1])
    check_close(om[1], refm, "persistent head blocks multi")
