"""CPU tests of the C ABI's host side: symbols, argument checks and planning.

No GPU is needed: every check in the library runs on the host before any HIP
call, and mqa_decode_plan makes no HIP call at all.  Calls here only use
invalid arguments (or NULL data with B == 0), so nothing is ever launched.
"""
import ctypes
import math

import pytest
import torch

from gqa_decode_attention_mqa_amd import binding

lib = binding.load_library()

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_ARG = range(8)


def test_every_declared_symbol_is_exported():
    names = binding.declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for s in range(8):
        assert lib.mqa_status_string(s)
    assert lib.mqa_status_string(99) == b"unknown status"
    assert lib.mqa_version() == 10600  # 1.6.0, as MAJOR*10000 + MINOR*100 + PATCH


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its checks first


def call(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, D=128, Lmax=64, scale=0.1, opts=None):
    return lib.mqa_decode_attention_ex(q, k, v, lens, out, B, Hq, Hkv, D, Lmax, scale, None,
                                       ctypes.byref(opts) if opts is not None else None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), ERR_NULL), (dict(k=0), ERR_NULL), (dict(v=0), ERR_NULL),
    (dict(lens=0), ERR_NULL), (dict(out=0), ERR_NULL),
    (dict(Hq=7), ERR_SHAPE), (dict(Hkv=0), ERR_SHAPE), (dict(Hq=0), ERR_SHAPE),
    (dict(B=-1), ERR_SHAPE), (dict(Lmax=-3), ERR_SHAPE), (dict(D=0), ERR_SHAPE),
    (dict(D=96), ERR_UNSUPPORTED), (dict(D=512), ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), ERR_ALIGN), (dict(k=FAKE + 2), ERR_ALIGN), (dict(out=FAKE + 4), ERR_ALIGN),
    (dict(lens=FAKE + 2), ERR_ALIGN),
    (dict(scale=math.inf), ERR_ARG), (dict(scale=math.nan), ERR_ARG),
])
def test_invalid_arguments_are_rejected_before_any_hip_call(kw, expect):
    assert call(**kw) == expect
    assert lib.mqa_last_error()


@pytest.mark.parametrize("opts,expect", [
    (dict(variant=3), ERR_ARG), (dict(variant=-1), ERR_ARG),
    (dict(chunk=100), ERR_ARG), (dict(chunk=-128), ERR_ARG),
    (dict(combine=5), ERR_ARG), (dict(combine=-1), ERR_ARG),
])
def test_invalid_options_are_rejected(opts, expect):
    assert call(opts=binding.make_opts(**opts)) == expect


def test_fused_combine_is_refused_beyond_its_split_limit():
    # 100000 positions in chunks of 128 -> 782 chunks > 8
    assert call(Lmax=100000, opts=binding.make_opts(chunk=128, combine=2)) == ERR_ARG
    assert call(Lmax=1025, opts=binding.make_opts(chunk=128, combine=2)) == ERR_ARG  # 9 chunks
    assert binding.plan(2, 8, 2, 128, 100000, chunk=128)["combine"] == 1
    assert binding.plan(2, 8, 2, 128, 1024, chunk=128, combine="fused")["combine"] == 2


def test_empty_batch_is_a_no_op_even_with_null_pointers():
    assert call(q=0, k=0, v=0, lens=0, out=0, B=0) == OK
    assert lib.mqa_prefill_attention(0, 0, 0, 0, 0, 0, 8, 1, 64, 16, 0.125, None) == OK


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax", [(64, 48, 1, 256, 2048), (32, 64, 8, 128, 4096), (2, 3, 3, 64, 700),
                                              (3, 40, 2, 128, 97), (1, 112, 1, 64, 1)])
def test_prefill_plan_covers_every_row(B, Hq, Hkv, D, Lmax):
    """One workgroup per block of query rows of each (sequence, kv head), the blocks covering all
    Lmax * G rows, whole waves per workgroup, no workspace."""
    p = binding.prefill_plan(B, Hq, Hkv, D, Lmax, 0.1)
    rows, G = p["rows_per_block"], Hq // Hkv
    assert rows > 0 and rows % 16 == 0
    blocks = -(-Lmax * G // rows)
    assert p["grid_main"] == B * Hkv * blocks and (blocks - 1) * rows < Lmax * G <= blocks * rows
    assert p["block_main"] % 64 == 0 and 64 <= p["block_main"] <= 1024
    assert p["workspace_bytes"] == 0 and p["max_splits"] == 1


def test_prefill_checks_arguments_too():
    assert lib.mqa_prefill_attention(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 6, 4, 64, 16, 0.1, None) == ERR_SHAPE


@pytest.mark.parametrize("B,Hq,Hkv,D,Lmax", [
    (1, 8, 1, 64, 128), (64, 48, 1, 256, 2048), (32, 64, 8, 128, 4096),
    (256, 32, 8, 128, 8192), (4, 48, 1, 256, 131072), (3, 80, 1, 128, 1000), (2, 6, 2, 64, 1),
    (5, 8, 8, 256, 0),
])
def test_plan_invariants(B, Hq, Hkv, D, Lmax):
    p = binding.plan(B, Hq, Hkv, D, Lmax)
    G = Hq // Hkv
    assert p["chunk"] > 0 and p["chunk"] % 128 == 0
    assert p["max_splits"] >= 1 and p["chunk"] * p["max_splits"] >= Lmax
    assert (p["max_splits"] - 1) * p["chunk"] < max(Lmax, 1)
    assert p["variant"] == "mfma"  # the matrix-core kernel serves every group by default
    per_block = min(G, 96) if p["variant"] == "mfma" else min(G, 8)
    assert p["head_blocks"] * per_block >= G
    assert p["grid_main"] == B * Hkv * p["max_splits"] * p["head_blocks"]
    # matrix cores: a compute wave per 16 heads and two load-only waves; vector ALU: four waves
    assert p["block_main"] == (64 * (-(-per_block // 16) + 2) if p["variant"] == "mfma" else 256)
    if p["max_splits"] > 1:
        assert p["combine"] == 1
        if p["max_splits"] <= 8:   # few chunks: one thread per (head, 8 columns), 2048/D heads per block
            assert p["grid_combine"] == B * Hkv * -(-G // (2048 // D))  # whole head blocks per unit
        else:                      # many chunks: 1 .. D/64 workgroups per (row, head), a slice of d each
            ds = p["grid_combine"] // (B * Hq)
            assert p["grid_combine"] == B * Hq * ds and ds in (1, 2, 4) and ds <= max(1, D // 64)
            assert ds == 1 or B * Hq * ds // 2 < 256  # slices only while the grid is below the CUs
        # fp16 partial rows plus an {lse, exponent} float pair per (chunk, head)
        assert p["workspace_bytes"] >= B * Hkv * p["max_splits"] * G * (2 * D + 8)
    else:
        assert p["combine"] == 0 and p["workspace_bytes"] == 0


def test_forced_variant_and_chunk_are_honoured():
    p = binding.plan(4, 8, 1, 128, 1000, variant="mfma", chunk=256)
    assert p["variant"] == "mfma" and p["chunk"] == 256 and p["max_splits"] == 4
    p = binding.plan(4, 48, 1, 256, 1000, variant="valu")
    assert p["variant"] == "valu" and p["head_blocks"] == 6


def test_block_size_counts_the_compute_and_load_waves():
    """One compute wave per 16 heads plus two loaders; 8-bit caches at D = 256
    with up to 48 heads per block give each 16-head tile two compute waves."""
    assert binding.plan(64, 48, 1, 256, 2048)["block_main"] == 64 * (3 + 2)
    for fmt in ("fp8", "int8"):
        assert binding.plan(64, 48, 1, 256, 2048, kv_format=fmt)["block_main"] == 64 * (6 + 2)
        assert binding.plan(4, 16, 1, 256, 4096, kv_format=fmt)["block_main"] == 64 * (2 + 2)
        assert binding.plan(32, 64, 8, 128, 4096, kv_format=fmt)["block_main"] == 64 * (1 + 2)
    p = binding.plan(2, 96, 1, 256, 4096, kv_format="fp8")  # 96 heads per block: one wave per tile
    assert p["head_blocks"] == 1 and p["block_main"] == 64 * (6 + 2)
    assert binding.plan(32, 64, 8, 128, 4096)["block_main"] == 64 * (1 + 2)


def test_default_plans_of_the_five_workloads():
    """The defaults are the measured best choices on MI355X."""
    assert binding.plan(64, 48, 1, 256, 2048)["chunk"] == 512
    assert binding.plan(4, 48, 1, 256, 131072)["chunk"] == 2048
    g = binding.plan(32, 64, 8, 128, 4096)
    assert g["variant"] == "mfma" and g["chunk"] == 2048
    r = binding.plan(256, 32, 8, 128, 8192)
    assert r["variant"] == "mfma" and r["chunk"] == 1024
    assert binding.plan(1, 8, 1, 64, 128)["max_splits"] == 1


def test_host_lengths_choose_coarse_chunks_for_uniform_batches():
    """With a host copy of the lengths the planner tells a uniform batch from a ragged one: uniform
    on a bf16 cache gets about one chunk per CU, up to whole sequences; 8-bit caches and ragged
    batches keep the short chunks.  The chunks always cover Lmax (or the window)."""
    full = lambda B, n: torch.full((B,), n, dtype=torch.int32)
    g = binding.plan(32, 64, 8, 128, 4096, host_seq_lens=full(32, 4096))
    assert g["chunk"] == 4096 and g["max_splits"] == 1 and g["grid_combine"] == 0
    assert binding.plan(32, 64, 8, 128, 4096, host_seq_lens=full(32, 4096), tokens=4)["chunk"] == 4096
    assert binding.plan(32, 64, 8, 128, 4096, kv_format="fp8", host_seq_lens=full(32, 4096))["chunk"] == 2048
    assert binding.plan(32, 64, 8, 128, 4096, kv_format="int8", host_seq_lens=full(32, 4096))["chunk"] == 2048
    assert binding.plan(16, 48, 1, 256, 131072, host_seq_lens=full(16, 131072))["chunk"] == 8192
    assert binding.plan(64, 48, 1, 256, 2048, host_seq_lens=full(64, 2048))["chunk"] == 512  # unchanged
    assert binding.plan(4, 48, 1, 256, 131072, host_seq_lens=full(4, 131072))["chunk"] == 2048
    gen = torch.Generator().manual_seed(5)
    ragged = torch.randint(1, 4097, (32,), generator=gen, dtype=torch.int32)
    assert binding.plan(32, 64, 8, 128, 4096, host_seq_lens=ragged)["chunk"] == 1024  # 256 units, ragged
    assert binding.plan(16, 64, 8, 128, 4096, host_seq_lens=ragged[:16])["chunk"] == 2048  # 128 units
    big = torch.randint(1, 8193, (256,), generator=gen, dtype=torch.int32)
    assert binding.plan(256, 32, 8, 128, 8192, host_seq_lens=big)["chunk"] == 1024
    # lengths within one quantum of each other count as uniform; a shorter batch keeps Lmax covered
    near = full(32, 4000)
    near[3] = 3900
    p = binding.plan(32, 64, 8, 128, 8192, host_seq_lens=near)
    assert p["chunk"] == 4096 and p["chunk"] * p["max_splits"] >= 8192
    w = binding.plan(32, 64, 8, 128, 8192, window=1024, host_seq_lens=full(32, 8000))
    assert w["chunk"] * w["max_splits"] >= 1024
    with pytest.raises(ValueError):  # the binding checks the count before the planner reads B values
        binding._checked_lens(full(31, 4096), 32)


def test_chunk_schedule_covers_every_valid_position_once():
    """The split kernel gives workgroup (unit, s) positions [s*chunk, min((s+1)*chunk, len))."""
    Lmax = 8192
    p = binding.plan(256, 32, 8, 128, Lmax)
    C, S = p["chunk"], p["max_splits"]
    assert C == 1024  # many units: short matrix-core chunks
    for n in [0, 1, 127, 128, 129, C - 1, C, C + 1, Lmax - 1, Lmax]:
        seen = []
        for s in range(S):
            p0 = s * C
            if s > 0 and p0 >= n:
                continue
            seen.extend(range(p0, min(p0 + C, n)))
        assert seen == list(range(n))


@pytest.mark.parametrize("window", [1, 31, 32, 33, 100, 1000, 4096, 8191, 8192, 9000])
def test_window_schedule_covers_the_window_once(window):
    """With a window W the split kernels start chunk s at base + s*chunk, where
    base is the first attended position lo = max(0, n - W) rounded down to a
    multiple of 32, mask positions below lo, and let the last of the plan's
    chunks run to n.  Every position of [lo, n) must fall in exactly one chunk,
    chunk starts must stay 32-aligned (tiles and pages), and no chunk may hold
    more than chunk + 31 positions."""
    Lmax = 8192
    p = binding.plan(256, 32, 8, 128, Lmax, window=window)
    C, S = p["chunk"], p["max_splits"]
    assert S == -(-min(Lmax, window) // C)
    for n in sorted({0, 1, 31, 32, 33, window - 1, window, window + 1, window + 31, window + 32,
                     Lmax - 33, Lmax - 1, Lmax} & set(range(0, Lmax + 1))):
        lo = max(0, n - window)
        base = lo & ~31
        nsplit = min(-(-(n - base) // C) if n > base else 1, S)
        seen = []
        for s in range(S):
            p0 = base + s * C
            assert p0 % 32 == 0
            if s > 0 and p0 >= n:
                continue
            p1 = n if s == S - 1 else min(p0 + C, n)
            assert s < nsplit or n == 0
            assert p1 - p0 <= C + 31
            seen.extend(t for t in range(p0, p1) if t >= lo)
        assert seen == list(range(lo, n))


def test_window_arguments():
    assert lib.mqa_decode_attention_window(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0, 0.1, None) == ERR_ARG
    assert lib.mqa_decode_attention_window(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, -5, 0.1, None) == ERR_ARG
    assert b"window" in lib.mqa_last_error()
    with pytest.raises(binding.MqaError):
        binding.plan(2, 8, 2, 128, 64, window=-1)
    # a window of at least Lmax plans exactly like no window
    assert binding.plan(8, 32, 8, 128, 4096, window=4096) == binding.plan(8, 32, 8, 128, 4096)
    assert binding.plan(8, 32, 8, 128, 4096, window=1 << 30) == binding.plan(8, 32, 8, 128, 4096)
    assert binding.plan(2, 8, 1, 64, 600, window=600) == binding.plan(2, 8, 1, 64, 600)
    # chunks sized for the window itself: PaLM-shaped batch, W = 1024 -> four 256-position chunks
    p = binding.plan(64, 48, 1, 256, 2048, window=1024)
    assert p["chunk"] == 256 and p["max_splits"] == 4
    # the window bounds the grid: 8 chunks of 512 without it, 1 with W = 512 (the
    # last chunk absorbs the window start's alignment to 32)
    assert binding.plan(64, 48, 1, 256, 4096, chunk=512)["max_splits"] == 8
    assert binding.plan(64, 48, 1, 256, 4096, chunk=512, window=512)["max_splits"] == 1


def quant_call(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lens=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, D=128, Lmax=64,
               fmt=1, scale=0.1, opts=None):
    return lib.mqa_decode_attention_quant(q, k, v, ks, vs, lens, out, B, Hq, Hkv, D, Lmax, fmt, scale, None, opts)


@pytest.mark.parametrize("kw,expect", [
    (dict(fmt=0), ERR_ARG), (dict(fmt=3), ERR_ARG), (dict(fmt=-1), ERR_ARG),
    (dict(ks=0), ERR_NULL), (dict(vs=0), ERR_NULL), (dict(ks=FAKE + 2), ERR_ALIGN), (dict(vs=FAKE + 1), ERR_ALIGN),
    (dict(k=0), ERR_NULL), (dict(k=FAKE + 8), ERR_ALIGN), (dict(Hq=7), ERR_SHAPE), (dict(D=96), ERR_UNSUPPORTED),
    (dict(fmt=2, ks=0), ERR_NULL),
])
def test_quant_arguments_are_rejected_before_any_hip_call(kw, expect):
    # every other argument is valid, and B = 2, so the call would launch if the checks passed
    assert quant_call(**kw) == expect
    assert lib.mqa_last_error()


def test_quant_empty_batch_and_cache_need_no_scales():
    assert quant_call(q=0, k=0, v=0, ks=0, vs=0, lens=0, out=0, B=0) == OK


def test_quant_plan():
    with pytest.raises(binding.MqaError):
        binding.plan(2, 8, 2, 128, 64, kv_format=3)
    # 8-bit caches hold twice the columns per lane in the vector kernel: at most 4 heads per block
    p = binding.plan(4, 16, 2, 128, 512, variant="valu", kv_format="fp8")
    assert p["head_blocks"] == 2 and p["block_main"] == 256
    assert binding.plan(4, 16, 2, 128, 512, variant="valu")["head_blocks"] == 1
    # the matrix-core plan depends on the format only through the workgroup
    # size (two compute waves per 16-head tile on 8-bit caches at D = 256)
    a = binding.plan(64, 48, 1, 256, 2048, kv_format="fp8")
    b = binding.plan(64, 48, 1, 256, 2048)
    assert a.pop("block_main") == 512 and b.pop("block_main") == 320
    assert a == b


def multi_call(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, T=4, Hq=8, Hkv=2, D=128, Lmax=64, scale=0.1,
               opts=None):
    return lib.mqa_decode_attention_multi(q, k, v, lens, out, B, T, Hq, Hkv, D, Lmax, scale, None, opts)


@pytest.mark.parametrize("kw,expect", [
    (dict(T=0), ERR_SHAPE), (dict(T=-2), ERR_SHAPE), (dict(T=1 << 15, Hq=64, D=256), ERR_UNSUPPORTED),
    (dict(opts=binding.make_opts(window=16)), ERR_ARG), (dict(q=0), ERR_NULL), (dict(Hq=7), ERR_SHAPE),
    (dict(opts=binding.make_opts(kv_format="fp8")), ERR_NULL),
])
def test_multi_arguments_are_rejected_before_any_hip_call(kw, expect):
    if "opts" in kw:
        kw["opts"] = binding.ctypes.byref(kw["opts"])
    assert multi_call(**kw) == expect
    assert lib.mqa_last_error()


def test_multi_plan_fills_tiles_with_tokens():
    # four tokens of a 4-head group make a full 16-row tile
    p = binding.plan(256, 32, 8, 128, 8192, tokens=4)
    assert p["variant"] == "mfma" and p["head_blocks"] == 1 and p["block_main"] == 64 * 3
    # 2 tokens x 48 heads = 96 query rows: one block of six 16-row tiles (six compute waves)
    p = binding.plan(64, 48, 1, 256, 2048, tokens=2)
    assert p["head_blocks"] == 1 and p["block_main"] == 64 * (6 + 2)
    # 3 tokens x 48 heads = 144 rows: two blocks of up to 96
    assert binding.plan(64, 48, 1, 256, 2048, tokens=3)["head_blocks"] == 2
    # the combine covers every (row, token, head)
    p = binding.plan(8, 16, 2, 128, 4096, tokens=3, chunk=512)
    assert p["grid_combine"] == 8 * 2 * -(-3 * 8 // (2048 // 128))  # per unit: T * G = 24 query rows
    assert p["workspace_bytes"] >= 8 * 2 * p["max_splits"] * 24 * (2 * 128 + 8)


def test_multi_empty_batch_is_a_no_op():
    assert multi_call(q=0, k=0, v=0, lens=0, out=0, B=0) == OK


def paged_call(q=FAKE, k=FAKE, v=FAKE, table=FAKE, lens=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, D=128,
               num_pages=16, page_size=64, max_blocks=4, scale=0.1):
    return lib.mqa_decode_attention_paged(q, k, v, table, lens, out, B, Hq, Hkv, D, num_pages, page_size,
                                          max_blocks, scale, None, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(page_size=48), ERR_UNSUPPORTED), (dict(page_size=16), ERR_UNSUPPORTED), (dict(page_size=96), ERR_UNSUPPORTED),
    (dict(page_size=0), ERR_SHAPE), (dict(page_size=-64), ERR_SHAPE),
    (dict(num_pages=-1), ERR_SHAPE), (dict(max_blocks=-1), ERR_SHAPE), (dict(num_pages=0), ERR_SHAPE),
    (dict(table=0), ERR_NULL), (dict(table=FAKE + 2), ERR_ALIGN),
    (dict(page_size=1 << 20, max_blocks=1 << 12), ERR_UNSUPPORTED),
    (dict(k=0), ERR_NULL), (dict(q=FAKE + 8), ERR_ALIGN), (dict(Hq=7), ERR_SHAPE), (dict(D=96), ERR_UNSUPPORTED),
])
def test_paged_arguments_are_rejected_before_any_hip_call(kw, expect):
    assert paged_call(**kw) == expect
    assert lib.mqa_last_error()


def test_paged_empty_batch_is_a_no_op():
    assert paged_call(q=0, k=0, v=0, table=0, lens=0, out=0, B=0) == OK


# ------------------------------------------------ the no-allocation entry point

NOALLOC_SCRATCH = 32 * 1024 * 1024


def call_noalloc(B=2, Hq=8, Hkv=2, D=128, Lmax=64, opts=None, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.mqa_decode_attention_noalloc(p["q"], p["k"], p["v"], p["lens"], p["out"], B, Hq, Hkv, D, Lmax, 0.1,
                                            None, ctypes.byref(opts) if opts is not None else None)


def test_noalloc_scratch_limit_matches_the_header():
    text = binding.HEADER_PATH.read_text()
    assert "#define MQA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)" in text


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    # B=256, Hkv=8, 32 heads, D=256, 131072 positions in 128-position chunks:
    # 256 * 8 * 1024 chunks * 4 heads * 256 * 2 bytes of partials, far beyond 32 MiB
    opts = binding.make_opts(chunk=128)
    need = binding.plan(256, 32, 8, 256, 131072, chunk=128)["workspace_bytes"]
    assert need > NOALLOC_SCRATCH
    assert call_noalloc(B=256, Hq=32, Hkv=8, D=256, Lmax=131072, opts=opts) == ERR_WORKSPACE
    assert b"no-allocation" in lib.mqa_last_error()


def test_noalloc_accepts_what_fits_and_checks_like_the_options_form():
    # the five workloads' plans all fit the scratch
    for B, Hq, Hkv, D, Lmax in ((1, 8, 1, 64, 128), (64, 48, 1, 256, 2048), (32, 64, 8, 128, 4096),
                                (256, 32, 8, 128, 8192), (4, 48, 1, 256, 131072)):
        assert binding.plan(B, Hq, Hkv, D, Lmax)["workspace_bytes"] <= NOALLOC_SCRATCH
    # the same argument errors as mqa_decode_attention_ex, before any HIP call
    assert call_noalloc(q=0) == ERR_NULL
    assert call_noalloc(Hq=7) == ERR_SHAPE
    assert call_noalloc(D=96) == ERR_UNSUPPORTED
    assert call_noalloc(out=FAKE + 4) == ERR_ALIGN
    assert call_noalloc(B=0, q=0, k=0, v=0, lens=0, out=0) == OK


def test_noalloc_refuses_the_fused_merge():
    assert call_noalloc(Lmax=1024, opts=binding.make_opts(chunk=128, combine=2)) == ERR_ARG
    assert b"separate combine" in lib.mqa_last_error()


# ------------------------------------------------ the streaming-read probe (calibration)

@pytest.mark.parametrize("args,expect", [
    ((0, 1 << 20, 256, FAKE), ERR_NULL), ((FAKE, 1 << 20, 256, 0), ERR_NULL),
    ((FAKE + 8, 1 << 20, 256, FAKE), ERR_ALIGN), ((FAKE, (1 << 20) + 4, 256, FAKE), ERR_ALIGN),
    ((FAKE, 1 << 20, 256, FAKE + 2), ERR_ALIGN),
    ((FAKE, 1 << 20, 0, FAKE), ERR_ARG), ((FAKE, 1 << 20, (1 << 24) + 1, FAKE), ERR_ARG),
    ((FAKE, 4 << 30, 2, FAKE), ERR_UNSUPPORTED),
])
def test_stream_read_probe_checks_its_arguments(args, expect):
    buf, nbytes, wgs, sink = args
    assert lib.mqa_stream_read_probe(buf, nbytes, wgs, sink, None, None, None) == expect
    assert lib.mqa_last_error()


def test_stream_read_probe_of_nothing_is_a_no_op():
    assert lib.mqa_stream_read_probe(0, 0, 1, 0, None, None, None) == OK


# ------------------------------------------------ workspace allocation failure

def test_workspace_allocation_failure_is_reported(monkeypatch):
    """MQA_FAIL_WORKSPACE_ALLOC=1 makes the split workspace allocation fail (before any HIP call):
    a split call reports MQA_ERR_WORKSPACE with a message; calls that need no workspace are unaffected."""
    monkeypatch.setenv("MQA_FAIL_WORKSPACE_ALLOC", "1")
    opts = binding.make_opts(chunk=128)
    assert binding.plan(2, 8, 2, 128, 4096, chunk=128)["workspace_bytes"] > 0
    assert call(Lmax=4096, opts=opts) == ERR_WORKSPACE
    assert b"workspace" in lib.mqa_last_error()
    assert lib.mqa_decode_attention_multi(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3, 8, 2, 128, 4096, 0.1, None,
                                          ctypes.byref(opts)) == ERR_WORKSPACE
    # B == 0 never allocates
    assert call(q=0, k=0, v=0, lens=0, out=0, B=0, Lmax=4096, opts=opts) == OK


def test_persistent_schedule_for_grids_of_many_items():
    """The planner runs the split kernel persistent (a resident grid taking work items from a queue)
    for grids of at least 2048 items, and one workgroup per item otherwise."""
    ragged = binding.plan(256, 32, 8, 128, 8192)
    assert ragged["persistent"] and ragged["grid_main"] >= 2048
    assert binding.plan(256, 32, 8, 128, 8192, kv_format="fp8")["persistent"]
    assert binding.plan(256, 32, 8, 128, 8192, window=4096)["persistent"]
    for shape in ((64, 48, 1, 256, 2048), (4, 48, 1, 256, 131072), (32, 64, 8, 128, 4096), (1, 8, 1, 64, 128)):
        p = binding.plan(*shape)
        assert not p["persistent"] and p["grid_main"] < 2048, shape
    # the fused merge and the vector kernel run one workgroup per item
    assert not binding.plan(256, 32, 8, 128, 1024, chunk=128, combine="fused")["persistent"]
    assert not binding.plan(256, 32, 8, 128, 8192, variant="valu")["persistent"]
    # forced either way; the rest of the plan does not change
    a = binding.plan(256, 32, 8, 128, 8192, schedule="per_item")
    b = binding.plan(256, 32, 8, 128, 8192, schedule="persistent")
    assert not a.pop("persistent") and b.pop("persistent")
    assert a.pop("workspace_bytes") == b.pop("workspace_bytes") and a == b
    assert binding.plan(64, 48, 1, 256, 2048, schedule="persistent")["persistent"]


def test_persistent_schedule_stays_within_its_32_bit_queue():
    """A grid of 2^31 items or more (here 2^24 - 1 split workgroups times 129 head blocks) runs one
    workgroup per item; forcing the persistent schedule on it is refused."""
    p = binding.plan(16777215, 12384, 1, 64, 128)
    assert p["head_blocks"] == 129 and p["grid_main"] >= 2 ** 31 and not p["persistent"]
    with pytest.raises(binding.MqaError):
        binding.plan(16777215, 12384, 1, 64, 128, schedule="persistent")
    assert binding.plan(16777215, 12288, 1, 64, 128)["persistent"]  # 2^31 - 128 items


def test_schedule_option_checks():
    assert call(opts=binding.make_opts(schedule=3)) == ERR_ARG
    assert call(opts=binding.make_opts(schedule=-1)) == ERR_ARG
    assert call(Lmax=1024, opts=binding.make_opts(chunk=128, combine=2, schedule=2)) == ERR_ARG
    assert call(opts=binding.make_opts(variant="valu", schedule=2)) == ERR_ARG
    with pytest.raises(binding.MqaError):
        binding.plan(2, 8, 2, 128, 64, schedule=3)


def test_noalloc_rejects_the_persistent_schedule():
    """Its queue would need memory that starts at zero; the planner's choice falls back silently."""
    assert call_noalloc(opts=binding.make_opts(schedule=2)) == ERR_ARG
    assert call_noalloc(opts=binding.make_opts(schedule=2, chunk=128)) == ERR_ARG
