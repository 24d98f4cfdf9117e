"""Seeded synthetic inputs for the decode-attention step.

This module is shared by the GPU path's tests and bench and by the CPU
oracle's tests.  It only draws random numbers and lays them out; it contains
none of the attention arithmetic, so neither side can lean on the other
through it.

Recipe (the same for every workload):
  * one ``torch.Generator`` on the generating device, seeded with the
    workload's seed;
  * draw order: sequence lengths (ragged workloads only), then q, then K,
    then V;
  * q, K and V are drawn as float32 N(0, 1) and rounded to bfloat16 with
    round-to-nearest-even (``Tensor.to(torch.bfloat16)``);
  * an optional power-of-two multiplier on q (exact in bfloat16) makes the
    softmax peaky;
  * ragged lengths are iid uniform integers in ``[len_lo, len_hi]``, both ends
    included; the cache is allocated at ``Lmax`` regardless;
  * optionally the padding (positions >= the sequence's length) is poisoned
    with the bfloat16 quiet-NaN pattern 0x7FC0 so that any read of it shows;
  * an 8-bit cache (fp8 E4M3 or int8) is made from the bfloat16 one by
    :func:`quantize_cache`: one fp32 scale per cached row (position, kv head)
    = the row's largest magnitude over the format's largest code (448 or 127),
    codes rounded to nearest-even; padding rows get NaN codes and scales.

The same seed on a different device yields different (but equally valid)
numbers; a test that compares two implementations always hands both the same
tensors, copied if needed, never two separate draws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

BF16_QNAN_BITS = 0x7FC0
FP8_E4M3_NAN_CODE = 0x7F
INT8_UNUSED_CODE = 0x80   # -128: the symmetric int8 quantizer never produces it
KV_FORMAT_MAX = {"fp8": 448.0, "int8": 127.0}


@dataclass(frozen=True)
class Workload:
    """Shape and input distribution of one decode step."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    seed: int
    len_lo: int | None = None   # None: every sequence has length Lmax
    len_hi: int | None = None
    q_mult: float = 1.0
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        """1/sqrt(D), rounded to float32 (the value the library receives)."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def ragged(self) -> bool:
        return self.len_lo is not None

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five decode workloads.  Shapes follow the attention shapes the source
# pages discuss: PaLM 540B multiquery attention (48 query heads sharing one
# 256-wide key/value head), a 70B-class grouped-query model (64 query heads,
# 8 key/value heads, head size 128), a ragged batch, and a long-context MQA
# case that forces the sequence axis to be split.
WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, Hq=8, Hkv=1, D=64, Lmax=128, seed=0,
                     description="tiny MQA decode B=1 Hq=8 Hkv=1 D=64 len=128"),
    "palm": Workload("palm", B=64, Hq=48, Hkv=1, D=256, Lmax=2048, seed=1,
                     description="PaLM-540B-shaped MQA decode B=64 Hq=48 Hkv=1 D=256 len=2048"),
    "gqa70b": Workload("gqa70b", B=32, Hq=64, Hkv=8, D=128, Lmax=4096, seed=2,
                       description="70B-class GQA decode B=32 Hq=64 Hkv=8 D=128 len=4096"),
    "ragged": Workload("ragged", B=256, Hq=32, Hkv=8, D=128, Lmax=8192, seed=3,
                       len_lo=1, len_hi=8192,
                       description="ragged GQA decode B=256 Hq=32 Hkv=8 D=128 len~U[1,8192] Lmax=8192"),
    "long": Workload("long", B=4, Hq=48, Hkv=1, D=256, Lmax=131072, seed=4, q_mult=4.0,
                     description="long-context MQA decode B=4 Hq=48 Hkv=1 D=256 len=131072, q*4"),
}


def draw_lengths(w: Workload, gen: torch.Generator, device) -> torch.Tensor:
    if w.ragged:
        return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=gen,
                             device=device, dtype=torch.int32)
    return torch.full((w.B,), w.Lmax, dtype=torch.int32, device=device)


def _randn_bf16(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def poison_padding_(cache: torch.Tensor, seq_lens: torch.Tensor) -> torch.Tensor:
    """Overwrite positions >= seq_lens[b] of a [B, Lmax, H, D] cache with bf16 NaN."""
    B, Lmax = cache.shape[0], cache.shape[1]
    pos = torch.arange(Lmax, device=cache.device, dtype=torch.int32).view(1, Lmax)
    pad = (pos >= seq_lens.to(cache.device).view(B, 1)).view(B, Lmax, 1, 1)
    cache.view(torch.int16).masked_fill_(pad, BF16_QNAN_BITS)
    return cache


def poison_positions_below_(cache: torch.Tensor, first: torch.Tensor) -> torch.Tensor:
    """Overwrite positions < first[b] of a [B, Lmax, H, D] cache with bf16 NaN
    (used to show that positions outside a sliding window are never read)."""
    B, Lmax = cache.shape[0], cache.shape[1]
    pos = torch.arange(Lmax, device=cache.device, dtype=torch.int32).view(1, Lmax)
    below = (pos < first.to(cache.device).view(B, 1)).view(B, Lmax, 1, 1)
    cache.view(torch.int16).masked_fill_(below, BF16_QNAN_BITS)
    return cache


def make_inputs(w: Workload, device="cpu", seed: int | None = None,
                poison_padding: bool = False, seq_lens=None) -> dict:
    """Draw q, K, V (bf16) and seq_lens (int32) for workload ``w`` on ``device``.

    ``seq_lens`` overrides the drawn lengths (the draw still happens, so the
    q/K/V streams do not shift).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else int(seed))
    lens = draw_lengths(w, gen, device)
    if seq_lens is not None:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).to(device).reshape(w.B).contiguous()
    q = _randn_bf16((w.B, w.Hq, w.D), gen, device)
    if w.q_mult != 1.0:
        q = q * w.q_mult
    k = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    v = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    if poison_padding:
        poison_padding_(k, lens)
        poison_padding_(v, lens)
    return {"q": q, "k": k, "v": v, "seq_lens": lens, "scale": w.scale}


def make_multi_inputs(w: Workload, tokens: int, device="cpu", seed: int | None = None,
                      poison_padding: bool = False, seq_lens=None) -> dict:
    """Like :func:`make_inputs` but with ``tokens`` new query tokens per sequence:
    q [B, tokens, Hq, D] (their keys and values sit at the last ``tokens`` cached positions).
    ``seq_lens`` overrides the drawn lengths as in :func:`make_inputs`."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed if seed is None else seed))
    lens = draw_lengths(w, gen, device)
    if seq_lens is not None:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).to(device).reshape(w.B).contiguous()
    q = _randn_bf16((w.B, tokens, w.Hq, w.D), gen, device)
    if w.q_mult != 1.0:
        q = q * w.q_mult
    k = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    v = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    if poison_padding:
        poison_padding_(k, lens)
        poison_padding_(v, lens)
    return {"q": q, "k": k, "v": v, "seq_lens": lens, "scale": w.scale}


def make_prefill_inputs(w: Workload, device="cpu", seed: int | None = None,
                        poison_padding: bool = False) -> dict:
    """Like :func:`make_inputs` but with one query per position: q_seq [B, Lmax, Hq, D]."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else int(seed))
    lens = draw_lengths(w, gen, device)
    q = _randn_bf16((w.B, w.Lmax, w.Hq, w.D), gen, device)
    if w.q_mult != 1.0:
        q = q * w.q_mult
    k = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    v = _randn_bf16((w.B, w.Lmax, w.Hkv, w.D), gen, device)
    if poison_padding:
        poison_padding_(k, lens)
        poison_padding_(v, lens)
    return {"q_seq": q, "k": k, "v": v, "seq_lens": lens, "scale": w.scale}


def _page_assignment(lens: torch.Tensor, Lmax: int, page_size: int, seed: int, spare_pages: int):
    """Seeded placement of each sequence's ceil(len / page_size) blocks on physical pages.

    Returns (block_table [B, max_blocks] int32 on the CPU, -1 past a sequence's
    last block; [(b, blk, page)] in placement order; num_pages; max_blocks).
    """
    B = lens.shape[0]
    max_blocks = max(1, -(-Lmax // page_size))
    lens_cpu = lens.to("cpu").tolist()
    nblocks = [-(-n // page_size) for n in lens_cpu]
    num_pages = sum(nblocks) + spare_pages
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    perm = torch.randperm(max(num_pages, 1), generator=gen)[:num_pages].tolist()
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    placed = []
    i = 0
    for b in range(B):
        for blk in range(nblocks[b]):
            table[b, blk] = perm[i]
            placed.append((b, blk, perm[i]))
            i += 1
    return table, placed, num_pages, max_blocks


def _placement_indices(placed, device):
    """(sequence, logical block, physical page) triples as three index tensors."""
    t = torch.tensor(placed, dtype=torch.int64).reshape(-1, 3).to(device)
    return t[:, 0], t[:, 1], t[:, 2]


def page_contiguous_cache(inp: dict, page_size: int, seed: int, spare_pages: int = 0,
                          poison_spare: bool = True) -> dict:
    """Move the contiguous caches of ``inp`` (from :func:`make_inputs`) into a paged pool.

    Each sequence b gets ceil(len_b / page_size) physical pages, in a seeded
    random order over the whole pool, plus ``spare_pages`` unused pages
    (bf16 NaN when ``poison_spare``).  block_table [B, max_blocks] holds the
    physical page of each logical block; entries past a sequence's last block
    are -1 and must never be read.  Rows of a sequence's last page past its
    length keep the cache's padding.  Adds ``k_pages``, ``v_pages``,
    ``block_table``, ``page_size`` and ``num_pages`` to a copy of ``inp``.
    """
    k, v, lens = inp["k"], inp["v"], inp["seq_lens"]
    B, Lmax, Hkv, D = k.shape
    device = k.device
    table, placed, num_pages, max_blocks = _page_assignment(lens, Lmax, page_size, seed, spare_pages)
    # padded contiguous caches so every block of page_size rows exists
    padded_len = max_blocks * page_size
    if padded_len > Lmax:
        fill = torch.full((B, padded_len - Lmax, Hkv, D), 0, dtype=k.dtype, device=device)
        fill.view(torch.int16).fill_(BF16_QNAN_BITS)
        kc, vc = torch.cat([k, fill], 1), torch.cat([v, fill.clone()], 1)
    else:
        kc, vc = k, v
    k_pages = torch.empty((max(num_pages, 1), page_size, Hkv, D), dtype=k.dtype, device=device)
    v_pages = torch.empty_like(k_pages)
    if poison_spare:
        k_pages.view(torch.int16).fill_(BF16_QNAN_BITS)
        v_pages.view(torch.int16).fill_(BF16_QNAN_BITS)
    else:
        k_pages.zero_()
        v_pages.zero_()
    if placed:
        # one gather per cache (a copy per page would be thousands of launches)
        bs, blks, pages = _placement_indices(placed, device)
        k_pages[pages] = kc.reshape(B, max_blocks, page_size, Hkv, D)[bs, blks]
        v_pages[pages] = vc.reshape(B, max_blocks, page_size, Hkv, D)[bs, blks]
    out = dict(inp)
    out.update({"k_pages": k_pages, "v_pages": v_pages, "block_table": table.to(device),
                "page_size": page_size, "num_pages": num_pages})
    return out


def page_quant_cache(inp: dict, qc: dict, page_size: int, seed: int, spare_pages: int = 0) -> dict:
    """Move an 8-bit cache (``qc`` from :func:`quantize_cache` of ``inp``) into a paged pool,
    with the same seeded placement as :func:`page_contiguous_cache`.

    Returns ``k_pages`` / ``v_pages`` (uint8 [num_pages, page_size, Hkv, D]),
    ``k_scale_pages`` / ``v_scale_pages`` (fp32 [num_pages, Hkv, page_size]),
    ``block_table``, ``page_size`` and ``num_pages``.  Spare pages and rows
    past Lmax hold 0xFF codes (NaN in E4M3) and NaN scales.
    """
    lens = inp["seq_lens"]
    kq = qc["k_codes"]
    B, Lmax, Hkv, D = kq.shape
    device = kq.device
    table, placed, num_pages, max_blocks = _page_assignment(lens, Lmax, page_size, seed, spare_pages)
    padded_len = max_blocks * page_size
    out = {"block_table": table.to(device), "page_size": page_size, "num_pages": num_pages}
    for name in ("k", "v"):
        codes, sc = qc[name + "_codes"], qc[name + "_scale"]          # [B,L,Hkv,D], [B,Hkv,L]
        if padded_len > Lmax:
            codes = torch.cat([codes, torch.full((B, padded_len - Lmax, Hkv, D), 0xFF, dtype=torch.uint8,
                                                 device=device)], 1)
            sc = torch.cat([sc, torch.full((B, Hkv, padded_len - Lmax), float("nan"), device=device)], 2)
        pages = torch.full((max(num_pages, 1), page_size, Hkv, D), 0xFF, dtype=torch.uint8, device=device)
        spages = torch.full((max(num_pages, 1), Hkv, page_size), float("nan"), dtype=torch.float32, device=device)
        if placed:
            bs, blks, idx = _placement_indices(placed, device)
            pages[idx] = codes.reshape(B, max_blocks, page_size, Hkv, D)[bs, blks]
            # a slice between the two index tensors: the result is [pages, Hkv, page_size]
            spages[idx] = sc.reshape(B, Hkv, max_blocks, page_size)[bs, :, blks]
        out[name + "_pages"] = pages
        out[name + "_scale_pages"] = spages
    return out


def quantize_cache(inp: dict, kv_format: str, pow2_scales: bool = False, poison_padding: bool = True) -> dict:
    """8-bit copies of the bf16 caches of ``inp`` (from :func:`make_inputs`).

    Returns ``k_codes`` / ``v_codes`` (uint8 bit patterns [B, Lmax, Hkv, D]:
    E4M3 for "fp8", two's complement for "int8") and ``k_scale`` / ``v_scale``
    (float32 [B, Hkv, Lmax], one per cached row), on the caches' device.  A
    row's scale is its largest magnitude over the format's largest code (a
    power of two at or above that when ``pow2_scales``), 1 for an all-zero
    row; codes are the row divided by its scale, rounded to nearest-even.
    Rows at or past a sequence's length get NaN scales and NaN (fp8) or -128
    (int8) codes when ``poison_padding``.
    """
    qmax = KV_FORMAT_MAX[kv_format]
    lens = inp["seq_lens"]
    out = {}
    for name in ("k", "v"):
        x = inp[name].float()                                   # [B, Lmax, Hkv, D]
        B, Lmax = x.shape[0], x.shape[1]
        amax = x.abs().amax(dim=-1)                             # [B, Lmax, Hkv]
        valid = torch.isfinite(amax) & (amax > 0)
        sc = torch.where(valid, amax / qmax, torch.ones_like(amax))
        if pow2_scales:
            sc = torch.exp2(torch.ceil(torch.log2(sc)))
        y = x / sc.unsqueeze(-1)
        if kv_format == "fp8":
            codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            codes = torch.round(y).clamp(-127, 127).to(torch.int8).view(torch.uint8)
        pos = torch.arange(Lmax, device=x.device, dtype=torch.int32).view(1, Lmax)
        pad = pos >= lens.to(x.device).view(B, 1)               # [B, Lmax]
        if poison_padding:
            fill = FP8_E4M3_NAN_CODE if kv_format == "fp8" else INT8_UNUSED_CODE
            codes = codes.masked_fill(pad.view(B, Lmax, 1, 1), fill)
            sc = sc.masked_fill(pad.view(B, Lmax, 1), float("nan"))
        out[name + "_codes"] = codes.contiguous()
        out[name + "_scale"] = sc.permute(0, 2, 1).contiguous().to(torch.float32)   # [B, Hkv, Lmax]
    return out
