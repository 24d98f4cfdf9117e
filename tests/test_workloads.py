"""The seeded input builders (CPU): paged pools against a literal per-page copy.

The pools are built with one gather per cache; these tests rebuild them page
by page from the block table alone and require bit equality, including the
NaN padding of a sequence's last page, the spare pages and the 8-bit scales.
"""
import pytest
import torch

from gqa_decode_attention_mqa_amd.workloads import (Workload, make_inputs, page_contiguous_cache, page_quant_cache,
                                                    quantize_cache)


def per_page_reference(cache, table, lens, page_size, num_pages, fill):
    """pages[p] = rows blk*page_size .. of sequence b, for every table entry (b, blk) -> p."""
    B, Lmax = cache.shape[0], cache.shape[1]
    out = torch.empty((max(num_pages, 1), page_size) + tuple(cache.shape[2:]), dtype=cache.dtype)
    out[...] = fill
    for b in range(B):
        nblk = -(-int(lens[b]) // page_size)
        for blk in range(nblk):
            p = int(table[b, blk])
            rows = cache[b, blk * page_size:min((blk + 1) * page_size, Lmax)]
            out[p] = fill
            out[p, :rows.shape[0]] = rows
        for blk in range(nblk, table.shape[1]):
            assert int(table[b, blk]) == -1
    return out


def check_table(table, lens, page_size, num_pages):
    used = [int(p) for p in table.flatten().tolist() if p >= 0]
    assert len(used) == len(set(used)), "a physical page is shared inside one pool"
    assert all(0 <= p < num_pages for p in used)
    assert len(used) == sum(-(-int(n) // page_size) for n in lens.tolist())


@pytest.mark.parametrize("page_size", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("lens", [None, [0, 0, 0], [1, 300, 33], [300, 300, 300]])
def test_paged_pool_equals_per_page_copies(page_size, lens):
    w = Workload("pool", B=3, Hq=4, Hkv=2, D=64, Lmax=300, seed=11, len_lo=0, len_hi=300)
    inp = make_inputs(w, poison_padding=True, seq_lens=lens)
    pg = page_contiguous_cache(inp, page_size, seed=page_size, spare_pages=2)
    table = pg["block_table"]
    check_table(table, inp["seq_lens"], page_size, pg["num_pages"])
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    for name in ("k", "v"):
        ref = per_page_reference(inp[name], table, inp["seq_lens"], page_size, pg["num_pages"], nan)
        got = pg[name + "_pages"]
        # padding past a length or past Lmax, and spare pages, are NaN on both sides
        assert torch.equal(torch.isnan(got), torch.isnan(ref))
        assert torch.equal(torch.nan_to_num(got.float()), torch.nan_to_num(ref.float()))


@pytest.mark.parametrize("kv_format", ["fp8", "int8"])
@pytest.mark.parametrize("page_size", [32, 128, 512])
def test_paged_quant_pool_equals_per_page_copies(kv_format, page_size):
    w = Workload("qpool", B=4, Hq=4, Hkv=2, D=64, Lmax=300, seed=12, len_lo=0, len_hi=300)
    inp = make_inputs(w, poison_padding=True, seq_lens=[1, 300, 0, 129])
    qc = quantize_cache(inp, kv_format)
    pq = page_quant_cache(inp, qc, page_size, seed=page_size, spare_pages=2)
    table = pq["block_table"]
    check_table(table, inp["seq_lens"], page_size, pq["num_pages"])
    for name in ("k", "v"):
        ref = per_page_reference(qc[name + "_codes"], table, inp["seq_lens"], page_size, pq["num_pages"], 0xFF)
        assert torch.equal(pq[name + "_pages"], ref)
        # scales: [B, Hkv, Lmax] -> pages [num_pages, Hkv, page_size]
        sc = qc[name + "_scale"].transpose(1, 2).contiguous()  # [B, Lmax, Hkv]
        sref = per_page_reference(sc, table, inp["seq_lens"], page_size, pq["num_pages"], float("nan"))
        got = pq[name + "_scale_pages"].transpose(1, 2)           # [pages, page_size, Hkv]
        assert torch.equal(torch.isnan(got), torch.isnan(sref))
        assert torch.equal(torch.nan_to_num(got), torch.nan_to_num(sref))
