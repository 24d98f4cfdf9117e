"""Decode steps captured in a HIP graph and replayed (torch.cuda.CUDAGraph over the library's stream).

A serving loop captures its per-token work once and replays it.  The library allocates its split
workspace on the first call per (device, stream), so the call is warmed up on the capture's side
stream first; the captured kernels then keep that workspace's address.  Each replay runs after eager
work of this test (new inputs copied into the captured tensors, an eager decode call on another
stream) and must give the eager call's bits; one replay per case is also checked against the oracle.
The persistent schedule's queue counter lives in the same workspace and is back at zero after every
replay.
"""
import numpy as np
import pytest
import torch

import oracle
from gqa_decode_attention_mqa_amd import binding
from gqa_decode_attention_mqa_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = {
    # a PaLM-like MQA step with split chunks (merge kernel or fused merge)
    "mqa": Workload("g-mqa", B=6, Hq=48, Hkv=1, D=256, Lmax=1536, seed=1600, len_lo=1, len_hi=1536),
    # grouped heads, ragged lengths, one of them zero
    "gqa": Workload("g-gqa", B=5, Hq=16, Hkv=2, D=128, Lmax=2000, seed=1601, len_lo=0, len_hi=2000),
}


def _inputs(w, i):
    inp = make_inputs(w, seed=w.seed + 100 * i, poison_padding=True)
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in inp.items()}, inp


@pytest.mark.parametrize("combine,schedule", [(None, None), ("fused", None), (None, "persistent")])
@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_give_the_eager_bits(case, combine, schedule):
    w = CASES[case]
    sets = [_inputs(w, i) for i in range(3)]
    static = {k: sets[0][0][k].clone() for k in ("q", "k", "v", "seq_lens")}
    scale = sets[0][0]["scale"]
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)

    def step():
        binding.decode(static["q"], static["k"], static["v"], static["seq_lens"], scale, out=out, chunk=256,
                       combine=combine, schedule=schedule)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # allocates this stream's workspace before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("case graph capture", case, combine, schedule, flush=True)
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for it in range(6):
        dev, cpu = sets[it % 3]
        for k in static:
            static[k].copy_(dev[k])
        out.fill_(float("nan"))
        print("case graph replay", case, combine, schedule, it, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        ref = binding.decode(dev["q"], dev["k"], dev["v"], dev["seq_lens"], scale, chunk=256, combine=combine,
                             schedule=schedule)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d of %s / %s / %s differs from the eager call" % (it, case, combine,
                                                                                              schedule)
        if it == 4:
            exp = oracle.decode(cpu["q"], cpu["k"], cpu["v"], cpu["seq_lens"], scale)
            got = out.cpu().double().numpy()
            exp = np.asarray(exp, dtype=np.float64)
            assert np.all(np.abs(got - exp) <= 1e-2 + 1e-2 * np.abs(exp)), "replay %d against the oracle" % it
    del graph
