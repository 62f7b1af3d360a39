"""HIP graph capture: a decode step (the split kernel and the combine) and a
prefill call, with every buffer supplied by the caller, captured once on a
side stream and replayed several times with eager work and synchronisation
between the replays. Every replay must reproduce the eager results bit for
bit (the library allocates nothing, synchronises nothing and clears no
memory with a memset inside a call)."""

import pytest
import torch

import gqa_flash_attention_amd as fa
import workloads
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replays_decode_and_prefill():
    shape = workloads.DecodeShape("graph", B=4, Sq=8, Hq=32, Hkv=4, D=128, page_size=16, max_len=1024,
                                  len_lo=8, len_hi=1024, kv_chunk=256, seed=77)
    di = workloads.decode_inputs(shape)
    q, kc, vc = di.q.to(DEV), di.kcache.to(DEV), di.vcache.to(DEV)
    table, lens = di.block_table.to(DEV), di.seq_lens.to(DEV)
    ws = torch.empty(fa.decode_workspace_bytes(shape.B, shape.Sq, shape.Hq, shape.D, shape.max_len,
                                               shape.kv_chunk), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(shape.B, shape.Hq, shape.Sq, dtype=torch.float32, device=DEV)
    pq, pk, pv = [t.to(DEV) for t in workloads.random_inputs(1, 300, 300, 8, 2, 128, seed=78)]
    po = torch.empty_like(pq)
    plse = torch.empty(1, 8, 300, dtype=torch.float32, device=DEV)

    def step():
        fa.decode_paged(q, kc, vc, table, lens, page_size=16, kv_chunk=shape.kv_chunk, causal=True,
                        scale=shape.scale, workspace=ws, out=o, lse=lse)
        fa.prefill(pq, pk, pv, causal=True, out=po, lse=plse)

    # eager reference (also warms the library's per-device caches)
    step()
    torch.cuda.synchronize()
    o_ref, lse_ref, po_ref, plse_ref = o.clone(), lse.clone(), po.clone(), plse.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for replay in range(4):
        # eager work between replays: clobber the outputs and the workspace
        o.fill_(0)
        po.fill_(0)
        lse.fill_(float("nan"))
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(o_ref)), f"decode O differs on replay {replay}"
        assert torch.equal(_bits(lse), _bits(lse_ref)), f"decode LSE differs on replay {replay}"
        assert torch.equal(_bits(po), _bits(po_ref)) and torch.equal(_bits(plse), _bits(plse_ref)), replay
