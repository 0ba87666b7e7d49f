"""The decode call captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay,
with new queries written in place by eager work between replays, must give exactly the results
of the eager call on the same inputs. The library launches only kernels (no memory fills, no
allocations), so the per-token call of a decode loop can be captured once and replayed.
Method: zh page, technical summary §3 (the set is re-selected for every query)."""
import numpy as np
import pytest

import dynamic_sparse_transformer_amd as topo
from tests._util import to_device, torch_cuda
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,n_ctx", [(2, None), (4, 16384)])
def test_decode_graph_replays_match_eager(cfg, n_ctx):
    torch = torch_cuda()
    over = {} if n_ctx is None else {"n_ctx": n_ctx}
    w = make_workload(cfg, **over)
    s = w.spec
    dq, dk, dv = (to_device(getattr(w, x), s.dtype) for x in ("q", "k", "v"))
    scale = float(s.softmax_scale)
    ws = torch.empty(topo.topo_workspace_bytes(dq, dk, s.W, s.k, scale), dtype=torch.uint8, device="cuda")
    out = torch.empty((s.B, s.Hq, 1, s.d), dtype=torch.float32, device="cuda")
    sel = torch.empty((s.B, s.Hq, 1, 1 + s.W + s.k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((s.B, s.Hq, 1), dtype=torch.int32, device="cuda")
    qbuf = dq.clone()

    def call(qq):
        topo.topo_attn_decode(qq, dk, dv, s.W, s.k, scale, out=out, sel_idx=sel, sel_count=cnt, workspace=ws)

    # warm up on a side stream, as graph capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(qbuf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(qbuf)
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for rep in range(4):
        # new queries (a permutation of the heads' queries plus a perturbation), written eagerly
        perm = rng.permutation(s.Hq)
        qnew = dq[:, perm] * (1.0 + 0.05 * rep)
        qbuf.copy_(qnew)
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_sel, g_cnt = out.clone(), sel.clone(), cnt.clone()
        call(qnew.contiguous())
        torch.cuda.synchronize()
        assert torch.equal(g_sel, sel) and torch.equal(g_cnt, cnt), f"replay {rep}: sets differ"
        assert torch.equal(g_out, out), f"replay {rep}: outputs differ"
