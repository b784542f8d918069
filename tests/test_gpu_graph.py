"""A decode step captured as a HIP graph and replayed several times gives the
outputs of the same step launched one by one, bit for bit, on every replay
(eager work, output clearing and synchronisations between the replays): the
step's kernels leave the selection counters cleared for the next replay and
record no memory set or copy of their own."""
import numpy as np
import pytest
import torch

from gpu_common import case, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pattern,B,Q,N,P,ratio", [
    ("FRRR", 2, 1, 300_000, 2048, 1),   # the pool over 37,500 block maxima: split + finish selection
    ("FUUU", 2, 1, 40_000, 0, 1),       # 40,000 entries per row: split + finish selection of the Top-K
    # a prefill chunk: screened selection of 256 rows, the group's staged fp16
    # copy of the cache, persistent attention of the Full and Reuse layers
    ("FUU", 1, 256, 16_384, 0, 2),
])
def test_graph_replays_match_eager_step(pattern, B, Q, N, P, ratio):
    require_gpu()
    from fp4_kv_cache_csa2_amd import inputs, workload

    w = inputs.Workload("graph_" + pattern, B=B, Q=Q, N=N, D=512, H=64, H_i=8, D_i=128, pattern=pattern,
                        P=P if P else 2048, ratio=ratio)
    inst = workload.make_instance(w, device="cuda:0")
    run = workload.StackRunner(inst)
    case(f"graph replay {pattern} N={N}: eager step")
    run.step(keep_indices=True)
    torch.cuda.synchronize()
    ref_o = [o.clone() for o in run.o]
    ref_lse = [l.clone() for l in run.lse]
    ref_sel = run.state.idx.clone()   # the last layer's selection
    ref_pool = run.state.pool.clone()

    case(f"graph replay {pattern} N={N}: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.step()
    torch.cuda.synchronize()

    scratch = torch.empty(1 << 20, device="cuda:0")
    for rep in range(3):
        case(f"graph replay {pattern} N={N}: replay {rep}")
        # clear what the step writes, and some unrelated eager work in between
        for t in run.o + run.lse:
            t.fill_(float("nan"))
        run.state.idx.fill_(-7)
        run.state.pool.fill_(-7)
        scratch.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.state.idx, ref_sel), f"replay {rep}: the last selection differs"
        for l in range(w.layers):
            assert np.array_equal(run.o[l].cpu().numpy().view(np.uint32), ref_o[l].cpu().numpy().view(np.uint32)), \
                f"replay {rep}: layer {l} o differs"
            assert np.array_equal(run.lse[l].cpu().numpy().view(np.uint32),
                                  ref_lse[l].cpu().numpy().view(np.uint32)), f"replay {rep}: layer {l} lse differs"
        if "R" in pattern:
            assert torch.equal(run.state.pool, ref_pool), f"replay {rep}: pool differs"
