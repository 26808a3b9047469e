"""The whole step -- routing and dispatch layout, the fused FFN, the combine
reduction -- captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed.
Every replay, with the program's own eager work and synchronisations between
replays, must give the eager step's combine rows and y_local bit for bit: the
step allocates nothing, records no memset node (the library clears with fill
kernels) and the persistent kernel's last workgroup resets its counters, so a
replay starts from the same state as an eager call."""
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as mo

from gpu_helpers import Uploaded, make_ffn, row_rel_err, run_forward

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 5e-2, "w4a8": 8e-2}


def _wl(dtype, seed):
    return mi.Workload(name="graph", num_slices=4, tokens_per_slice=160, num_experts=16, top_k=4,
                       local_begin=2, num_local=6, hidden=512, inter=384, dtype=dtype, skew=True,
                       seed=seed)


@pytest.mark.parametrize("dtype,sched", [("bf16", "interleaved"), ("bf16", "expert_wave"),
                                         ("fp8", "interleaved"), ("w4a8", "interleaved")])
def test_graph_replay_matches_eager_step(dtype, sched):
    wl = _wl(dtype, 8800 + len(dtype))
    inp = mi.make_inputs(wl)
    up = Uploaded(inp)
    ffn = make_ffn(wl)
    N, H = wl.num_tokens, wl.hidden
    y = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")

    def step():
        ffn.layout(logits=up.logits, bias=up.bias)
        run_forward(ffn, up, schedule=sched)
        ffn.combine_check(up.comb_slices, y=y)

    print(f"[graph] {dtype} {sched} eager", flush=True)
    up.reset_combine()
    step()
    torch.cuda.synchronize()
    ffn.check_status()
    want_c, want_y = up.comb_all.clone(), y.clone()
    ref = mo.run(inp, block_m=16)
    assert row_rel_err(up.combine_f64()[ref.written], ref.C[ref.written]).max() <= TOL[dtype]

    # warm up on a side stream, then capture on it (torch's recipe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print(f"[graph] {dtype} {sched} capture", flush=True)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work of the program between replays: clear the outputs
        up.reset_combine()
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[graph] {dtype} {sched} replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        ffn.check_status()
        assert torch.equal(up.comb_all, want_c)
        assert torch.equal(y.view(torch.int16), want_y.view(torch.int16))
