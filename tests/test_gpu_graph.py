"""moe_forward captured in a HIP graph replays bit-identical to the eager call.

The library allocates nothing, records no memset and never synchronises with
the host, so a forward can be captured; on the grouped path with a dense
branch the side stream joins the capture through the library's fork/join
events.  Each graph is replayed several times with the program's own eager
work and a synchronisation between replays, and every replay is compared with
the eager result."""
import pytest
import torch

from mixture_experts_ffn_router_amd import workloads as W
from tests.test_gpu_forward import DECODE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_ffn_router_amd import binding
    binding.load()
    return binding


def _specs():
    gemma_grouped = W.LayerSpec("graph_gemma", 40, 256, 16, 4, 128, "gelu_tanh", "bf16", router_mode="gemma",
                                per_expert_scale="uniform", I_dense=192)
    w8a8 = W.LayerSpec("graph_w8a8", 40, 256, 16, 4, 192, "silu", "fp8", scoring="sigmoid", n_groups=4,
                       topk_groups=2, act_quant="fp8_dynamic")
    return [(gemma_grouped, 40), (w8a8, 40), (DECODE["gemma_gammas"], 4), (DECODE["mxfp4_wide"], 16),
            (DECODE["e512_k64_bf16"], 16)]


@pytest.mark.parametrize("spec,T", _specs(), ids=["gemma-grouped", "w8a8-grouped", "gemma-decode",
                                                   "mxfp4-wave-items", "e512-k64-staged-down"])
def test_graph_replay_equals_eager(B, spec, T):
    L = W.make_layer(spec.with_T(T), seed=3)
    dl = B.DeviceLayer.from_generated(L)
    out = torch.empty_like(dl.t["x"])
    ws = torch.empty(dl.workspace_size(T), dtype=torch.uint8, device="cuda")
    dl.forward(out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        dl.forward(out=out, workspace=ws)
    torch.cuda.synchronize()
    for k in range(3):
        out.zero_()                       # the program's own work between replays
        ws.fill_(0xA5 if k % 2 else 0)    # the graph must not rely on the workspace's old contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {k} differs from the eager forward"
