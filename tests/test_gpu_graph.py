"""GPU: the layer forward captured into a HIP graph, as the benchmark times it,
gives the eager result on every replay.

The library allocates nothing and never synchronises, so a whole layer step
can be captured.  Each case runs the step eagerly on two inputs, captures it
on the first, then replays the graph several times with an eager step on the
second input -- over the same workspace and output buffers -- before each
replay, and checks every result bit for bit against the eager ones.  The
cases cover the decode path with the shared expert in the router's launches
(GLM, 1 and 16 tokens), the decode path without a shared expert (Granite),
int2 experts on the LDS ring, and the prefill grouped GEMM with its split-K
router.
"""
import numpy as np
import pytest

import gen
from tests.gpu_common import print_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

DEV = "cuda:0"

CASES = [("c2", None, 1), ("c2", None, 16), ("c1", None, 1), ("c4", gen.I2, 2),
         ("c3", None, 300)]
REPLAYS = 3


@pytest.mark.parametrize("name,dtype,T", CASES)
def test_graph_replays_match_eager(name, dtype, T):
    cfg = gen.get_config(name)
    print_case("graph replay", name, dtype, T)
    if name in ("c0", "c1"):
        layer = gdev.upload_host_layer(gen.host_layer(cfg, 0, experts="all"), DEV)
    else:
        layer = gdev.generate_device_layer(cfg, 0, DEV, dtype=dtype)
    desc = capi.make_desc(layer.desc_spec)
    wts = capi.make_weights(layer.pointers())
    nb = capi.moe_workspace_bytes(desc, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)

    def xdev(batch_id):
        x = gen.x_tokens(cfg, T, batch_id=batch_id)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(DEV)

    xa, xb = xdev(41), xdev(42)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    torch.cuda.synchronize()

    def step(x):
        capi.moe_layer_forward_ex(desc, wts, x, T, out, idx, tw, ws, nb, stream=s.cuda_stream)

    def snapshot():
        s.synchronize()
        return out.clone(), idx.clone(), tw.clone()

    def same(got, want):
        return all(torch.equal(g, w) for g, w in zip(got, want))

    step(xa)
    ref_a = snapshot()
    step(xb)
    ref_b = snapshot()
    assert not torch.equal(ref_a[0], ref_b[0])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        step(xa)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        step(xb)
        assert same(snapshot(), ref_b), f"eager step between replays, round {r}"
        with torch.cuda.stream(s):
            g.replay()
        assert same(snapshot(), ref_a), f"graph replay {r}"
    torch.cuda.synchronize()
