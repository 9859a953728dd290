"""alexnet_forward captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library enqueues only kernels on the caller's stream (no memory
sets, copies, allocations or host waits), so a capture of one call replays
that call.  The graph is replayed several times with the program's own eager
library calls and synchronisations between the replays, and every replay's
output is compared bit for bit with an eager call on the same inputs."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, stream_handle, to_device

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,batch", [(B.F32, 1), (B.BF16, 4)])
def test_forward_graph_replays_match_eager(dtype, batch):
    say(f"[gpu] graph capture of alexnet_forward dtype={dtype} batch={batch}")
    syn = I.synthetic(31, batch, groups=1, bf16=dtype == B.BF16)
    other = I.synthetic(32, batch, groups=1, bf16=dtype == B.BF16)
    sess = Session(batch, 1, dtype, B.MODE_FORWARD, DEV)
    params = sess.upload_params(syn.weights, syn.biases)
    x = to_device(syn.x, dtype, DEV)
    x_other = to_device(other.x, dtype, DEV)
    eager = torch.empty((batch, 1000), dtype=torch.float32, device=DEV)
    B.alexnet_forward(sess.cfg, params, x, eager, sess.ws, sess.ws_bytes, stream_handle())
    torch.cuda.synchronize()
    want = eager.cpu().numpy()

    out = torch.full((batch, 1000), float("nan"), dtype=torch.float32, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.alexnet_forward(sess.cfg, params, x, out, sess.ws, sess.ws_bytes, stream_handle())
    torch.cuda.synchronize()
    scratch = torch.empty_like(eager)
    for rep in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, want), f"replay {rep} differs from the eager call"
        # eager work between replays, on the same workspace and a different image
        B.alexnet_forward(sess.cfg, params, x_other, scratch, sess.ws, sess.ws_bytes, stream_handle())
        torch.cuda.synchronize()
        assert not np.array_equal(scratch.cpu().numpy(), want)
    say(f"[gpu]   4 replays bit-identical to the eager call")
    del graph
