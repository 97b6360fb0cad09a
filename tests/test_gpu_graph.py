"""The decode and prefill products replayed from a HIP graph.

Every launch of qw_gemv (fp32 kernel at one row of x, matrix-core kernel at
4 and 8 rows), qw_gemv_batched (matrix-core kernel, groups of 32 codes) and
qw_gemm goes on the caller's stream and none of them
allocates or clears memory with a memset node, so a caller can capture them.
The graph is replayed several times with the program's own eager work and
synchronizations between replays, the outputs poisoned before each replay,
and every replay must give the eager call's bits (the kernels are
deterministic).
"""

import numpy as np
import pytest
import torch

from int8_int4_dequant_amd import inputs, qw

pytestmark = pytest.mark.gpu


def test_products_replay_from_a_hip_graph():
    dev = torch.device("cuda")
    n, k = 300, 1024
    w = torch.from_numpy(inputs.weight(31, n, k, 0.02)).to(dev)
    rec4 = qw.quantize_pack(w, 4, 128)
    rec8 = qw.quantize_pack(w, 8, 256)
    x1 = torch.from_numpy(inputs.activations(1, 1, k)).to(dev)
    x4 = torch.from_numpy(inputs.activations(2, 4, k)).to(dev)
    x8 = torch.from_numpy(inputs.activations(3, 8, k)).to(dev)
    xb = torch.from_numpy(inputs.bf16_activations(4, 40, k).view(np.int16)).to(dev)
    # a batch for the matrix-core kernel's groups-of-32 layout
    w32 = [torch.from_numpy(inputs.weight(40 + i, nn, kk, 0.02)).to(dev)
           for i, (nn, kk) in enumerate([(64, 512), (33, 256), (130, 1024)])]
    recs32 = [qw.quantize_pack(wi, 4, 32) for wi in w32]
    xs32 = [torch.from_numpy(inputs.activations(50 + i, 8, r["shape"][1])).to(dev)
            for i, r in enumerate(recs32)]
    outs = [torch.empty((mm, n), dtype=torch.float32, device=dev) for mm in (1, 4, 8, 40)]
    outs += [torch.empty((8, r["shape"][0]), dtype=torch.float32, device=dev) for r in recs32]

    def run():
        qw.gemv(rec4, x1, out=outs[0])
        qw.gemv(rec4, x4, out=outs[1])
        qw.gemv(rec8, x8, out=outs[2])
        qw.gemm(rec4, xb, out=outs[3])
        qw.gemv_batched(recs32, xs32, outs[4:])

    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    other = torch.empty((4, n), dtype=torch.float32, device=dev)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        qw.gemv(rec8, x4 * (rep + 2), out=other)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), f"replay {rep}"
