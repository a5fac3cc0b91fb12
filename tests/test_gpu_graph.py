"""One rank's ring step captured in a HIP graph.

The step is shard balance, the forward over every chunk with the fused
merge, the bf16 output, and the backward. No call in it allocates outside
torch's graph pool, synchronises or writes memory with a memset, so the
captured step replays the same kernels. The kernels are deterministic (no
atomics), so every replay must equal the eager step bit for bit. Replays run
with new inputs copied in, with eager work and synchronisations between them
and the outputs overwritten before each one, so a replay that did nothing
cannot pass.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp, ring
    mmsp.lib()
    return mmsp, ring


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_equal_eager(mm, fused):
    import torch
    mmsp, ring = mm
    n, p, rank, hq, hkv, d = 4096, 4, 1, 8, 2, 128
    shard = n // p
    dev = "cuda"
    print(f"[graph] n={n} P={p} rank={rank} hq={hq} hkv={hkv} d={d} fused={fused}", flush=True)

    def draw(seed):
        rng = np.random.default_rng(seed)

        def f(shape):
            return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(
                torch.bfloat16)
        return [f((shard, hq, d)), f((p, shard, hkv, d)), f((p, shard, hkv, d)),
                f((shard, hq, d))]

    sets = [draw(s) for s in (21, 22, 23)]
    q = torch.empty((shard, hq, d), dtype=torch.bfloat16, device=dev)
    k_all = torch.empty((p, shard, hkv, d), dtype=torch.bfloat16, device=dev)
    v_all = torch.empty_like(k_all)
    do = torch.empty_like(q)
    o = torch.empty((shard, hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((hq, shard), dtype=torch.float32, device=dev)
    o16 = torch.empty((shard, hq, d), dtype=torch.bfloat16, device=dev)
    dq = torch.empty((shard, hq, d), dtype=torch.float32, device=dev)
    dks = [torch.empty((shard, hkv, d), dtype=torch.float32, device=dev) for _ in range(p)]
    dvs = [torch.empty_like(t) for t in dks]
    delta = torch.empty((hq, shard), dtype=torch.float32, device=dev)
    outs = [o, lse, o16, dq, *dks, *dvs]
    names = ["o", "lse", "o16", "dq"] + [f"dk{c}" for c in range(p)] + [f"dv{c}" for c in range(p)]

    def step():
        perm, _ = mmsp.shard_balance(n, p, device=dev)
        qp = perm[rank * shard:(rank + 1) * shard]
        kps = [perm[c * shard:(c + 1) * shard] for c in range(p)]
        ks = [k_all[c] for c in range(p)]
        vs = [v_all[c] for c in range(p)]
        ring.ring_forward(q, ks, vs, qp, kps, rank=rank, fused=fused, o=o, lse=lse,
                          o_final=o16)
        ring.ring_backward(q, ks, vs, do, o16, lse, qp, kps, rank=rank, dq=dq, dks=dks,
                           dvs=dvs, delta=delta)

    def load(i):
        for dst, src in zip((q, k_all, v_all, do), sets[i]):
            dst.copy_(src)
        torch.cuda.synchronize()

    expected = []
    for i in range(len(sets)):
        load(i)
        step()
        torch.cuda.synchronize()
        expected.append([t.clone() for t in outs])
    assert not torch.equal(expected[0][0], expected[1][0])

    # warm up on a side stream (default priority), then capture
    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i in (1, 0, 2, 2):
        load(i)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, expected[i]):
            assert torch.equal(got, want), f"replay with input set {i}: {name} differs from eager"
