"""A decode step of a serving loop captured in a HIP graph (through torch.cuda.CUDAGraph): decode over a
paged cache, then append the new tokens' keys and values to it.  These entry points allocate nothing,
synchronise nothing and launch only kernels (no memset nodes), so they can be captured; the launch shapes
come from max_cache_len, fixed at capture, and the lengths, page table and positions are read from device
memory at every replay.  Three steps with new inputs each, eager work and host synchronisation between the
replays: every replay's output and the pool after it equal the eager run bit for bit."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _gpu():
    import global_gqa_attention_amd as ga

    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the -m gpu tests")
    return ga


def test_paged_decode_step_graph_replays():
    ga = _gpu()
    dev = "cuda"
    g = torch.Generator().manual_seed(61)
    B, hq, hkv, steps, base = 8, 64, 4, 3, 1e7
    lens = torch.randint(1, 600, (B,), generator=g)
    lens[0] = 0                                   # a sequence with an empty cache
    cap = int(lens.max()) + steps
    P = B * cap + 100
    rows = torch.randperm(P, generator=g)[: B * cap].to(torch.int32).view(B, cap)   # each sequence's pool rows
    kp0 = torch.randn(P, hkv, 192, generator=g).to(torch.bfloat16)
    vp0 = torch.randn(P, hkv, 128, generator=g).to(torch.bfloat16)
    step_in = [(torch.randn(B, hq, 192, generator=g).to(torch.bfloat16),
                torch.randn(B, hkv, 192, generator=g).to(torch.bfloat16),
                torch.randn(B, hkv, 128, generator=g).to(torch.bfloat16)) for _ in range(steps)]

    def step_index(s):
        """(page table, cu_pages, positions, append slots) before step s: sequence b holds lens[b] + s rows."""
        n = lens + s
        cu = torch.zeros(B + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(n, 0)
        table = torch.zeros(B * cap, dtype=torch.int32)
        table[: int(cu[-1])] = torch.cat([rows[b, : int(n[b])] for b in range(B)])
        slots = torch.stack([rows[b, int(n[b])] for b in range(B)]).to(torch.int32)
        return table, cu, n.to(torch.int32), slots

    # static device buffers (the graph's fixed addresses)
    q, kn, vn = (torch.empty_like(t, device=dev) for t in step_in[0])
    table, cu, pos, slots = (torch.empty_like(t, device=dev) for t in step_index(0))
    kp, vp = kp0.to(dev), vp0.to(dev)
    out = torch.empty(B, hq, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ga.decode_workspace_size(B, cap, hq, -1), dtype=torch.uint8, device=dev)

    def load(s):
        for dst, src in zip((q, kn, vn), step_in[s]):
            dst.copy_(src)
        for dst, src in zip((table, cu, pos, slots), step_index(s)):
            dst.copy_(src)

    def step():
        ga.decode_paged(q, kn, vn, kp, vp, table, cu, pos, None, cap, -1, base, out=out, workspace=ws)
        ga.cache_append(kn, vn, pos, slots, kp, vp, base)

    # eager reference
    print("case graph decode step: eager", flush=True)
    ref_out = []
    for s in range(steps):
        load(s)
        step()
        ref_out.append(out.clone())
    torch.cuda.synchronize()
    ref_kp, ref_vp = kp.clone(), vp.clone()

    # capture (after a warm-up on a side stream, as torch asks), then replay from the initial pool
    kp.copy_(kp0)
    vp.copy_(vp0)
    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ga.decode_paged(q, kn, vn, kp, vp, table, cu, pos, None, cap, -1, base, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("case graph decode step: capture", flush=True)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    kp.copy_(kp0)
    vp.copy_(vp0)
    scratch = torch.randn(1 << 20, device=dev)
    for s in range(steps):
        load(s)
        print(f"case graph decode step: replay {s}", flush=True)
        graph.replay()
        scratch.mul_(1.5).add_(1.0)               # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out[s].view(torch.int16)), f"replay {s}"
    assert torch.equal(kp.view(torch.int16), ref_kp.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), ref_vp.view(torch.int16))
