"""Graph replay of whole decode steps (rswa_note_steps): a captured graph of
K fused decode steps + advance, replayed several times with fresh inputs
copied into its buffers and eager work between replays, gives bit-identical
outputs and state to the same steps run eagerly on a second cache; the state
of both is checked against the oracle's closed forms for ring_pos, cache_len
and position.  The fused eager outputs themselves are compared with the
oracle's RingCache in test_gpu_parity.py (test_fused_ring_write_decode)."""

import numpy as np
import pytest

from oracle import rswa_oracle as O

pytestmark = pytest.mark.gpu


def _make(torch, R, plens, window, layers, heads, dim, table=None, max_positions=4096):
    n = len(plens)
    rows = sum(p + window for p in plens)
    c = R.RSWACache(layers, heads, dim, window, max_requests=n, num_slots=rows, dtype="bf16",
                    max_positions=max_positions, slot_table=table, max_prefill_tokens=sum(plens))
    return c


# (prompt lengths, window, layers, heads): a few small requests (single-wave
# blocks), a one-round batch (blocks of four) and a batch beyond one round
# (blocks of eight, one per CU).
GRAPH_CONFIGS = {
    "small": ([40, 0, 300], 16, 2, 3),
    "one_round": ([5000 - 37 * i for i in range(24)], 128, 1, 10),
    "beyond_one_round": ([6000 - 29 * i for i in range(32)], 128, 1, 10),
}


@pytest.mark.parametrize("config", sorted(GRAPH_CONFIGS))
@pytest.mark.parametrize("paged", [False, True])
def test_graph_replay_matches_eager(paged, config):
    import torch
    from kv_cache_management_amd import rswa as R

    plens, window, layers, heads = GRAPH_CONFIGS[config]
    dim = 128
    n = len(plens)
    K, replays = 4, 6
    rows = sum(p + window for p in plens)
    table = None
    if paged:
        table = np.random.default_rng(3).permutation(rows).astype(np.int32)
    dev = torch.device("cuda", torch.cuda.current_device())
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    tot = sum(plens)
    pf = [[torch.randn((tot, heads, dim), device=dev, generator=gen).bfloat16() for _ in range(3)]
          for _ in range(layers)]
    caches = [_make(torch, R, plens, window, layers, heads, dim, table, max_positions=8192)
              for _ in range(2)]
    bases = np.concatenate([[0], np.cumsum([p + window for p in plens])[:-1]]).astype(np.int64)
    scratch = torch.empty((tot, heads, dim), device=dev, dtype=torch.bfloat16)
    for c in caches:
        for l in range(layers):
            c.prefill(l, list(range(n)), plens, bases.tolist(), *pf[l], scratch)
        c.set_batch(list(range(n)))
    # all decode inputs, [replay][step][layer][kind][n][H][D]
    inputs = torch.randn((replays, K, layers, 3, n, heads, dim), device=dev, generator=gen).bfloat16()
    stat_in = torch.zeros((K, layers, 3, n, heads, dim), device=dev, dtype=torch.bfloat16)
    stat_out = torch.zeros((K, layers, n, heads, dim), device=dev, dtype=torch.bfloat16)
    eager_out = torch.zeros_like(stat_out)
    torch.cuda.synchronize()

    gcache, ecache = caches
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(K):
                for l in range(layers):
                    gcache.decode_step_fused(l, stat_in[i, l, 0], stat_in[i, l, 1], stat_in[i, l, 2],
                                             stat_out[i, l])
                gcache.advance()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for r in range(replays):
        stat_in.copy_(inputs[r])
        if r > 0:
            gcache.note_steps(K)
        graph.replay()
        for i in range(K):
            for l in range(layers):
                ecache.decode_step_fused(l, inputs[r, i, l, 0], inputs[r, i, l, 1], inputs[r, i, l, 2],
                                         eager_out[i, l])
            ecache.advance()
        torch.cuda.synchronize()
        assert torch.equal(stat_out, eager_out), f"replay {r}"
        # eager work between replays, then the state of both caches
        rp_g, cl_g, np_g = gcache.get_state(list(range(n)))
        rp_e, cl_e, np_e = ecache.get_state(list(range(n)))
        assert list(rp_g) == list(rp_e) and list(cl_g) == list(cl_e) and list(np_g) == list(np_e)
        t = (r + 1) * K
        for b, p in enumerate(plens):
            assert rp_g[b] == O.ring_pos(t, window)
            assert cl_g[b] == O.cache_len(p, t - 1, window)
            assert np_g[b] == O.position(p, t)
    # the host view kept pace: a further whole-step call is accepted
    gcache.note_steps(0)
    # a new batch (the same ids) invalidates the graph captured before it
    gcache.set_batch(list(range(n)))
    with pytest.raises(R.RSWAError) as e:
        gcache.note_steps(K)
    assert e.value.status == R.RSWA_E_STATE
    for c in caches:
        c.close()


def _capture_one_step(torch, c, layers, z, zo):
    """Captures one whole fused step of c's batch into a graph (not replayed)."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for l in range(layers):
                c.decode_step_fused(l, z, z, z, zo)
            c.advance()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graph


def test_note_steps_rejects_half_step_and_position_overflow():
    import torch
    from kv_cache_management_amd import rswa as R

    c = _make(torch, R, [10], 8, 2, 2, 64)
    dev = torch.device("cuda", torch.cuda.current_device())
    x = torch.zeros((10, 2, 64), device=dev, dtype=torch.bfloat16)
    xo = torch.empty_like(x)
    for l in range(2):
        c.prefill(l, [0], [10], [0], x, x, x, xo)
    c.set_batch([0])
    z = torch.zeros((1, 2, 64), device=dev, dtype=torch.bfloat16)
    zo = torch.empty_like(z)
    with pytest.raises(R.RSWAError) as e:  # nothing captured for this batch
        c.note_steps(1)
    assert e.value.status == R.RSWA_E_STATE
    graph = _capture_one_step(torch, c, 2, z, zo)  # counts as step 0
    c.decode_step_fused(0, z, z, z, zo)
    with pytest.raises(R.RSWAError) as e:  # step 1 half done
        c.note_steps(1)
    assert e.value.status == R.RSWA_E_STATE
    c.decode_step_fused(1, z, z, z, zo)
    c.advance()
    c.note_steps(4096 - 10 - 2)
    with pytest.raises(R.RSWAError) as e:
        c.note_steps(1)
    assert e.value.status == R.RSWA_E_POSITION
    # calls that upload or synchronize refuse a capturing stream
    g2 = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    codes = []
    with torch.cuda.stream(side):
        with torch.cuda.graph(g2, stream=side):
            codes.append(R.rswa_set_batch(c.handle, [0], side.cuda_stream))
            codes.append(R.rswa_get_state(c.handle, [0], side.cuda_stream)[0])
    torch.cuda.synchronize()
    assert codes == [R.RSWA_E_STATE, R.RSWA_E_STATE]
    del graph, g2
    c.close()
