"""Capture of the library's calls into a HIP graph (needs an MI355X).

The entry points take caller-owned buffers and a stream and never allocate, copy to the host or
synchronise, and the counters of the split hand-offs are cleared by the preparation kernels (no
memset nodes), so a training step (forward + backward) or a decode step can be captured once and
replayed.  Each test replays its graph several times, with eager calls of the library on other
inputs and host synchronisations between the replays, and requires every replay to reproduce the
eager result: bitwise, except dq of the atomic backward, whose adds land in a varying order (the bar
of its repeat test in test_gpu_parity, plus one unit in the last place of a 16-bit output).
"""
import pytest
import torch

from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import ATOMIC, BWD_FLAGS, BWD_IDS, DEV, bwd_workspace
from tests.test_gpu_decode import fill_cache, seqs

pytestmark = pytest.mark.gpu


def _replays(graph, outs, ref, other, exact):
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            if exact[i]:
                assert torch.equal(a, b), (rep, i)
            else:   # rounding of a differently ordered sum: 1e-5 of the scale, plus one ulp of a 16-bit output
                x, y = a.float(), b.float()
                ulp = torch.finfo(a.dtype).eps * y.abs() if a.dtype != torch.float32 else 0.0
                bad = ((x - y).abs() > 1e-5 * float(y.abs().max()) + ulp).sum().item()
                assert bad == 0, (rep, i, bad, float((x - y).abs().max()))
        other()   # eager work of the program between the replays
        torch.cuda.synchronize()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("flags", BWD_FLAGS, ids=BWD_IDS)
@pytest.mark.parametrize("shape,out_dt", [
    ((1, 1000, 4, 1, 128), torch.bfloat16),   # one group: split plans in all three passes
    ((2, 300, 6, 2, 64), torch.float32),
])
def test_training_step_replays_from_a_graph(shape, out_dt, flags):
    B, T, Hq, Hkv, D = shape
    q, k, v, dO = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=41, dtype="bf16"))
    q2, k2, v2, dO2 = (t.to(DEV) for t in inputs.random_case(B, T, Hq, Hkv, D, seed=42, dtype="bf16"))
    base = 1.0e4
    ws = bwd_workspace(q, k, base, flags)
    ws2 = bwd_workspace(q, k, base, flags)
    o = torch.empty((B, T, Hq, D), dtype=out_dt, device=DEV)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    dq, dk = torch.empty_like(o), torch.empty((B, T, Hkv, D), dtype=out_dt, device=DEV)
    dv = torch.empty_like(dk)

    def step():
        binding.ne_rope_attn_fwd(q, k, v, base, o=o, lse=lse, workspace=ws)
        binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, base, dq=dq, dk=dk, dv=dv, workspace=ws, flags=flags)

    def other():
        o2, lse2 = binding.ne_rope_attn_fwd(q2, k2, v2, base, out_dtype=out_dt, workspace=ws2)
        binding.ne_rope_attn_bwd(q2, k2, v2, o2, lse2, dO2, base, workspace=ws2, flags=flags)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    g = _capture(step)
    exact = [True, True, flags != ATOMIC, True, True]
    _replays(g, [o, lse, dq, dk, dv], ref, other, exact)


def test_decode_step_replays_from_a_graph():
    """One new token per sequence against a filled cache, as a serving loop would capture it."""
    B, P, Hq, Hkv, D, Tcap, base = 3, 200, 8, 2, 128, 256, 1.0e4
    q, k, v = seqs(B, P, Hq, Hkv, D, 700, "bf16")
    cache = fill_cache(k, v, Tcap, base, (64, 64, 72))
    lens = torch.tensor([0, 57, 199], dtype=torch.int32, device=DEV)
    q_new = torch.stack([q[b, int(lens[b]):int(lens[b]) + 1] for b in range(B)]).to(DEV)
    q_other = torch.flip(q_new, dims=(0,)).contiguous()
    o = torch.empty((B, 1, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=DEV)
    n = binding.decode_workspace_bytes(B, 1, Tcap, Hq, Hkv, D, q_new.dtype)
    ws, ws2 = binding.alloc_workspace(n, DEV), binding.alloc_workspace(n, DEV)

    def step():
        binding.ne_rope_attn_decode(q_new, cache, lens, Tcap, Hkv, base, 0, out_dtype=torch.float32, o=o, lse=lse,
                                    workspace=ws)

    def other():
        binding.ne_rope_attn_decode(q_other, cache, lens, Tcap, Hkv, base, 0, out_dtype=torch.float32, workspace=ws2)

    step()
    torch.cuda.synchronize()
    ref = [o.clone(), lse.clone()]
    g = _capture(step)
    _replays(g, [o, lse], ref, other, [True, True])
