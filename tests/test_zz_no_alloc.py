"""The decode entry point that allocates nothing (ne_rope_attn_decode_noalloc): its split partials go
to the library's own scratch array instead of a caller workspace.  Checked through the C ABI against
ne_rope_attn_decode with a workspace (the same kernels, so the same bits) and against the decode
oracle at the bar of test_gpu_parity.py, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents, which the second must not see)."""
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding
from tests.test_gpu_decode import fill_cache, seqs
from tests.test_gpu_parity import DEV, check, f64

pytestmark = pytest.mark.gpu


def one_call(B, P, Tq, Hq, Hkv, D, lens, window, seed):
    Tcap = (P + 63) // 64 * 64
    q, k, v = seqs(B, P, Hq, Hkv, D, seed, "bf16")
    cache = fill_cache(k, v, Tcap, 1.0e4, (64,) * 1000)
    q_new = torch.stack([q[b, lens[b]:lens[b] + Tq] for b in range(B)]).to(DEV)
    o = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=DEV)
    binding.ne_rope_attn_decode_noalloc(q_new, cache, lens, Tcap, Hkv, 1.0e4, window, o=o, lse=lse)
    ref_o, ref_lse = binding.ne_rope_attn_decode(q_new, cache, lens, Tcap, Hkv, 1.0e4, window)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    ro, rlse = oracle.decode_fwd(f64(q_new.cpu()), [f64(k[b]) for b in range(B)], [f64(v[b]) for b in range(B)],
                                 lens, 1.0e4, window)
    check("o", o.cpu(), ro, torch.bfloat16, torch.float32)
    check("lse", lse.cpu(), rlse, torch.bfloat16, torch.float32)


def test_noalloc_decode_matches_the_workspace_call_twice_in_a_row():
    one_call(4, 1000, 5, 8, 2, 128, [0, 377, 994, 610], 0, 700)
    one_call(2, 300, 1, 4, 2, 64, [299, 41], 100, 710)


def test_noalloc_decode_rejects_partials_beyond_the_scratch():
    """64 sequences of an 8192-token cache (Hq 32, Hkv 8, D 128) need more partials than the scratch
    holds: rejected before anything is enqueued (the cache is never read)."""
    B, Tcap, Hq, Hkv, D = 64, 8192, 32, 8, 128
    assert binding.decode_workspace_bytes(B, 1, Tcap, Hq, Hkv, D, torch.bfloat16) > binding.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    cache = torch.empty(binding.kv_cache_bytes(B, Tcap, Hkv, D, torch.bfloat16), dtype=torch.uint8, device=DEV)
    with pytest.raises(binding.NeError) as e:
        binding.ne_rope_attn_decode_noalloc(q, cache, [0] * B, Tcap, Hkv, 1.0e4)
    assert e.value.status == 5 and "scratch" in str(e.value)
