"""fsq_decode_attn_noalloc (the decode call whose workspace is the library's
fixed per-GPU scratch area) against fsq_decode_attn on the same inputs, through
the C ABI: two calls in a row on one GPU, the second with a smaller input, each
bit for bit equal to fsq_decode_attn with a caller workspace and within the
attention bar of the fp64 oracle; sizes that need more scratch than the area
holds are rejected before anything is enqueued."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import fsq_oracle as orc

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3


@pytest.fixture(scope="module")
def fsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fsq_latent_decode_amd as m
    m.lib()
    return m


def _case(seed, B, n_q, n_kv, d_h, G, cap, lens):
    g = synth.rng(230, seed, 0)
    q = synth.normal_bf16(g, (B, n_q, d_h))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    packed = synth.uniform_code_bytes(g, (B, cap), G)
    return q, packed, W, np.asarray(lens, np.int32)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _head_errors(got, ref):
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)


def test_noalloc_matches_workspace_call_twice_then_smaller(fsq):
    # first call: a long ragged batch (streaming kernel, 17 MB of scratch);
    # second: a smaller one (split kernel) that reuses the area the first left
    cases = [(1, 8, 16, 8, 128, 256, 65536, [65536, 4096, 0, 30000, 1, 777, 65535, 12345]),
             (2, 2, 32, 8, 128, 84, 5000, [5000, 33])]
    for seed, B, n_q, n_kv, d_h, G, cap, lens in cases:
        q, packed, W, lens = _case(seed, B, n_q, n_kv, d_h, G, cap, lens)
        assert fsq.decode_workspace_bytes(B, n_q, G, cap) <= fsq.NOALLOC_SCRATCH_BYTES
        qd, cd, Wd = _dev_bf16(q), torch.from_numpy(packed).cuda(), _dev_bf16(W)
        ld = torch.from_numpy(lens).cuda()
        want = torch.empty((B, n_q, d_h), dtype=torch.bfloat16, device="cuda")
        got = torch.full((B, n_q, d_h), float("nan"), dtype=torch.bfloat16, device="cuda")
        fsq.fsq_decode_attn(qd, cd, Wd, ld, want, n_kv)
        fsq.fsq_decode_attn_noalloc(qd, cd, Wd, ld, got, n_kv)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want.cpu()), (seed, "differs from fsq_decode_attn")
        ref = orc.decode_attn(synth.bf16_bits_to_f64(q), packed, synth.bf16_bits_to_f64(W), lens, n_kv, G)
        g64 = got.float().cpu().numpy().astype(np.float64)
        for b in range(B):
            if lens[b] == 0:
                assert np.all(g64[b] == 0)
            else:
                assert float(_head_errors(g64[b], ref[b]).max()) < REL_L2, (seed, b)
        print(f"noalloc call {seed}: B={B} G={G} cap={cap} equal to fsq_decode_attn")


def test_noalloc_rejects_sizes_beyond_the_scratch_area(fsq):
    B, n_q, n_kv, d_h, G, cap = 36, 32, 8, 128, 256, 32768   # all 36 G=256 layers in one call
    assert fsq.decode_workspace_bytes(B, n_q, G, cap) > fsq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, n_q, d_h), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((B, cap, (G + 1) // 2), dtype=torch.uint8, device="cuda")
    W = torch.zeros((2 * n_kv * d_h, G), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    out = torch.full((B, n_q, d_h), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fsq.FsqError, match="WORKSPACE"):
        fsq.fsq_decode_attn_noalloc(q, codes, W, lens, out, n_kv)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)        # nothing was enqueued
