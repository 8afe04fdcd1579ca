"""Parity of the HIP path (through the C ABI) with the fp64 oracle on seeded inputs.

Bars (the workload's stated tolerances):
  * codes: bit-exact except that at most 1e-4 of them may differ, each by +-1,
    and only where the oracle's bounded value u~ lies within tie_tol of a
    half-integer, tie_tol being the worst-case error of the kernel's fp32
    evaluation of u~ for that code (see tie_tol); at least one such flip is
    allowed in any case (see check_codes);
  * attention output: relative L2 error <= 5e-3 per sequence AND per (sequence,
    query head) (fp32 accumulation, fp16 operands, bf16 output).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import fsq_oracle as orc

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
FLIP_RATE = 1e-4
U32 = 2.0 ** -24          # unit roundoff of fp32


@pytest.fixture(scope="module")
def fsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fsq_latent_decode_amd as m
    m.lib()          # fails loudly if the library is missing
    return m


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def head_rel_l2(got, ref):
    """Relative L2 error of every (sequence, head) output row: [B, n_q]."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return num / den


def check_decode(got, ref, lens, what=""):
    """The attention bar, per sequence AND per (sequence, head).

    A sequence of length 0 must give exactly zero. Otherwise both the relative
    L2 error of the sequence's whole output [n_q, d_h] and that of every head's
    row [d_h] must be below REL_L2: the per-head bound keeps an error confined
    to one head (a wrong GQA mapping, a padded head group, one head's merge)
    from hiding in the pooled norm. Returns and prints the worst of each."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    lens = np.asarray(lens)
    worst_seq, worst_head, where = 0.0, 0.0, None
    for b in range(len(lens)):
        if lens[b] <= 0:
            assert np.all(got[b] == 0), (what, b, "empty sequence must give 0")
            continue
        e = rel_l2(got[b], ref[b])
        hr = head_rel_l2(got[b], ref[b])
        h = int(np.argmax(hr))
        worst_seq = max(worst_seq, e)
        if hr[h] > worst_head:
            worst_head, where = float(hr[h]), (b, h)
        assert e < REL_L2, (what, b, e)
        assert hr[h] < REL_L2, (what, "worst head", b, h, float(hr[h]))
    print(f"{what}: worst sequence rel L2 {worst_seq:.2e}, worst (b, h) {where} {worst_head:.2e}")
    return worst_seq, worst_head


def tie_tol(x, E, levels=16):
    """Per-code bound on |u~_fp32 - u~_exact| for the kernels' evaluation of Eq. 2.

    u = E x: the bf16 products are exact in fp32, and along any path of the
    kernels' sums (MFMA K-blocks of 16 accumulated in order, then at most seven
    cross-wave additions; or, for a few tokens, C/64 terms per lane and six
    cross-lane levels) there are at most d = C/16 + 16 rounded fp32 additions,
    so |du| <= gamma_d sum_i |x_i E_i| with gamma_d = d u / (1 - d u) (the
    standard bound for a floating-point dot product, any summation order of
    depth d). The bound then goes through u~ = h tanh(u + s) - delta, whose
    slope is at most h, plus the fp32 rounding of u + s, tanhf (a few ulp),
    the product by h and the subtraction: <= h (|u| + 8) u_32.
    Returns an array of the codes' shape."""
    h = orc.H_BOUND if levels == 16 else orc.h_of_levels(levels)
    C = x.shape[1]
    d = C / 16 + 16
    gamma = d * U32 / (1 - d * U32)
    s = np.abs(x) @ np.abs(E).T
    u = x @ E.T
    return h * gamma * s + h * (np.abs(u) + 8.0) * U32


def check_codes(gpu_packed, x_bits, E_bits, G, levels=16):
    """Compare GPU codes with the oracle's under the tie rule; return (flips, the
    largest tie distance among them).

    A flip (a code differing by +-1) is allowed only where the oracle's u~ lies
    within tie_tol of a half-integer, i.e. where the fp32 evaluation may land on
    the other side of the rounding threshold. The number of flips must not
    exceed 1e-4 of the codes, but one flip is allowed in any case: whether a
    given case holds a code that close to a threshold is a matter of chance (a
    few codes per million do at C = 4096), so for cases of fewer than 10^4
    codes the allowance is one flip rather than the rate."""
    x = synth.bf16_bits_to_f64(x_bits)
    E = synth.bf16_bits_to_f64(E_bits)
    u = orc.projection(x, E)
    bits = orc.bits_of_levels(levels)
    ref = orc.fsq_codes(u, levels)
    got = orc.unpack_codes(gpu_packed, G, bits)
    # the unused high bits of a token's last byte must be zero
    used = G * bits - 8 * (gpu_packed.shape[1] - 1)
    if used < 8:
        assert np.all(gpu_packed[:, -1] >> used == 0)
    diff = got.astype(int) - ref.astype(int)
    bad = np.nonzero(diff)
    n_bad = len(bad[0])
    assert np.all(np.abs(diff) <= 1), "a code differs by more than 1"
    assert n_bad <= max(1, int(FLIP_RATE * ref.size)), f"{n_bad} flipped codes"
    max_dist = 0.0
    if n_bad:
        ut = orc.fsq_bound(u[bad], h=orc.H_BOUND if levels == 16 else orc.h_of_levels(levels))
        dist = np.abs(ut - (np.floor(ut) + 0.5))
        tol = tie_tol(x, E, levels)[bad]
        assert np.all(dist < tol), f"flip away from a tie: {dist.max()} (bound {tol.min()})"
        max_dist = float(dist.max())
        print(f"{n_bad} flips of {ref.size} codes at L={levels}, largest tie distance {max_dist:.2e} "
              f"(bound there {float(tol[np.argmax(dist)]):.2e})")
    return n_bad, max_dist


def run_append(fsq, x_bits, E_bits, dest_rows=None, row0=0, levels=16):
    n, C = x_bits.shape
    G = E_bits.shape[0]
    P = orc.bytes_per_token(G, orc.bits_of_levels(levels))
    rows = n if dest_rows is None else dest_rows
    cache = torch.full((rows, P), 0xAB, dtype=torch.uint8, device="cuda")
    fsq.fsq_append(dev_bf16(x_bits), dev_bf16(E_bits), cache[row0:row0 + n], levels=levels)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@pytest.mark.parametrize("n,C,G", [
    (1, 1024, 64), (5, 512, 83), (17, 256, 7), (31, 4096, 84),     # vector path
    (32, 1024, 64), (33, 1024, 64), (100, 520, 84), (1024, 1024, 64),  # MFMA path, ragged tails
    (257, 2048, 256), (64, 8, 3), (96, 24, 1),
    # register-staged kernel: two batches in flight (GP = 128), all-zero batches
    # that round the batch count up to a multiple of four (C = 1288: 6 -> 8), a
    # k tail inside a batch, many batches at the smallest width
    (70, 1288, 128), (45, 4096, 120), (40, 1288, 96), (300, 4096, 20),
    # widths above 128: 128-wide k-batches, sums reduced in passes of 128 codes
    (45, 136, 161), (64, 8, 200), (96, 4096, 224), (300, 2056, 256),
])
def test_append_parity(fsq, n, C, G):
    g = synth.rng(100, n, C + G)
    x = synth.normal_bf16(g, (n, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    got = run_append(fsq, x, E)
    check_codes(got, x, E, G)


# L = 4 and 256 levels (2- and 8-bit codes): the vector (n < 32) and MFMA paths,
# odd G and G not a multiple of the codes per byte
@pytest.mark.parametrize("levels", [4, 256])
@pytest.mark.parametrize("n,C,G", [
    (1, 1024, 64), (5, 512, 83), (31, 4096, 84), (32, 1024, 64), (100, 520, 84), (257, 2048, 256),
    (64, 8, 3), (40, 256, 42), (33, 512, 168), (70, 1288, 250), (96, 4096, 168),
])
def test_append_levels_parity(fsq, levels, n, C, G):
    g = synth.rng(102, n + levels, C + G)
    x = synth.normal_bf16(g, (n, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    got = run_append(fsq, x, E, levels=levels)
    check_codes(got, x, E, G, levels)


def test_append_into_cache_rows_keeps_other_rows(fsq):
    g = synth.rng(101, 0, 0)
    x = synth.normal_bf16(g, (40, 256))
    E = synth.normal_bf16(g, (84, 256), 1 / 16)
    got = run_append(fsq, x, E, dest_rows=50, row0=3)          # row offset 3*42: 2-byte aligned
    assert np.all(got[:3] == 0xAB) and np.all(got[43:] == 0xAB)
    check_codes(got[3:43], x, E, 84)
    got1 = run_append(fsq, x[:1], E, dest_rows=5, row0=3)       # one-token (decode-step) append
    assert np.all(got1[:3] == 0xAB) and np.all(got1[4:] == 0xAB)
    check_codes(got1[3:4], x[:1], E, 84)


def test_append_prefill_chunk_g84(fsq):
    """The 8192-token prefill chunk of the G=84 Qwen3-8B workload, full size."""
    w = synth.WORKLOADS["qwen3_8b_g84"]
    E, _ = synth.layer_weights(w, 0)
    x = synth.layer_x(w, 0, w.append_tokens)
    got = run_append(fsq, x, E)
    flips, dist = check_codes(got, x, E, w.G)
    print(f"g84 prefill chunk: {flips} of {x.shape[0] * w.G} codes at fp32 ties (largest tie distance {dist:.2e})")


@pytest.mark.parametrize("G,levels", [(256, 16), (168, 4)])
def test_append_prefill_chunk_wide(fsq, G, levels):
    """An 8192 x 4096 prefill chunk at the widths whose append takes 128-wide
    k-batches and sums the waves in passes of 128 codes: G = 256 (4 bits, the
    32x operating point) and G = 168 at 2 bits (the G=84 byte budget)."""
    g = synth.rng(104, G, levels)
    x = synth.normal_bf16(g, (8192, 4096))
    E = synth.normal_bf16(g, (G, 4096), 1.0 / 64.0)
    got = run_append(fsq, x, E, levels=levels)
    flips, dist = check_codes(got, x, E, G, levels)
    print(f"G={G} L={levels} prefill chunk: {flips} of {x.shape[0] * G} codes at fp32 ties "
          f"(largest tie distance {dist:.2e})")


@pytest.mark.parametrize("G", [84, 256])
def test_append_position_in_call(fsq, G):
    """A token's codes do not depend on where it sits in the call beyond the tie
    rule: the CTA of 32 tokens that holds it starts its k-batches at its own
    index mod C / KPB, so the same rows appended after 32 and after 40 other
    rows go through other CTAs, other batch orders and other tile rows. Both
    calls are checked against the oracle, and against each other, where a code
    may differ only if one of them is a flip."""
    g = synth.rng(105, G, 0)
    n, C = 300, 2048
    x = synth.normal_bf16(g, (n + 40, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    a = run_append(fsq, x[40:], E)                       # rows 0.. of the call
    assert np.array_equal(a, run_append(fsq, x[40:], E)), "a repeated append call changed bits"
    b = run_append(fsq, x[8:], E)[32:]                   # the same rows after 32 others
    c = run_append(fsq, x, E)[40:]                       # ... and after 40 others
    for got in (a, b, c):
        check_codes(got, x[40:], E, G)
    P = a.shape[1]
    da = orc.unpack_codes(a, G, 4).astype(int)
    for other in (b, c):
        do = orc.unpack_codes(other, G, 4).astype(int)
        assert np.all(np.abs(da - do) <= 1)
        allowed = 2 * max(1, int(FLIP_RATE * da.size))   # each side's tie flips against the oracle
        assert np.count_nonzero(da != do) <= allowed, "positions in the call changed codes beyond the tie flips"
    assert a.shape == (n, P)


# ------------------------------------------------------------------ decode
def run_decode(fsq, q_bits, packed, W_bits, lens, n_kv, workspace=None):
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn(q, dev_u8(packed), dev_bf16(W_bits),
                        torch.from_numpy(np.asarray(lens, np.int32)).cuda(), out, n_kv,
                        workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_decode(q_bits, packed, W_bits, lens, n_kv, G):
    q = synth.bf16_bits_to_f64(q_bits)
    W = synth.bf16_bits_to_f64(W_bits)
    return orc.decode_attn(q, packed, W, lens, n_kv, G)


def decode_case(seed, B, n_q, n_kv, d_h, G, cap, lens):
    g = synth.rng(200, seed, 0)
    q = synth.normal_bf16(g, (B, n_q, d_h))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    packed = synth.uniform_code_bytes(g, (B, cap), G)
    return q, packed, W, np.asarray(lens, np.int32)


@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens", [
    (1, 16, 8, 128, 64, 1024, [1024]),          # the tiny single-layer workload shape
    (1, 32, 8, 128, 256, 1, [1]),
    (1, 32, 8, 128, 256, 33, [33]),
    (1, 32, 8, 128, 84, 700, [700]),
    (2, 32, 8, 128, 84, 1000, [1000, 257]),
    (4, 16, 8, 128, 256, 600, [0, 1, 31, 600]),
    (1, 64, 8, 128, 64, 300, [300]),             # two 32-head groups
    (1, 8, 1, 64, 37, 130, [129]),               # MQA, odd G, d_h 64
    (3, 12, 4, 96, 96, 2100, [2100, 1500, 33]),
    (1, 32, 8, 128, 160, 5000, [4999]),
    (1, 8, 2, 256, 64, 100, [100]),              # d_h 256: one thread per output row
    (2, 16, 4, 64, 30, 300, [300, 7]),           # G % 4 == 2: 4-byte W_v loads
    (1, 8, 2, 128, 131, 64, [64]),               # odd G: W_v vectors past the register set
    (1, 4, 1, 128, 130, 90, [90]),               # G % 4 == 2: the same with 2-wide vectors
    (1, 32, 8, 128, 20, 131072, [131072]),       # G = 20 (409.6x, 10 B/token)
    (1, 32, 8, 128, 32, 131072, [131000]),       # G = 32 (256x, 16 B/token)
    # widths 64 and 96 over >= 2 x 256 x 256 tokens of work: 8-wave split CTAs
    # of two or more rounds (ragged, unaligned rows, a chunk ending mid-round)
    (2, 32, 8, 128, 64, 65600, [65600, 40001]),
    (1, 32, 8, 128, 84, 131072, [130999]),
    (3, 16, 8, 128, 90, 50000, [50000, 9, 33333]),
    # one query head per kv head: four sequences share an absorption CTA (the
    # last group partial), 24 padded query rows each
    (5, 8, 8, 64, 64, 300, [300, 1, 0, 77, 256]),
    # widths above 128 with 129..256 splits: the one-barrier merge with 8 splits
    # per lane (196 splits: the last lanes' slots partly past the sequence)
    (1, 32, 8, 128, 256, 65536, [65536]),
    (1, 32, 8, 128, 200, 100000, [99999]),
    # the narrowest latents: one or two codes per token, 30-31 zero-padded
    # coordinates of the 32-wide operand
    (2, 8, 2, 64, 1, 200, [200, 3]),
    (1, 16, 8, 128, 2, 5000, [4999]),
])
def test_decode_parity(fsq, B, n_q, n_kv, d_h, G, cap, lens):
    q, packed, W, lens = decode_case(G * 7 + cap, B, n_q, n_kv, d_h, G, cap, lens)
    got = run_decode(fsq, q, packed, W, lens, n_kv)
    ref = oracle_decode(q, packed, W, lens, n_kv, G)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


# Caches whose capacity (batch x seq_cap) is large enough for the streaming
# split-K kernel (every wave gets at least 4 tiles of 32 tokens: more than
# 196608 tokens at GP >= 128, 393216 below; the test checks the plan), with
# lengths mostly far shorter than the capacity so the oracle stays cheap: empty
# and one-token sequences, tails inside a tile, sequences spanning several
# chunks, odd capacities (rows of a sequence not 16-byte aligned), odd G, every
# pooling block count 1..8, and two head groups.
@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens", [
    (2, 32, 8, 128, 256, 131072, [3000, 1]),
    (2, 32, 8, 128, 256, 131072, [20000, 4097]),
    (4, 32, 8, 128, 84, 131072, [0, 5000, 700, 12345]),
    (4, 32, 8, 128, 64, 131072, [0, 5000, 700, 12345]),   # whole 1024-token items at widths 64, 32
    (4, 32, 8, 128, 32, 131072, [0, 5000, 700, 12345]),
    (4, 32, 8, 128, 84, 131073, [65537, 1, 31, 33]),
    (4, 16, 8, 128, 64, 131072, [1000, 65536, 0, 2]),
    (4, 8, 1, 64, 37, 131072, [3001, 129, 1, 64]),
    (2, 40, 8, 128, 200, 131072, [7000, 333]),
    (2, 32, 8, 128, 160, 131072, [9999, 65536]),
    (2, 32, 4, 128, 128, 131072, [4096, 100]),
    (4, 32, 8, 128, 32, 131072, [2000, 1, 0, 513]),
    (4, 64, 8, 128, 96, 131072, [1500, 4000, 10, 600]),
    (3, 16, 8, 128, 256, 131071, [65521, 40000, 77]),
])
def test_decode_stream_parity(fsq, B, n_q, n_kv, d_h, G, cap, lens):
    assert fsq.decode_plan(B, n_q, G, cap)["kernel"] == "decode_stream_kernel"
    q, packed, W, lens = decode_case(G * 13 + cap, B, n_q, n_kv, d_h, G, cap, lens)
    got = run_decode(fsq, q, packed, W, lens, n_kv)
    ref = oracle_decode(q, packed, W, lens, n_kv, G)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


# The device-side split of streaming calls (up to 64 sequences): the chunk
# comes from the sum of the actual lengths, and consecutive work items cover
# the sequences in order, so very uneven batches, empty sequences, a length far
# below the capacity, the 64-sequence limit and the static split just past it
# (65 sequences) all take different item layouts.
@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens", [
    (64, 8, 2, 64, 32, 8192, "skew"),
    (65, 8, 2, 64, 32, 8192, "skew"),
    (8, 16, 8, 128, 84, 65536, [0, 0, 60000, 3, 0, 129, 0, 5]),
    (8, 16, 8, 128, 84, 65536, [0] * 8),                 # nothing to attend to anywhere
    (1, 32, 8, 128, 84, 1 << 20, [300001]),
    (6, 16, 4, 128, 256, 65536, [1, 2, 3, 4, 5, 65536]),
])
def test_decode_stream_device_split_parity(fsq, B, n_q, n_kv, d_h, G, cap, lens):
    if lens == "skew":
        g = synth.rng(201, B, 0)
        lens = [int(x) for x in g.integers(0, 3000, size=B)]
        lens[3], lens[10], lens[B - 1] = 0, 8192, 1
    q, packed, W, lens = decode_case(G * 7 + cap + B, B, n_q, n_kv, d_h, G, cap, lens)
    assert fsq.decode_plan(B, n_q, G, cap)["kernel"] == "decode_stream_kernel"
    got = run_decode(fsq, q, packed, W, lens, n_kv)
    ref = oracle_decode(q, packed, W, lens, n_kv, G)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


def test_decode_stream_deterministic(fsq):
    assert fsq.decode_plan(4, 32, 84, 131072)["kernel"] == "decode_stream_kernel"
    q, packed, W, lens = decode_case(8, 4, 32, 8, 128, 84, 131072, [30000, 17, 65536, 4100])
    a = run_decode(fsq, q, packed, W, lens, 8)
    b = run_decode(fsq, q, packed, W, lens, 8)
    assert np.array_equal(a, b)


def run_decode_recon(fsq, q_bits, packed, W_bits, lens, n_kv):
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn_recon(q, dev_u8(packed), dev_bf16(W_bits),
                              torch.from_numpy(np.asarray(lens, np.int32)).cuda(), out, n_kv)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# The key-reconstruction variant (keys rebuilt per tile instead of absorbed
# queries) against the same oracle: short and long caches, odd G, every d_h it
# takes (32..128), MQA and wide GQA groups, empty and one-token sequences.
@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens", [
    (1, 16, 8, 128, 64, 1024, [1024]),
    (1, 32, 8, 128, 256, 33, [33]),
    (2, 32, 8, 128, 84, 1000, [1000, 257]),
    (4, 16, 8, 128, 256, 600, [0, 1, 31, 600]),
    (1, 8, 1, 64, 37, 130, [129]),
    (3, 12, 4, 96, 96, 2100, [2100, 1500, 33]),
    (1, 32, 8, 128, 160, 5000, [4999]),
    (2, 16, 4, 32, 30, 300, [300, 7]),
    (1, 32, 1, 128, 200, 700, [699]),
    (2, 32, 8, 128, 256, 65536, [20000, 4097]),
    (4, 32, 8, 128, 84, 65537, [65537, 1, 31, 33]),
])
def test_decode_recon_parity(fsq, B, n_q, n_kv, d_h, G, cap, lens):
    q, packed, W, lens = decode_case(G * 11 + cap, B, n_q, n_kv, d_h, G, cap, lens)
    got = run_decode_recon(fsq, q, packed, W, lens, n_kv)
    ref = oracle_decode(q, packed, W, lens, n_kv, G)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


def test_decode_recon_deterministic(fsq):
    q, packed, W, lens = decode_case(9, 2, 32, 8, 128, 84, 9000, [9000, 4097])
    a = run_decode_recon(fsq, q, packed, W, lens, 8)
    assert np.array_equal(a, run_decode_recon(fsq, q, packed, W, lens, 8))


def run_decode_rope(fsq, q_bits, packed, W_bits, gam_bits, lens, n_kv, theta, eps):
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn_rope(q, dev_u8(packed), dev_bf16(W_bits), dev_bf16(gam_bits),
                             torch.from_numpy(np.asarray(lens, np.int32)).cuda(), out, n_kv, theta, eps)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# Eq. 5 keys in full (key RMS norm with a seeded gain, RoPE at each cache
# position, theta 1e6 / 1e4, eps 1e-6) against the oracle: positions up to
# 65536 check the rotation angles far from 0.
@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens,theta", [
    (1, 32, 8, 128, 256, 1024, [1024], 1e6),
    (2, 32, 8, 128, 84, 1000, [1000, 1], 1e6),
    (4, 16, 8, 128, 256, 600, [0, 1, 31, 600], 1e4),
    (1, 8, 1, 64, 37, 130, [129], 1e4),
    (3, 12, 4, 64, 96, 2100, [2100, 1500, 33], 1e6),
    (2, 32, 8, 128, 256, 65536, [65536, 4097], 1e6),
    (4, 32, 8, 128, 84, 65537, [65537, 1, 31, 33], 1e6),
])
def test_decode_rope_parity(fsq, B, n_q, n_kv, d_h, G, cap, lens, theta):
    q, packed, W, lens = decode_case(G * 17 + cap, B, n_q, n_kv, d_h, G, cap, lens)
    gam = synth.normal_bf16(synth.rng(300, d_h, 0), (d_h,), 0.1)
    gam = synth.f32_to_bf16_bits(synth.bf16_bits_to_f64(gam).astype(np.float32) + 1.0)
    got = run_decode_rope(fsq, q, packed, W, gam, lens, n_kv, theta, 1e-6)
    ref = orc.decode_attn_rope(synth.bf16_bits_to_f64(q), packed, synth.bf16_bits_to_f64(W), lens, n_kv,
                               G, synth.bf16_bits_to_f64(gam), 1e-6, theta)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


def run_decode_levels(fsq, q_bits, packed, W_bits, lens, n_kv, levels):
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn_levels(q, dev_u8(packed), dev_bf16(W_bits),
                               torch.from_numpy(np.asarray(lens, np.int32)).cuda(), out, n_kv, levels)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# Decode over 2- and 8-bit code caches (L = 4, 256): aligned and unaligned
# rows, odd G, ragged and empty sequences, long caches (the split kernel
# streams them in several rounds), the same byte budget as G = 84 at 4 bits.
@pytest.mark.parametrize("levels", [4, 256])
@pytest.mark.parametrize("B,n_q,n_kv,d_h,G,cap,lens", [
    (1, 16, 8, 128, 64, 1024, [1024]),
    (2, 32, 8, 128, 84, 1000, [1000, 257]),
    (4, 16, 8, 128, 256, 600, [0, 1, 31, 600]),
    (1, 8, 1, 64, 37, 130, [129]),
    (1, 32, 8, 128, 128, 5000, [4999]),
    (2, 32, 8, 128, 20, 3000, [3000, 17]),
    (1, 32, 8, 128, 32, 70000, [70000]),
    (2, 32, 8, 128, 64, 65600, [65600, 40001]),  # 8-wave split CTAs (widths 64, 96 on long work)
    (1, 32, 8, 128, 84, 131072, [130999]),
    (1, 32, 8, 128, 168, 131072, [131072]),      # the 2-bit operating point's width: 256 splits, 8 per merge lane
    (2, 8, 2, 64, 1, 300, [300, 2]),               # one code per token
])
def test_decode_levels_parity(fsq, levels, B, n_q, n_kv, d_h, G, cap, lens):
    g = synth.rng(210, levels, G + cap)
    q = synth.normal_bf16(g, (B, n_q, d_h))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    bits = orc.bits_of_levels(levels)
    packed = synth.uniform_code_bytes(g, (B, cap), G, bits)
    lens = np.asarray(lens, np.int32)
    got = run_decode_levels(fsq, q, packed, W, lens, n_kv, levels)
    ref = orc.decode_attn(synth.bf16_bits_to_f64(q), packed, synth.bf16_bits_to_f64(W), lens, n_kv, G,
                          levels=levels)
    check_decode(got, ref, lens, f"B={B} n_q={n_q} G={G} cap={cap}")


@pytest.mark.parametrize("levels", [4, 16, 256])
def test_timed_decode_is_bitwise_the_untimed_one(fsq, levels):
    """The event-timed entry points give the untimed results bit for bit, and
    their events bracket a positive duration."""
    B, n_q, n_kv, d_h, G, cap = 2, 32, 8, 128, 84, 3000
    g = synth.rng(211, levels, 0)
    q = dev_bf16(synth.normal_bf16(g, (B, n_q, d_h)))
    W = dev_bf16(synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G)))
    codes = dev_u8(synth.uniform_code_bytes(g, (B, cap), G, orc.bits_of_levels(levels)))
    lens = torch.tensor([3000, 1234], dtype=torch.int32, device="cuda")
    outs = []
    for timed in (False, True):
        out = torch.empty((B, n_q, d_h), dtype=torch.bfloat16, device="cuda")
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
        if levels == 16:
            fsq.fsq_decode_attn(q, codes, W, lens, out, n_kv, split_events=ev)
        else:
            fsq.fsq_decode_attn_levels(q, codes, W, lens, out, n_kv, levels, split_events=ev)
        torch.cuda.synchronize()
        if timed:
            assert ev[0].elapsed_time(ev[1]) > 0
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("levels,G", [(4, 168), (256, 42)])
def test_levels_append_then_decode_at_the_g84_byte_budget(fsq, levels, G):
    """42 bytes per token (the G = 84 budget) spent on 2- or 8-bit codes:
    append 2000 tokens through the library, decode, compare with the oracle's
    encode-then-decode."""
    g = synth.rng(211, levels, G)
    C, n_q, n_kv, d_h, T = 1024, 32, 8, 128, 2000
    x = synth.normal_bf16(g, (T, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    q = synth.normal_bf16(g, (1, n_q, d_h))
    got_codes = run_append(fsq, x, E, levels=levels)
    assert got_codes.shape[1] == 42
    check_codes(got_codes, x, E, G, levels)
    got = run_decode_levels(fsq, q, got_codes[None], W, [T], n_kv, levels)
    bits = orc.bits_of_levels(levels)
    ref_codes = orc.pack_codes(orc.encode(synth.bf16_bits_to_f64(x), synth.bf16_bits_to_f64(E), levels), bits)
    ref = orc.decode_attn(synth.bf16_bits_to_f64(q), ref_codes[None], synth.bf16_bits_to_f64(W), [T], n_kv, G,
                          levels=levels)
    check_decode(got, ref, [T], f"L={levels} G={G} append then decode")


def test_decode_deterministic(fsq):
    """Run-to-run: the same call twice gives the same bits (fixed merge order)."""
    q, packed, W, lens = decode_case(5, 2, 32, 8, 128, 84, 9000, [9000, 4097])
    a = run_decode(fsq, q, packed, W, lens, 8)
    b = run_decode(fsq, q, packed, W, lens, 8)
    assert np.array_equal(a, b)
    check_decode(a, oracle_decode(q, packed, W, lens, 8, 84), lens, "deterministic")


# Split-count invariance (the result must not depend on how the tokens are
# split): one 9000-token sequence (a tail of 8 tokens in its last tile) placed
# in caches of growing capacity. The plan depends on the capacity, so the same
# tokens are split into different chunk lengths and counts, by 4- and 8-wave
# CTAs of the split kernel and, at the largest capacity, by the streaming
# kernel with the split chosen on the device. Rows past the length hold other
# random codes and must not matter.
@pytest.mark.parametrize("G,caps", [
    (84, [9000, 70000, 200000, 400000]),
    (256, [9000, 70000, 150000, 200000]),
])
def test_decode_split_count_invariance(fsq, G, caps):
    T, n_q, n_kv, d_h = 9000, 32, 8, 128
    g = synth.rng(220, G, 0)
    q = synth.normal_bf16(g, (1, n_q, d_h))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    seq = synth.uniform_code_bytes(g, (1, T), G)
    plans = [fsq.decode_plan(1, n_q, G, cap) for cap in caps]
    keys = {(p["kernel"], p["device_split"], p["splits"], p["chunk"]) for p in plans}
    assert len(keys) == len(caps), plans                       # four different splits
    assert plans[-1]["kernel"] == "decode_stream_kernel" and plans[0]["kernel"] == "decode_split_kernel"
    ref = oracle_decode(q, seq, W, [T], n_kv, G)
    outs = []
    for cap, plan in zip(caps, plans):
        packed = np.concatenate([seq, synth.uniform_code_bytes(synth.rng(221, G, cap), (1, cap - T), G)], axis=1)
        a = run_decode(fsq, q, packed, W, [T], n_kv)
        assert np.array_equal(a, run_decode(fsq, q, packed, W, [T], n_kv)), plan   # and bitwise repeatable
        check_decode(a, ref, [T], f"G={G} cap={cap} {plan}")
        outs.append(a)
    # the results of the different splits agree with each other within the bar,
    # per head; they differ only by the rounding of the fp16 partial states
    worst = 0.0
    for i in range(len(outs)):
        for j in range(i + 1, len(outs)):
            worst = max(worst, float(head_rel_l2(outs[i][0], outs[j][0]).max()))
    print(f"G={G}: largest per-head rel L2 between two splits {worst:.2e}")
    assert worst < REL_L2


def test_decode_workspace_reuse_across_calls(fsq):
    """Two calls with different inputs through one workspace: the second result
    must match the oracle for the second inputs (no stale partial state)."""
    ws = fsq.alloc_workspace(1, 32, 256, 4096)
    for seed in (11, 12):
        q, packed, W, lens = decode_case(seed, 1, 32, 8, 128, 256, 4096, [4096 - seed])
        got = run_decode(fsq, q, packed, W, lens, 8, workspace=ws)
        check_decode(got, oracle_decode(q, packed, W, lens, 8, 256), lens, f"workspace reuse, call {seed}")


def test_decode_on_side_stream_without_workspace(fsq):
    """A call on an explicit side stream with no workspace: the binding allocates
    the workspace on that stream, so memory the current stream allocates and
    writes right after the call returns cannot be the workspace the queued
    kernels still use. Repeated with a raw stream handle."""
    q, packed, W, lens = decode_case(13, 2, 32, 8, 128, 256, 20000, [20000, 777])
    ref = oracle_decode(q, packed, W, lens, 8, 256)
    nbytes = fsq.decode_workspace_bytes(2, 32, 256, 20000)
    qd, cd, Wd = dev_bf16(q), dev_u8(packed), dev_bf16(W)
    ld = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    torch.cuda.synchronize()
    for as_handle in (False, True):
        side = torch.cuda.Stream()
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        side.wait_stream(torch.cuda.current_stream())
        fsq.fsq_decode_attn(qd, cd, Wd, ld, out, 8, stream=side.cuda_stream if as_handle else side)
        junk = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)                    # would overwrite a workspace taken from this stream's pool
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        check_decode(out.float().cpu().numpy().astype(np.float64), ref, lens, f"side stream (handle={as_handle})")
        del junk


def test_decode_workspace_too_small_raises(fsq):
    q, packed, W, lens = decode_case(6, 1, 32, 8, 128, 64, 100, [100])
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(fsq.FsqError, match="WORKSPACE"):
        run_decode(fsq, q, packed, W, lens, 8, workspace=ws)


def test_tiny_workload_append_then_decode(fsq):
    """The tiny workload end to end: append the 1024-token context, then decode
    one query, compared with the oracle's encode-then-decode."""
    w = synth.WORKLOADS["tiny"]
    E, W = synth.layer_weights(w, 0)
    x = synth.layer_x(w, 0, w.append_tokens)
    q = synth.layer_query(w, 0)
    got_codes = run_append(fsq, x, E)
    check_codes(got_codes, x, E, w.G)
    out = torch.empty((1, w.n_q, w.d_h), dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn(dev_bf16(q), dev_u8(got_codes[None]), dev_bf16(W),
                        torch.tensor([w.context], dtype=torch.int32, device="cuda"), out, w.n_kv)
    torch.cuda.synchronize()
    ref_codes = orc.pack_codes(orc.encode(synth.bf16_bits_to_f64(x), synth.bf16_bits_to_f64(E)))
    ref = oracle_decode(q, ref_codes[None], W, [w.context], w.n_kv, w.G)
    check_decode(out.float().cpu().numpy(), ref, [w.context], "tiny workload")


@pytest.mark.parametrize("name", ["qwen3_8b_g256", "qwen3_8b_g84"])
def test_decode_full_size_layer(fsq, name):
    """One layer of the Qwen3-8B-shaped workloads at full context (layers 0 and last)."""
    w = synth.WORKLOADS[name]
    for layer in (0, w.layers - 1):
        _, W = synth.layer_weights(w, layer)
        q = synth.layer_query(w, layer)
        lens = synth.seq_lens(w)
        packed = synth.layer_codes(w, layer)
        got = run_decode(fsq, q, packed, W, lens, w.n_kv)
        ref = oracle_decode(q, packed, W, lens, w.n_kv, w.G)
        check_decode(got, ref, lens, f"{name} layer {layer}")


def test_decode_ragged_batch_full_size(fsq):
    """The ragged Qwen3-1.7B-shaped batch (16 sequences, 4096..65536 tokens), layer 0."""
    w = synth.WORKLOADS["qwen3_1p7b_ragged"]
    _, W = synth.layer_weights(w, 0)
    q = synth.layer_query(w, 0)
    lens = synth.seq_lens(w)
    packed = synth.layer_codes(w, 0, lens=lens)
    got = run_decode(fsq, q, packed, W, lens, w.n_kv)
    ref = oracle_decode(q, packed, W, lens, w.n_kv, w.G)
    check_decode(got, ref, lens, "ragged Qwen3-1.7B batch, layer 0")


# ------------------------------------------------------------- decode step
def run_step(fsq, x_bits, E_bits, q_bits, packed, W_bits, lens, n_kv, workspace=None):
    codes = dev_u8(packed)
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_step(dev_bf16(x_bits), dev_bf16(E_bits), q, codes, dev_bf16(W_bits),
                        torch.from_numpy(np.asarray(lens, np.int32)).cuda(), out, n_kv,
                        workspace=workspace)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), out.float().cpu().numpy().astype(np.float64)


def run_two_calls(fsq, x_bits, E_bits, q_bits, packed, W_bits, lens, n_kv):
    """fsq_append of each sequence's new row (one token per call), then fsq_decode_attn."""
    codes = dev_u8(packed)
    cap = packed.shape[1]
    x = dev_bf16(x_bits)
    E = dev_bf16(E_bits)
    for b, T in enumerate(lens):
        if 1 <= T <= cap:
            fsq.fsq_append(x[b:b + 1], E, codes[b, T - 1:T])
    q = dev_bf16(q_bits)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn(q, codes, dev_bf16(W_bits), torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                        out, n_kv)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), out.float().cpu().numpy().astype(np.float64)


def check_step(got_codes, got_out, x, E, q, packed, W, lens, n_kv, G):
    """Appended rows vs the oracle's codes (tie rule), other rows untouched, and
    the output vs the oracle's decode of the oracle-appended cache."""
    cap = packed.shape[1]
    app = [b for b, T in enumerate(lens) if 1 <= T <= cap]
    ref_cache = packed.copy()
    if app:
        rows = np.stack([got_codes[b, lens[b] - 1] for b in app])
        check_codes(rows, x[app], E, G)
        new = orc.pack_codes(orc.encode(synth.bf16_bits_to_f64(x[app]), synth.bf16_bits_to_f64(E)))
        for i, b in enumerate(app):
            ref_cache[b, lens[b] - 1] = new[i]
    mask = np.ones(packed.shape[:2], bool)
    for b in app:
        mask[b, lens[b] - 1] = False
    assert np.array_equal(got_codes[mask], packed[mask]), "a row other than the new token's changed"
    eff = np.minimum(np.maximum(lens, 0), cap)
    ref = oracle_decode(q, ref_cache, W, eff, n_kv, G)
    check_decode(got_out, ref, eff, f"decode step B={len(lens)} G={G} cap={cap}")


@pytest.mark.parametrize("B,C,n_q,n_kv,d_h,G,cap,lens", [
    (1, 1024, 16, 8, 128, 64, 1024, [1024]),
    (2, 512, 32, 8, 128, 84, 700, [700, 1]),                        # 2 tokens per append CTA
    (3, 256, 12, 4, 96, 37, 300, [0, 300, 299]),                    # 4 per CTA, odd G, empty sequence
    (5, 4096, 32, 8, 128, 256, 400, [400, 17, 1, 0, 250]),          # 8 per CTA
    (9, 64, 8, 2, 64, 96, 100, [100, 5, 0, 1, 64, 33, 99, 100, 2]),  # two CTAs of 8 tokens per byte
    (2, 64, 8, 1, 64, 30, 50, [60, 50]),                            # length > cap: no append, clamped
    (6, 256, 16, 8, 128, 64, 200, [200, 3, 0, 150, 1, 77]),         # 2 sequences per absorption CTA
    (5, 128, 4, 4, 64, 32, 90, [90, 1, 50, 0, 2]),                  # 4 per absorption CTA, last group of 1
    (3, 256, 8, 2, 64, 1, 120, [120, 1, 60]),                       # one code per token (half a byte)
])
def test_decode_step_parity(fsq, B, C, n_q, n_kv, d_h, G, cap, lens):
    q, packed, W, lens = decode_case(G * 11 + cap + B, B, n_q, n_kv, d_h, G, cap, lens)
    g = synth.rng(210, B, G + cap)
    x = synth.normal_bf16(g, (B, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    got_codes, got_out = run_step(fsq, x, E, q, packed, W, lens, n_kv)
    check_step(got_codes, got_out, x, E, q, packed, W, lens, n_kv, G)
    two_codes, two_out = run_two_calls(fsq, x, E, q, packed, W, lens, n_kv)
    assert np.array_equal(got_codes, two_codes)
    assert np.array_equal(got_out, two_out)


@pytest.mark.parametrize("levels", [4, 256])
@pytest.mark.parametrize("B,C,n_q,n_kv,d_h,G,cap,lens", [
    (1, 1024, 16, 8, 128, 64, 1024, [1024]),
    (3, 256, 12, 4, 96, 37, 300, [0, 300, 299]),                    # odd G, an empty sequence
    (5, 4096, 32, 8, 128, 168, 400, [400, 17, 1, 0, 250]),          # the 2-bit operating point's width
    (9, 64, 8, 2, 64, 42, 100, [100, 5, 0, 1, 64, 33, 99, 100, 2]),  # the 8-bit operating point's width
    (2, 64, 8, 1, 64, 30, 50, [60, 50]),                            # length > cap: no append
    (3, 256, 8, 2, 64, 1, 120, [120, 1, 60]),                       # one code per token
])
def test_decode_step_levels_parity(fsq, levels, B, C, n_q, n_kv, d_h, G, cap, lens):
    """fsq_decode_step with 2- and 8-bit codes: the appended rows against the
    oracle (tie rule), every other row untouched, the output against the
    oracle's decode of the oracle-appended cache, and bit-identical results to
    fsq_append (one token per call) followed by fsq_decode_attn_levels."""
    bits = orc.bits_of_levels(levels)
    g = synth.rng(212, levels * 7 + B, G + cap)
    q = synth.normal_bf16(g, (B, n_q, d_h))
    W = synth.normal_bf16(g, (2 * n_kv * d_h, G), 1.0 / math.sqrt(G))
    packed = synth.uniform_code_bytes(g, (B, cap), G, bits)
    x = synth.normal_bf16(g, (B, C))
    E = synth.normal_bf16(g, (G, C), 1.0 / math.sqrt(C))
    lens = np.asarray(lens, np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    codes = dev_u8(packed)
    out = torch.empty((B, n_q, d_h), dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_step(dev_bf16(x), dev_bf16(E), dev_bf16(q), codes, dev_bf16(W), lens_d, out, n_kv,
                        levels=levels)
    codes2 = dev_u8(packed)
    for b, T in enumerate(lens):
        if 1 <= T <= cap:
            fsq.fsq_append(dev_bf16(x[b:b + 1]), dev_bf16(E), codes2[b, T - 1:T], levels=levels)
    out2 = torch.empty_like(out)
    fsq.fsq_decode_attn_levels(dev_bf16(q), codes2, dev_bf16(W), lens_d, out2, n_kv, levels)
    torch.cuda.synchronize()
    got_codes = codes.cpu().numpy()
    assert np.array_equal(got_codes, codes2.cpu().numpy()), "step and two-call appends differ"
    assert torch.equal(out, out2), "step and two-call outputs differ"
    app = [b for b, T in enumerate(lens) if 1 <= T <= cap]
    ref_cache = packed.copy()
    if app:
        rows = np.stack([got_codes[b, lens[b] - 1] for b in app])
        check_codes(rows, x[app], E, G, levels)
        new = orc.pack_codes(orc.encode(synth.bf16_bits_to_f64(x[app]), synth.bf16_bits_to_f64(E), levels),
                             bits)
        for i, b in enumerate(app):
            ref_cache[b, lens[b] - 1] = new[i]
    mask = np.ones(packed.shape[:2], bool)
    for b in app:
        mask[b, lens[b] - 1] = False
    assert np.array_equal(got_codes[mask], packed[mask]), "a row other than the new token's changed"
    eff = np.minimum(np.maximum(lens, 0), cap)
    ref = orc.decode_attn(synth.bf16_bits_to_f64(q), ref_cache, synth.bf16_bits_to_f64(W), eff, n_kv, G,
                          levels=levels)
    check_decode(out.float().cpu().numpy().astype(np.float64), ref, eff,
                 f"decode step L={levels} B={B} G={G} cap={cap}")


@pytest.mark.parametrize("name", ["qwen3_8b_g256", "qwen3_8b_g84"])
def test_decode_step_full_size_layer(fsq, name):
    """One decode step of layer 0 of the Qwen3-8B-shaped workloads at full context,
    as the benchmark runs it: the new token is appended at row T - 1."""
    w = synth.WORKLOADS[name]
    E, W = synth.layer_weights(w, 0)
    q = synth.layer_query(w, 0)
    x = synth.layer_x(w, 0, w.batch, synth.T_XNEW)
    lens = synth.seq_lens(w)
    packed = synth.layer_codes(w, 0)
    got_codes, got_out = run_step(fsq, x, E, q, packed, W, lens, w.n_kv)
    check_step(got_codes, got_out, x, E, q, packed, W, lens, w.n_kv, w.G)


def test_million_token_workload_layer0(fsq):
    """The million-token G=84 workload, layer 0, full size. Its cache holds
    codes = FSQ(E x) of 128 prefill chunks of 8192 tokens (x ~ N(0,1) bf16 per
    chunk). The oracle encodes every chunk into a reference cache; the GPU
    appends the same chunks (codes compared under the tie rule, one chunk at a
    time) and decodes over the reference cache (compared with the oracle's
    decode of it)."""
    from concurrent.futures import ThreadPoolExecutor
    w = synth.WORKLOADS["qwen3_8b_g84_1m"]
    chunk = 8192
    n_chunks = w.context // chunk
    E, W = synth.layer_weights(w, 0)
    Ef = synth.bf16_bits_to_f64(E)
    E_dev = dev_bf16(E)
    ref_cache = np.empty((w.context, w.P), np.uint8)
    gpu_cache = torch.zeros((w.context, w.P), dtype=torch.uint8, device="cuda")
    flips, max_dist = 0, 0.0
    depth = 6
    with ThreadPoolExecutor(depth) as ex:
        futs = [ex.submit(synth.layer_x_chunk, w, 0, c, chunk) for c in range(min(depth, n_chunks))]
        for c in range(n_chunks):
            x = futs[c].result()
            if c + depth < n_chunks:
                futs.append(ex.submit(synth.layer_x_chunk, w, 0, c + depth, chunk))
            rows = slice(c * chunk, (c + 1) * chunk)
            fsq.fsq_append(dev_bf16(x), E_dev, gpu_cache[rows])
            u = orc.projection(synth.bf16_bits_to_f64(x), Ef)
            ref = orc.fsq_codes(u)
            ref_cache[rows] = orc.pack_codes(ref)
            got = orc.unpack_codes(gpu_cache[rows].cpu().numpy(), w.G)
            diff = got.astype(int) - ref.astype(int)
            bad = np.nonzero(diff)
            if len(bad[0]):
                assert np.all(np.abs(diff) <= 1), f"chunk {c}: a code differs by more than 1"
                ut = orc.fsq_bound(u[bad])
                dist = np.abs(ut - (np.floor(ut) + 0.5))
                tol = tie_tol(synth.bf16_bits_to_f64(x), Ef)[bad]
                assert np.all(dist < tol), f"chunk {c}: flip away from a tie ({dist.max()})"
                max_dist = max(max_dist, float(dist.max()))
            flips += len(bad[0])
    assert flips <= FLIP_RATE * w.context * w.G, f"{flips} flipped codes"
    # level statistics of FSQ(E x) (not uniform): every code value occurs
    assert len(np.unique(orc.unpack_codes(ref_cache[:chunk], w.G))) == 16
    q = synth.layer_query(w, 0)
    lens = synth.seq_lens(w)
    got = run_decode(fsq, q, ref_cache[None], W, lens, w.n_kv)
    want = oracle_decode(q, ref_cache[None], W, lens, w.n_kv, w.G)
    print(f"million-token layer 0: {flips} of {w.context * w.G} codes at fp32 ties "
          f"(largest tie distance {max_dist:.2e})")
    check_decode(got, want, lens, "million-token layer 0")
