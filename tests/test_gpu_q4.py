"""Q4 cache on the GPU: the encoder bit for bit against oracle.q4_cache.encode
(packed nibbles and scales), and attention over Q4 pools against the
oracle's attention over the decoded pools (oracle.q4_cache.decode), at the
bf16 path's tolerance. The GPU inputs are the oracle's codes and scales; the
pools' unused slots hold NaN, which encodes to NaN scales the kernel must
never read."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from oracle import q4_cache
from workloads import make_config, make_tiny_case
from workloads.bf16 import f32_to_bf16_bits
from tests.gpu_util import say, dev_bf16, dev_i32, assert_close
from tests.test_gpu_parity import TINY
from tests.test_gpu_q8 import special_rows


@pytest.fixture(scope="module")
def pk():
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


@pytest.mark.parametrize("D", [64, 128])
def test_q4_encoder_matches_the_oracle_bit_for_bit(pk, D):
    rng = np.random.default_rng(9100 + D)
    n = 1037
    x = rng.standard_normal((n, D)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (n, 1))).astype(np.float32)
    tie = np.zeros(D, np.float32)
    tie[:6] = [7.0, 2.5, 3.5, -2.5, 0.5, -1.5]              # scale 1: ties to even
    x = np.concatenate([x, special_rows(D), tie[None, :]])
    bits = f32_to_bf16_bits(x)
    say(f"q4 encode: {bits.shape[0]} rows, D {D}")
    codes = torch.full((bits.shape[0], D // 2), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((bits.shape[0],), 7.0, dtype=torch.float32, device="cuda")
    pk.pkv_q4_encode(dev_bf16(bits), codes, scales)
    torch.cuda.synchronize()
    ec, es = q4_cache.encode(bits)
    np.testing.assert_array_equal(codes.cpu().numpy(), ec)
    got = scales.cpu().numpy()
    ok = ~np.isnan(es)
    assert np.array_equal(got.view(np.uint32)[ok], es.view(np.uint32)[ok])
    assert np.array_equal(np.isnan(got), np.isnan(es))


def test_q4_encoder_strides_past_its_grid(pk):
    # more rows than the capped grid covers in one pass (65536 workgroups of 4 rows)
    rng = np.random.default_rng(9200)
    n, D = 4 * 65536 + 77, 64
    bits = f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32))
    say(f"q4 encode: {n} rows, past the grid cap")
    codes = torch.full((n, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    pk.pkv_q4_encode(dev_bf16(bits), codes, scales)
    torch.cuda.synchronize()
    ec, es = q4_cache.encode(bits)
    np.testing.assert_array_equal(codes.cpu().numpy(), ec)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), es.view(np.uint32))


class Q4Case:
    """A case's pools encoded by the oracle, resident on the GPU."""

    def __init__(self, case, pk, plan=True):
        self.case, self.pk = case, pk
        kc, ks = q4_cache.encode(case.k_pool)
        vc, vs = q4_cache.encode(case.v_pool)
        self.ref_k, self.ref_v = q4_cache.decode(kc, ks), q4_cache.decode(vc, vs)
        self.q = dev_bf16(case.q)
        self.kc, self.ks = torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda()
        self.vc, self.vs = torch.from_numpy(vc).cuda(), torch.from_numpy(vs).cuda()
        self.bt, self.sl, self.ql = dev_i32(case.block_table), dev_i32(case.seq_lens), dev_i32(case.q_lens)
        self.shape = pk.attn_shape(self.q, self.kc, self.bt, max(1, case.max_q_len), case.scale)
        if plan:
            pk.pkv_attn_plan(self.shape, case.seq_lens)
        self.ws = pk.new_attn_workspace(self.shape)
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")

    def run(self):
        self.pk.pkv_attn_fwd_q4(self.q, self.kc, self.ks, self.vc, self.vs, self.bt, self.sl, self.ql, self.out,
                                self.shape, self.ws)
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.pk.pkv_attn_check_errors(self.ws)

    def expected(self):
        c = self.case
        return oracle.attention_decoded(c.q, self.ref_k, self.ref_v, c.block_table, c.seq_lens, c.q_lens, c.scale)


@pytest.mark.parametrize("i", range(len(TINY)))
def test_q4_attention_tiny_shapes(pk, i):
    seq_lens, q_lens, Hq, Hkv, D = TINY[i]
    say(f"q4 tiny case {i}: seq_lens={seq_lens} q_lens={q_lens} Hq={Hq} Hkv={Hkv} D={D}")
    qc = Q4Case(make_tiny_case(100 + i, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D), pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q4 tiny {i}")


@pytest.mark.parametrize("pps", [1, 2, 0])
def test_q4_attention_split_lengths(pk, pps):
    say(f"q4 splits: pages per split {pps}")
    qc = Q4Case(make_tiny_case(170, [2000, 700, 300, 9], [1, 3, 6, 2], Hq=8, Hkv=2, D=64), pk, plan=False)
    qc.shape.pages_per_split = pps
    qc.ws = pk.new_attn_workspace(qc.shape)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q4 pps {pps}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_q4_attention_configs(pk, cfg):
    say(f"q4 config {cfg}")
    case, _ = make_config(cfg)
    qc = Q4Case(case, pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q4 config {cfg}")


def test_q4_attention_is_deterministic_and_rejects_long_windows(pk):
    say("q4: two runs, long window refused, bad code extent refused")
    qc = Q4Case(make_tiny_case(180, [1500, 600], [4, 2], Hq=16, Hkv=4, D=128), pk)
    a, _ = qc.run()
    b, _ = qc.run()
    np.testing.assert_array_equal(a, b)
    long = Q4Case(make_tiny_case(181, [900], [300], Hq=8, Hkv=2, D=128), pk, plan=False)
    with pytest.raises(pk.PkvError):
        long.run()
    with pytest.raises(ValueError):   # Q8-sized code pools for a Q4 call
        pk.pkv_attn_fwd_q4(qc.q, torch.zeros(qc.kc.numel() * 2, dtype=torch.uint8, device="cuda"), qc.ks, qc.vc,
                           qc.vs, qc.bt, qc.sl, qc.ql, qc.out, qc.shape, qc.ws)


def test_q4_huge_values_take_the_exact_fallback(pk):
    """A V vector near the bf16 maximum (scale above 2^124, so -8 * scale
    overflows) makes its wave decode by subtract-then-multiply: the result
    still matches the oracle. Sequence 0 has 2 tokens, so its outputs (a
    weighted mean of the values) stay finite."""
    say("q4: a value vector near the bf16 maximum")
    case = make_tiny_case(190, [2, 300, 45], [1, 1, 1], Hq=8, Hkv=2, D=128)
    v = case.v_pool.copy()
    page = int(case.block_table[0, 0])
    rng = np.random.default_rng(191)
    for g in range(v.shape[1]):
        x = rng.uniform(-1, 1, 128) * 1.0e38
        x[7] = 1.6e38                                        # scale = 1.6e38 / 7 > 2^124
        v[page, g, 0] = f32_to_bf16_bits(x.astype(np.float32))
    from workloads import AttnCase
    big = AttnCase(case.name + "-huge", case.q, case.k_pool, v, case.block_table, case.seq_lens, case.q_lens,
                   case.scale)
    qc = Q4Case(big, pk)
    assert np.all(qc.vs.cpu().numpy()[page, :, 0] > 2.0 ** 124)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), "q4 huge values")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("qbits,max_window", [(8, 1), (4, 3)])
def test_quantized_large_ragged_batch(pk, qbits, max_window):
    """The bf16 suite's large ragged batch (2500 sequences of 1..512 tokens,
    about 20 000 workgroups) over a Q8 or Q4 cache, on the decode tile
    (windows of 1) and the MFMA tile (windows of 1..3)."""
    from tests.test_gpu_q8 import Q8Case
    rng = np.random.default_rng(40 + max_window)
    B = 2500
    seq_lens = rng.integers(1, 513, B)
    q_lens = np.minimum(rng.integers(1, max_window + 1, B), seq_lens)
    say(f"Q{qbits} large ragged batch: {B} sequences, windows up to {max_window}")
    case = make_tiny_case(460 + max_window, seq_lens.tolist(), q_lens.tolist(), Hq=4, Hkv=1, D=64)
    qc = (Q8Case if qbits == 8 else Q4Case)(case, pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"Q{qbits} large batch, windows up to {max_window}")
