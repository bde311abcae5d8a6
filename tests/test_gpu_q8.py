"""Q8 cache on the GPU: the encoder bit for bit against oracle.q8_cache.encode,
and attention over Q8 pools against the oracle's attention over the decoded
pools (oracle.q8_cache.decode), at the bf16 path's tolerance. The GPU inputs
are the oracle's codes and scales, so the two paths share nothing but the
seeded bf16 data. Pools come from make_tiny_case / make_config, whose slots
past every sequence end hold NaN: they encode to NaN scales, which the kernel
must never read."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle
from oracle import q8_cache
from workloads import make_config, make_tiny_case
from workloads.bf16 import f32_to_bf16_bits
from tests.gpu_util import say, dev_bf16, dev_i32, assert_close
from tests.test_gpu_parity import TINY


@pytest.fixture(scope="module")
def pk():
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def special_rows(D):
    """Rows that pin the encoder's edge cases: zeros, exact ties, a non-finite
    value, subnormal and near-maximal magnitudes."""
    rows = []
    rows.append(np.zeros(D, np.float32))
    tie = np.zeros(D, np.float32)                       # scale 1: codes round half to even
    tie[:6] = [127.0, 2.5, 3.5, -2.5, 100.5, -0.5]
    rows.append(tie)
    r = np.linspace(-1, 1, D).astype(np.float32)
    r[3] = np.inf
    rows.append(r)
    r = np.linspace(-1, 1, D).astype(np.float32)
    r[D - 1] = np.nan
    rows.append(r)
    rows.append((np.linspace(-1, 1, D) * 1e-38).astype(np.float32))     # subnormal scale
    rows.append((np.linspace(-1, 1, D) * 3.0e38).astype(np.float32))    # near the bf16 maximum
    one = np.zeros(D, np.float32)
    one[D // 2] = -7.0                                   # a single non-zero value
    rows.append(one)
    return np.stack(rows)


@pytest.mark.parametrize("D", [64, 128])
def test_encoder_matches_the_oracle_bit_for_bit(pk, D):
    rng = np.random.default_rng(9000 + D)
    n = 1037                                             # not a multiple of the 4 rows per workgroup
    x = rng.standard_normal((n, D)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (n, 1))).astype(np.float32)
    x = np.concatenate([x, special_rows(D)])
    bits = f32_to_bf16_bits(x)
    say(f"q8 encode: {bits.shape[0]} rows, D {D}")
    src = dev_bf16(bits)
    codes = torch.full((bits.shape[0], D), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((bits.shape[0],), 7.0, dtype=torch.float32, device="cuda")
    pk.pkv_q8_encode(src, codes, scales)
    torch.cuda.synchronize()
    ec, es = q8_cache.encode(bits)
    np.testing.assert_array_equal(codes.cpu().numpy(), ec)
    got = scales.cpu().numpy()
    assert np.array_equal(got.view(np.uint32)[~np.isnan(es)], es.view(np.uint32)[~np.isnan(es)])
    assert np.array_equal(np.isnan(got), np.isnan(es))


def test_encoder_strides_past_its_grid(pk):
    # more rows than the capped grid covers in one pass (65536 workgroups of 4 rows)
    rng = np.random.default_rng(9100)
    n, D = 4 * 65536 + 77, 64
    bits = f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32))
    say(f"q8 encode: {n} rows, past the grid cap")
    codes = torch.full((n, D), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    pk.pkv_q8_encode(dev_bf16(bits), codes, scales)
    torch.cuda.synchronize()
    ec, es = q8_cache.encode(bits)
    np.testing.assert_array_equal(codes.cpu().numpy(), ec)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), es.view(np.uint32))


def test_encoder_empty_and_bad_shapes(pk):
    src = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    pk.pkv_q8_encode(src, torch.zeros((0, 128), dtype=torch.int8, device="cuda"),
                     torch.zeros((0,), dtype=torch.float32, device="cuda"))
    src = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pk.PkvError):
        pk.pkv_q8_encode(src, torch.zeros((4, 96), dtype=torch.int8, device="cuda"),
                         torch.zeros((4,), dtype=torch.float32, device="cuda"))


class Q8Case:
    """A case's pools encoded by the oracle, resident on the GPU."""

    def __init__(self, case, pk, plan=True):
        self.case, self.pk = case, pk
        kc, ks = q8_cache.encode(case.k_pool)
        vc, vs = q8_cache.encode(case.v_pool)
        self.ref_k, self.ref_v = q8_cache.decode(kc, ks), q8_cache.decode(vc, vs)
        self.q = dev_bf16(case.q)
        self.kc = torch.from_numpy(kc).cuda()
        self.ks = torch.from_numpy(ks).cuda()
        self.vc = torch.from_numpy(vc).cuda()
        self.vs = torch.from_numpy(vs).cuda()
        self.bt = dev_i32(case.block_table)
        self.sl = dev_i32(case.seq_lens)
        self.ql = dev_i32(case.q_lens)
        self.shape = pk.attn_shape(self.q, self.kc, self.bt, max(1, case.max_q_len), case.scale)
        if plan:
            pk.pkv_attn_plan(self.shape, case.seq_lens)
        self.ws = pk.new_attn_workspace(self.shape)
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")

    def run(self):
        self.pk.pkv_attn_fwd_q8(self.q, self.kc, self.ks, self.vc, self.vs, self.bt, self.sl, self.ql, self.out,
                                self.shape, self.ws)
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.pk.pkv_attn_check_errors(self.ws)

    def expected(self):
        c = self.case
        return oracle.attention_decoded(c.q, self.ref_k, self.ref_v, c.block_table, c.seq_lens, c.q_lens, c.scale)


@pytest.mark.parametrize("i", range(len(TINY)))
def test_q8_attention_tiny_shapes(pk, i):
    seq_lens, q_lens, Hq, Hkv, D = TINY[i]
    say(f"q8 tiny case {i}: seq_lens={seq_lens} q_lens={q_lens} Hq={Hq} Hkv={Hkv} D={D}")
    qc = Q8Case(make_tiny_case(100 + i, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D), pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q8 tiny {i}")


@pytest.mark.parametrize("pps", [1, 2, 0])
def test_q8_attention_split_lengths(pk, pps):
    say(f"q8 splits: pages per split {pps}")
    case = make_tiny_case(140, [2000, 700, 300, 9], [1, 3, 6, 2], Hq=8, Hkv=2, D=128)
    qc = Q8Case(case, pk, plan=False)
    qc.shape.pages_per_split = pps
    qc.ws = pk.new_attn_workspace(qc.shape)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q8 pps {pps}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_q8_attention_configs(pk, cfg):
    say(f"q8 config {cfg}")
    case, _ = make_config(cfg)
    qc = Q8Case(case, pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q8 config {cfg}")


def test_q8_attention_is_deterministic_and_rejects_long_windows(pk):
    say("q8: two runs, long window refused")
    qc = Q8Case(make_tiny_case(150, [1500, 600], [4, 2], Hq=16, Hkv=4, D=64), pk)
    a, _ = qc.run()
    b, _ = qc.run()
    np.testing.assert_array_equal(a, b)
    long = Q8Case(make_tiny_case(151, [900], [300], Hq=8, Hkv=2, D=128), pk, plan=False)
    with pytest.raises(pk.PkvError):
        long.run()


def test_q8_encode_and_attention_replay_bit_exact(pk):
    """pkv_q8_encode of the pools and Q8 attention over a split shape,
    captured together in a HIP graph: every replay equals the eager result
    bit for bit (codes, scales and attention), with eager calls in between."""
    say("q8 graph: encode + attention (split merge), 4 replays")
    case = make_tiny_case(160, [4000, 2600, 900], [6, 4, 2], Hq=8, Hkv=2, D=128, num_pages=64)
    qc = Q8Case(case, pk)
    k, v = dev_bf16(case.k_pool), dev_bf16(case.v_pool)

    def step():
        pk.pkv_q8_encode(k, qc.kc, qc.ks)
        pk.pkv_q8_encode(v, qc.vc, qc.vs)
        pk.pkv_attn_fwd_q8(qc.q, qc.kc, qc.ks, qc.vc, qc.vs, qc.bt, qc.sl, qc.ql, qc.out, qc.shape, qc.ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_kc, ref_ks = qc.out.clone(), qc.kc.clone(), qc.ks.clone()
    assert_close(ref_out.cpu().numpy(), qc.expected(), "q8 graph eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        qc.out.fill_(float("nan"))
        qc.kc.fill_(99)
        qc.ks.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qc.out, ref_out), f"replay {rep}: attention differs"
        assert torch.equal(qc.kc, ref_kc), f"replay {rep}: codes differ"
        assert torch.equal(qc.ks.isnan(), ref_ks.isnan())
        assert torch.equal(torch.nan_to_num(qc.ks), torch.nan_to_num(ref_ks)), f"replay {rep}: scales differ"
        step()
        torch.cuda.synchronize()
        assert torch.equal(qc.out, ref_out), f"eager after replay {rep}: attention differs"
    assert pk.pkv_attn_check_errors(qc.ws) == 0


@pytest.mark.parametrize("i", range(4))
def test_q8_dominant_keys_with_cancelling_values(pk, i):
    """The peaky rows of the bf16 suite (three planted keys carrying almost all
    of a row's weight, values v, -1.1 v, 0.3 v) over a Q8 cache."""
    from tests.test_gpu_peaky import SHAPES, plant
    seq_lens, q_lens, Hq, Hkv, D = SHAPES[i]
    if max(q_lens) * (Hq // Hkv) > pk.PKV_MAX_ROWS:
        pytest.skip("long windows are not served over a Q8 cache")
    say(f"q8 peaky rows {i}: seq_lens {seq_lens} q_lens {q_lens} Hq {Hq} Hkv {Hkv} D {D}")
    case = plant(make_tiny_case(600 + i, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D), 700 + i)
    qc = Q8Case(case, pk)
    got, flags = qc.run()
    assert flags == 0
    assert_close(got, qc.expected(), f"q8 peaky {i}")
