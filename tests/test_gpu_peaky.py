"""Rows that a few keys dominate, with values that nearly cancel: the case
where rounding P to bf16 does not average out. For every (sequence, KV head)
three keys are planted along the q vector of the last window row of the
group's first head, with scaled scores 10, 9.9 and 9.6 (natural-log units
above keys whose scores are about N(0, 1)), so they carry almost all of that
row's weight, and their values are v, -1.1 v and 0.3 v. Every kernel is
compared with the oracle: the decode tile, the verify tile (32 and 64 rows),
the long-window kernel and the shared-prefix call (planted in the tails)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import AttnCase, make_tiny_case
from workloads.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from tests.gpu_util import say, attn_gpu, assert_close

SCORES = (10.0, 9.9, 9.6)
VALUES = (1.0, -1.1, 0.3)


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def plant(case, seed, first_token=0, vscale=1.0):
    """A copy of the case with the dominant keys planted at token positions
    >= first_token that every window row of the sequence sees; their values
    are VALUES times vscale times one random vector."""
    rng = np.random.default_rng(seed)
    k = case.k_pool.copy()
    v = case.v_pool.copy()
    Hq, Hkv = case.q.shape[1], case.k_pool.shape[1]
    group = Hq // Hkv
    q = bf16_bits_to_f32(case.q)
    r0 = 0
    for b in range(case.num_seqs):
        L, ql = int(case.seq_lens[b]), int(case.q_lens[b])
        if ql == 0:
            continue
        seen = L - ql + 1                        # tokens every window row sees
        span = seen - first_token
        assert span >= 3, "no room for the planted keys"
        toks = [first_token + (span * j) // 3 + int(rng.integers(0, max(1, span // 3))) for j in range(3)]
        toks = sorted(set(min(t, seen - 1) for t in toks))
        for g in range(Hkv):
            qv = q[r0 + ql - 1, g * group].astype(np.float64)
            v0 = rng.standard_normal(case.head_dim)
            for t, sc, vf in zip(toks, SCORES, VALUES):
                page, slot = int(case.block_table[b, t // 256]), t % 256
                # score * scale = sc (natural log units) for this row
                kv = qv * (sc / (case.scale * float(qv @ qv)))
                k[page, g, slot] = f32_to_bf16_bits(kv.astype(np.float32))
                v[page, g, slot] = f32_to_bf16_bits((vscale * vf * v0).astype(np.float32))
        r0 += ql
    return AttnCase(case.name + "-peaky", case.q, k, v, case.block_table, case.seq_lens, case.q_lens, case.scale)


def oracle_attn(case):
    return oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.q_lens,
                            case.scale)


SHAPES = [
    # seq_lens, q_lens, Hq, Hkv, D
    ([2000, 700, 300], [1, 1, 1], 8, 2, 128),       # decode, VALU tile
    ([2000, 700], [6, 3], 8, 2, 128),               # verify, MFMA 32-row tile
    ([1500, 900], [16, 2], 16, 4, 64),              # MFMA 64-row tile
    ([900, 400], [300, 100], 8, 2, 128),            # long window (prefill kernel)
]


# vscale 8: the planted values 8x larger than the other keys' (about N(0, 1)),
# so the rounding of the dominant keys' P weighs 8x more against the
# tolerance (single-term bf16 P would use about two thirds of it on the
# decode rows, by a float64 emulation of that rounding)
@pytest.mark.parametrize("vscale", [1.0, 8.0])
@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_dominant_keys_with_cancelling_values(pk, i, vscale):
    seq_lens, q_lens, Hq, Hkv, D = SHAPES[i]
    say(f"peaky rows {i}: seq_lens {seq_lens} q_lens {q_lens} Hq {Hq} Hkv {Hkv} D {D}, values x{vscale:g}")
    case = plant(make_tiny_case(600 + i, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D), 700 + i, vscale=vscale)
    got, flags = attn_gpu(case, pk)
    assert flags == 0
    assert_close(got, oracle_attn(case), f"peaky {i} x{vscale:g}")


def test_dominant_keys_in_the_tails_of_a_shared_prefix(pk):
    from tests.test_gpu_shared import shared_case, run_shared
    say("peaky rows: shared-prefix call, dominant keys in the private tails")
    base = shared_case(710, 2, [300, 700, 260], [1, 3, 2])
    case = plant(base, 711, first_token=2 * 256)
    got, again, flags = run_shared(pk, case, 2)
    assert flags == 0
    assert_close(got, oracle_attn(case), "peaky shared")
