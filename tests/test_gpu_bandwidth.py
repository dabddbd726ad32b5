"""GPU parity of the shard-sum (all-reduce stand-in) and the vocabulary-parallel
gather: bit-exact against the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, bf16_dev, bits_host, f32_dev, note
from workloads import CONFIGS, embed_inputs, shard_sum_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("n,numel", [(1, 1000), (2, 4096), (8, 1000003), (16, 77), (3, 1)])
def test_shard_sum_f32_bit_exact(n, numel):
    note(f"shard_sum f32 n={n} numel={numel}")
    parts = shard_sum_inputs(n, numel, 3000 + n, 1.0)
    out = torch.empty(numel, dtype=torch.float32, device=DEV)
    tp.shard_sum([f32_dev(p) for p in parts], out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.shard_sum_f32_ordered(parts))


@pytest.mark.parametrize("n,numel", [(2, 999), (8, 65536 + 5)])
def test_shard_sum_bf16_bit_exact(n, numel):
    note(f"shard_sum bf16 n={n} numel={numel}")
    parts = shard_sum_inputs(n, numel, 3100 + n, 1.0, dtype="bf16")
    out = torch.empty(numel, dtype=torch.bfloat16, device=DEV)
    tp.shard_sum([bf16_dev(p) for p in parts], out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_host(out), oracle.shard_sum_bf16_ordered(parts))


def test_shard_sum_in_place():
    note("shard_sum in place")
    parts = shard_sum_inputs(4, 5000, 3200, 1.0)
    dev = [f32_dev(p) for p in parts]
    tp.shard_sum(dev, dev[0])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev[0].cpu().numpy(), oracle.shard_sum_f32_ordered(parts))


def test_shard_sum_gpt3_full_size():
    c = CONFIGS["gpt3_mlp_rank_shard"]
    numel = c["b"] * c["s"] * c["h"]
    note(f"shard_sum GPT-3 shard: 8 x {numel} fp32")
    parts = shard_sum_inputs(c["n_partials"], numel, 2003, c["sigma_p"])
    out = torch.empty(numel, dtype=torch.float32, device=DEV)
    tp.shard_sum([f32_dev(p) for p in parts], out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.shard_sum_f32_ordered(parts))


def test_pages_worked_example_on_gpu():
    from tests.test_oracle_pins import _read_golden_split
    ids, vocab, ranks = _read_golden_split()
    h = 8
    rng = np.random.default_rng(61)
    from oracle.bf16 import f64_to_bf16_bits
    E = f64_to_bf16_bits(rng.standard_normal((vocab, h)))
    idt = torch.tensor(ids, dtype=torch.int32, device=DEV)
    note("vocab gather: worked example")
    for lo, hi, rows in ranks:
        out = torch.empty(len(ids), h, dtype=torch.bfloat16, device=DEV)
        tp.vocab_embed(idt, bf16_dev(E[lo:hi]), lo, hi, out)
        torch.cuda.synchronize()
        got = bits_host(out)
        for t, r in enumerate(rows):
            want = np.zeros(h, np.uint16) if r < 0 else E[lo:hi][r]
            np.testing.assert_array_equal(got[t], want)


def test_gather_out_of_range_and_ragged():
    note("vocab gather: out-of-range ids, h=40")
    rng = np.random.default_rng(62)
    v, h, lo, hi = 100, 40, 30, 70
    from oracle.bf16 import f64_to_bf16_bits
    E = f64_to_bf16_bits(rng.standard_normal((v, h)) * 0.02)
    ids = np.concatenate([rng.integers(-50, 150, 333), [lo, hi - 1, hi, lo - 1, -2**31, 2**31 - 1]]).astype(np.int32)
    out = torch.empty(ids.size, h, dtype=torch.bfloat16, device=DEV)
    tp.vocab_embed(torch.from_numpy(ids).to(DEV), bf16_dev(E[lo:hi]), lo, hi, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_host(out), oracle.vocab_embed_shard(ids, E[lo:hi], lo, hi))
    empty = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    tp.vocab_embed(torch.empty(0, dtype=torch.int32, device=DEV), bf16_dev(E[lo:hi]), lo, hi, empty)


def test_vocab_embed_full_size_all_shards():
    c = CONFIGS["vocab_parallel_embed"]
    v, h, N = c["v"], c["h"], c["N"]
    n = c["b"] * c["s"]
    note("vocab gather full size: generating table")
    ei = embed_inputs(v, h, n, c["seed"], c["sigma_w"])
    E, ids = ei["E"], ei["ids"]
    assert not np.any(E == 0x8000), "table holds -0.0"
    idt = torch.from_numpy(ids).to(DEV)
    Edev = bf16_dev(E)
    outs = []
    per = v // N
    for i in range(N):
        lo, hi = i * per, (i + 1) * per
        note(f"vocab gather full size shard {i}")
        out = torch.empty(n, h, dtype=torch.bfloat16, device=DEV)
        tp.vocab_embed(idt, Edev[lo:hi], lo, hi, out)
        want = bf16_dev(oracle.vocab_embed_shard(ids, E[lo:hi], lo, hi))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"shard {i}"
        outs.append(out)
    tot = torch.empty_like(outs[0])
    note("vocab gather full size: shard-sum of 8 shards")
    tp.shard_sum(outs, tot)
    torch.cuda.synchronize()
    assert torch.equal(tot.view(torch.int16), bf16_dev(E[ids]).view(torch.int16))
