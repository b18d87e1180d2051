"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
seeded inputs, element by element.

* The five named workloads at full size, in the launch configuration the
  benchmark times.  Small ones are compared on every head; large ones on a
  seeded sample of whole heads (the oracle computes each sampled head
  exactly, so every element of those heads is checked).
* Ragged sequence lengths (1, tails that leave partial tiles) and both head
  sizes of each precision.
"""

import pytest

from causal_self_attention_gptattn_amd import workloads as W

from gpu_helpers import compare, need_gpu, run_gpu, run_oracle, sample_heads, say

pytestmark = pytest.mark.gpu

# workload -> (seeds, heads compared per seed; None = all)
FULL = {
    "tiny_fp32": ((0, 1, 2), None),
    "char_gpt": ((0, 1, 2), 48),
    "gpt2_124m": ((0, 1, 2), 12),
    "gpt2_xl": ((0, 1, 2), 10),
    "gpt3_2048": ((0, 1, 2), 12),
}


@pytest.mark.parametrize("name", list(FULL))
def test_workload_parity(name):
    dev = need_gpu()
    seeds, count = FULL[name]
    w = W.WORKLOADS[name]
    for seed in seeds:
        say("parity", name, "seed", seed, (w.B, w.H, w.T, w.D, w.dtype))
        inp = W.workload_inputs(name, seed)
        got = run_gpu(inp, dev)
        heads = None if count is None else sample_heads(w.B, w.H, count, seed)
        ref = run_oracle(inp, heads)
        compare(got, ref, w.dtype, heads, label="%s/seed%d" % (name, seed),
                strict=(name == "tiny_fp32"))


RAGGED_BF16 = [(1, 2, T, D) for D in (64, 128) for T in (1, 2, 7, 31, 63, 64, 65, 127, 129, 200, 257)]
RAGGED_BF16 += [(2, 3, 384, 64), (1, 2, 300, 128)]


@pytest.mark.parametrize("B,H,T,D", RAGGED_BF16)
def test_ragged_bf16(B, H, T, D):
    dev = need_gpu()
    say("ragged bf16", B, H, T, D)
    inp = W.make_inputs(B, H, T, D, "bf16", seed=T + D)
    compare(run_gpu(inp, dev), run_oracle(inp), "bf16", label="bf16 T=%d D=%d" % (T, D))


RAGGED_F32 = [(1, 2, T, D) for D in (16, 32, 64) for T in (1, 3, 63, 64, 65, 130)]


@pytest.mark.parametrize("B,H,T,D", RAGGED_F32)
def test_ragged_f32(B, H, T, D):
    dev = need_gpu()
    say("ragged f32", B, H, T, D)
    inp = W.make_inputs(B, H, T, D, "f32", seed=T + D, recipe="iid")
    compare(run_gpu(inp, dev), run_oracle(inp), "f32", label="f32 T=%d D=%d" % (T, D))


# Long sequences: the backward kernels walk 128 tiles of 64 rows; whole heads
# of the sample are compared exactly (the oracle's T x T matrices are formed
# for the sampled heads only).
LONG = [(1, 4, 8192, 64, 2), (1, 2, 8192, 128, 1)]


@pytest.mark.parametrize("B,H,T,D,count", LONG)
def test_long_sequence_forward_and_backward(B, H, T, D, count):
    dev = need_gpu()
    say("long", B, H, T, D)
    inp = W.make_inputs(B, H, T, D, "bf16", seed=T + D)
    got = run_gpu(inp, dev)
    heads = sample_heads(B, H, count, seed=D)[:count]
    compare(got, run_oracle(inp, heads), "bf16", heads, label="long T=%d D=%d" % (T, D))


def test_peaked_scores_bf16():
    """Large-magnitude scores (std ~8) exercise the running-max rescaling."""
    dev = need_gpu()
    inp = W.make_inputs(1, 4, 320, 64, "bf16", seed=9)
    inp["scale"] = 1.25
    compare(run_gpu(inp, dev), run_oracle(inp), "bf16", label="peaked")
