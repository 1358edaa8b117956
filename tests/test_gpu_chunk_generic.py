"""GPU parity of the chunked prefill for every head size other than the bf16
128 x 128 head, and for the all-fp32 layer (gdn_chunk_generic.hip: fp32 MFMA),
against the fp64 oracle through the C ABI.  Sequences of two or more tokens take
the chunk kernel, one-token and empty ones the token kernel.

Bar as for every layer: per (sequence, value head) relative L2 error of the
outputs and final states within 1e-4 in fp32 and 1e-2 in bf16; the conv pool
bit-exact; blocks no sequence writes untouched.  Each case also checks that the
chunk kernel ran (the library's per-kernel timing names it)."""
import pytest

import linear_attention_state_amd as gdn
import workloads
from gpu_util import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

# lengths around the chunk size, one-token and empty sequences among them
LENGTHS = [2, 63, 64, 65, 1, 130, 0, 3, 200]

SHAPES = [
    ("f32-d16", workloads.Layer(2, 2, 16, 16, 4, "f32")),
    ("f32-d16-gqa2", workloads.Layer(2, 4, 16, 16, 4, "f32")),
    ("f32-dk32-dv64", workloads.Layer(2, 4, 32, 64, 3, "f32")),
    ("f32-d128", workloads.Layer(2, 4, 128, 128, 4, "f32")),
    ("f32-dk64-dv128-w1", workloads.Layer(1, 2, 64, 128, 1, "f32")),
    ("bf16-d64", workloads.Layer(4, 8, 64, 64, 4, "bf16")),
    ("bf16-dk128-dv32", workloads.Layer(2, 4, 128, 32, 2, "bf16")),
    ("bf16-d16", workloads.Layer(4, 4, 16, 16, 4, "bf16")),
]


def _run_timed(batch):
    gdn.gdn_kernel_timing(True)
    try:
        gpu = run_gpu(batch)
        kt = gdn.gdn_kernel_times()
    finally:
        gdn.gdn_kernel_timing(False)
    return gpu, kt


@pytest.mark.parametrize("idx", range(len(SHAPES)), ids=[s[0] for s in SHAPES])
def test_ragged_lengths(idx):
    name, layer = SHAPES[idx]
    b = workloads.random_batch(layer, LENGTHS, seed=300 + idx, fresh=[i % 3 == 0 for i in range(len(LENGTHS))])
    print("case %s: lengths %s" % (name, LENGTHS), flush=True)
    gpu, kt = _run_timed(b)
    assert kt.get("chunk_generic", (0.0, 0))[1] == 1, kt
    err = compare(b, gpu, run_oracle(b))
    print(name, err, flush=True)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_long_sequence_many_chunks(act):
    """1500 and 2100 tokens (24 and 33 chunks) continuing from their blocks, beside
    a decode token: the state carried across many chunks stays within the bar."""
    layer = workloads.Layer(2, 4, 64, 64, 4, act)
    b = workloads.random_batch(layer, [1500, 1, 2100], seed=320)
    print("case long-%s" % act, flush=True)
    gpu, kt = _run_timed(b)
    assert kt.get("chunk_generic", (0.0, 0))[1] == 1, kt
    print(act, compare(b, gpu, run_oracle(b)), flush=True)


def test_tiny_fp32_workload_takes_the_chunk_kernel():
    """The tiny all-fp32 workload (d = 16): its 5- and 17-token sequences run chunked."""
    b = workloads.config(0)
    gpu, kt = _run_timed(b)
    assert kt.get("chunk_generic", (0.0, 0))[1] == 1, kt
    compare(b, gpu, run_oracle(b))


def test_more_sequences_than_the_launch_order_holds():
    """1,030 chunked sequences beside short ones, more than the 1,024 the
    longest-first launch order holds: the fp32 chunk kernel then covers every
    sequence in index order."""
    layer = workloads.Layer(2, 4, 32, 64, 3, "f32")
    lengths = ([2, 3, 66, 5, 2, 9, 4, 2, 7, 3] * 103)[:1030] + [1, 0, 1, 1]
    b = workloads.random_batch(layer, lengths, seed=301)
    print("case many: %d sequences, T=%d" % (len(lengths), b.total_tokens), flush=True)
    gpu, kt = _run_timed(b)
    assert kt.get("chunk_generic", (0.0, 0))[1] == 1, kt
    compare(b, gpu, run_oracle(b))
