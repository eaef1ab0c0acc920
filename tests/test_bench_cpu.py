"""The measurement's host-side contract (no GPU): the one-GPU guard, and the
algorithmic bytes and FLOPs behind roofline.achieved, each derived here by hand
from what a call must move at least once.

Bytes of a prefill call: q, k, v read and o written once in the io type;
log alpha (fp32, one per head-token, or d_k of them with the channel gate) and
beta (fp32) read once; the final state written and the start state read once
(fp32, d_v x d_k per head).  Decode: the fp32 state read and written once, q,
k, v read and o written in fp32, log alpha and beta read.  FLOPs of a prefill
call: 6 d^2 + 3 C d + C^2 per head-token (the "FG2-GDN" page's per-head kernel
accounting, section 3.6)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_long_context_prefill_bytes_and_flops():
    # B=1, T=32768, H=32, d=128, bf16 io, scalar gate, with a start state, chunk 64
    tokens_heads = 32768 * 32
    per_head_token = 4 * 128 * 2 + 4 + 4            # q, k, v, o (bf16) + log alpha + beta
    state = 32 * 128 * 128 * 4
    nbytes, flops = bench.prefill_algorithmic(1, 32768, 32, 128, 64, s0=True)
    assert nbytes == tokens_heads * per_head_token + 2 * state == 1_086_324_736
    assert flops == tokens_heads * (6 * 128 ** 2 + 3 * 64 * 128 + 64 ** 2) == 133_143_986_176


def test_channel_gate_prefill_bytes():
    # B=2, T=8192, H=32, d=128, bf16 io, per-channel log alpha, no start state
    tokens_heads = 2 * 8192 * 32
    per_head_token = 4 * 128 * 2 + 128 * 4 + 4
    nbytes, _ = bench.prefill_algorithmic(2, 8192, 32, 128, 64, channel=True)
    assert nbytes == tokens_heads * per_head_token + 2 * 32 * 128 * 128 * 4 == 811_597_824


def test_two_rate_prefill_bytes():
    # FG2-GDN+ / Gated DeltaNet-2: two fp32 d-vectors per head-token replace beta
    tokens_heads = 2 * 8192 * 32
    per_head_token = 4 * 128 * 2 + 128 * 4 + 2 * 128 * 4
    nbytes, _ = bench.prefill_algorithmic(2, 8192, 32, 128, 64, channel=True, fg2=True)
    assert nbytes == tokens_heads * per_head_token + 2 * 32 * 128 * 128 * 4


def test_decode_bytes():
    # B=256, H=32, d=128, fp32 state and io
    heads = 256 * 32
    per_head = 2 * 128 * 128 * 4 + 4 * 128 * 4 + 2 * 4
    assert bench.decode_algorithmic(256, 32, 128) == heads * per_head == 1_090_584_576
