"""GPU parity of the gate prologue (L2-normalised q and k, beta from logits,
fused into the kernels' loads) against the oracle's prologue, through the C
ABI.  Inputs are raw: q and k rows of norm 1..8, beta as logits."""
import numpy as np
import pytest

from linear_attention_sequence_03_amd import gdr, synth
from gpu_helpers import dev, host, io_dtype, rel_err, torch_mod
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _call(inp, io, chunk, flags):
    from linear_attention_sequence_03_amd import gdr_chunk_fwd
    torch = torch_mod()
    dt = io_dtype(io)
    o, st = gdr_chunk_fwd(dev(inp["q"], dt), dev(inp["k"], dt), dev(inp["v"], dt),
                          dev(inp["log_alpha"]), dev(inp["beta"]),
                          None if inp["S0"] is None else dev(inp["S0"]), chunk=chunk, prologue=flags)
    torch.cuda.synchronize()
    return o, st


def _ref(inp, flags):
    return oracle.chunk_fwd_prologue(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                     inp["S0"], flags=flags)


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("gate,chunk,d,H", [("scalar", 64, 128, 3), ("scalar", 64, 64, 3),
                                            ("scalar", 64, 128, 40),     # two compute waves
                                            ("channel", 64, 128, 3), ("channel", 32, 64, 3),
                                            ("channel", 16, 128, 2)])
def test_prologue_chunk(gate, chunk, d, H, flags):
    base = synth.chunk_inputs(2, 170, H, d, d, gate, "bf16", seed=300 + d + chunk + H, s0_std=0.1)
    inp = synth.raw_prologue_inputs(base, "bf16", seed=300 + flags)
    if not flags & 1:            # without the normalisation the keys must already be unit rows
        inp["q"], inp["k"] = base["q"], base["k"]
    if not flags & 2:
        inp["beta"] = base["beta"]
    o, st = _call(inp, "bf16", chunk, flags)
    o_ref, st_ref = _ref(inp, flags)
    eo, es = rel_err(host(o), o_ref), rel_err(host(st), st_ref)
    print("gate=%s chunk=%d d=%d H=%d flags=%d err_o=%.3g err_S=%.3g" % (gate, chunk, d, H, flags, eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


def test_prologue_zero_flags_is_the_plain_call():
    inp = synth.chunk_inputs(1, 100, 2, 128, 128, "scalar", "bf16", seed=310, s0_std=0.1)
    o1, s1 = _call(inp, "bf16", 64, 0)
    from linear_attention_sequence_03_amd import gdr_chunk_fwd
    torch = torch_mod()
    dt = io_dtype("bf16")
    o2, s2 = gdr_chunk_fwd(dev(inp["q"], dt), dev(inp["k"], dt), dev(inp["v"], dt),
                           dev(inp["log_alpha"]), dev(inp["beta"]), dev(inp["S0"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(o1), host(o2)) and np.array_equal(host(s1), host(s2))


@pytest.mark.parametrize("io,gate,chunk", [("f32", "scalar", 64), ("bf16", "scalar", 32)])
def test_prologue_unfused_paths_are_refused(io, gate, chunk):
    inp = synth.chunk_inputs(1, 40, 2, 64, 64, gate, io, seed=311)
    with pytest.raises(gdr.GdrError) as e:
        _call(inp, io, chunk, 1)
    assert e.value.status == gdr.GDR_ERR_UNSUPPORTED


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("io,d", [("f32", 128), ("f32", 64), ("bf16", 128)])
def test_prologue_decode(io, d, gate):
    from linear_attention_sequence_03_amd import gdr_decode_step
    torch = torch_mod()
    base = synth.decode_inputs(8, 4, d, d, gate, io, seed=320 + d)
    inp = synth.raw_prologue_inputs(base, io, seed=320)
    dt = io_dtype(io)
    o, S1 = gdr_decode_step(dev(inp["q"], dt), dev(inp["k"], dt), dev(inp["v"], dt),
                            dev(inp["log_alpha"]), dev(inp["beta"]), dev(inp["S"]), prologue=3)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode_step_prologue(inp["q"], inp["k"], inp["v"], inp["log_alpha"],
                                               inp["beta"], inp["S"], flags=3)
    assert rel_err(host(o), o_ref) <= (4e-3 if io == "bf16" else 1e-5)
    assert rel_err(host(S1), S_ref) <= 1e-5


def test_prologue_full_size_headline_shape():
    """The Gated DeltaNet prefill workload's shape (B=4, H=16, T=4096, d=128,
    bf16) from raw inputs; sampled (b,h) pairs against the oracle."""
    w = synth.WORKLOADS[1]
    inp = synth.raw_prologue_inputs(synth.workload_inputs(w), "bf16", seed=w.seed)
    o, st = _call(inp, "bf16", 64, 3)
    o, st = host(o), host(st)
    for b, h in [(0, 0), (3, 15), (2, 9)]:
        sl = lambda a: None if a is None else a[b:b + 1, :, h:h + 1]  # noqa: E731
        o_ref, st_ref = oracle.chunk_fwd_prologue(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                                  sl(inp["log_alpha"]), sl(inp["beta"]), None, flags=3)
        assert rel_err(o[b, :, h], o_ref[0, :, 0]) <= TOL["bf16"]
        assert rel_err(st[b, h], st_ref[0, 0]) <= TOL["bf16"]
