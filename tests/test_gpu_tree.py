"""GPU parity of the draft-tree calls (gdr_decode_tree, gdr_decode_tree_commit)
against the oracle's node-by-node tree decode, through the C ABI: every tree
shape (chain, star, binary, random), tree sizes 1..64, both gates, both io
types, head sizes 64 and 128; the written values D; the commit of every kind
of node, in place and out of place; a chain against gdr_decode_multi; parents
outside [-1, i) read as -1; the decode workload's full size on sampled
sequences.  Metric: normwise max|gpu - oracle| / max|oracle| per tensor."""
import numpy as np
import pytest

from linear_attention_sequence_03_amd import synth
from gpu_helpers import dev, host, io_dtype, rel_err, torch_mod
import oracle

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-4, "bf16": 4e-3}   # bf16: the outputs' own rounding
TOL_FP32 = 1e-4                       # D and states: fp32 arithmetic for both io types


def _inputs(B, Td, H, d, gate, io, seed):
    inp = synth.chunk_inputs(B, Td, H, d, d, gate, io, seed=seed, s0_std=0.05)
    return inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"]


def _gpu_tree(q, k, v, la, be, S, par, io):
    torch = torch_mod()
    from linear_attention_sequence_03_amd import gdr_decode_tree
    dt = io_dtype(io)
    o, D = gdr_decode_tree(dev(q, dt), dev(k, dt), dev(v, dt), dev(la), dev(be), dev(S),
                           dev(par, torch.int32))
    torch.cuda.synchronize()
    return o, D


def _commit(k, la, par, D, acc, S, io, inplace=False):
    torch = torch_mod()
    from linear_attention_sequence_03_amd import gdr_decode_tree_commit
    Sd = dev(S)
    out = gdr_decode_tree_commit(dev(k, io_dtype(io)), dev(la), dev(par, torch.int32), D,
                                 dev(np.asarray(acc, np.int32), torch.int32), Sd, inplace=inplace)
    torch.cuda.synchronize()
    assert (out.data_ptr() == Sd.data_ptr()) == inplace
    return out


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("d", [64, 128])
# 17 and 40 nodes: two and three node tiles of 16 with a ragged last tile (the
# verify kernel is specialised on the tile count; 64 nodes is four)
@pytest.mark.parametrize("kind,Td", [("chain", 7), ("star", 5), ("binary", 16), ("random", 16),
                                     ("random", 17), ("binary", 40), ("random", 64), ("chain", 64),
                                     ("random", 1)])
def test_tree_verify_and_commit(kind, Td, d, gate, io):
    B, H = 2, 3
    q, k, v, la, be, S = _inputs(B, Td, H, d, gate, io, seed=40 + Td + d)
    par = synth.draft_tree(kind, B, Td, seed=Td)
    o, D = _gpu_tree(q, k, v, la, be, S, par, io)
    o_ref, u_ref, states = oracle.decode_tree(q, k, v, la, be, S, par)
    eo, ed = rel_err(host(o), o_ref), rel_err(host(D), u_ref)
    print("tree %s Td=%d d=%d %s %s: err_o=%.3g err_D=%.3g" % (kind, Td, d, gate, io, eo, ed))
    assert eo <= TOL_O[io] and ed <= TOL_FP32, (eo, ed)
    # commit: the last node, a middle one, and nothing
    for acc in ([Td - 1, Td // 2], [-1, 0]):
        s_ref = oracle.decode_tree_commit(S, states, acc)
        for inplace in (False, True):
            s = _commit(k, la, par, D, acc, S, io, inplace=inplace)
            es = rel_err(host(s), s_ref)
            assert es <= TOL_FP32, (acc, inplace, es)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_chain_matches_decode_multi(gate):
    torch = torch_mod()
    from linear_attention_sequence_03_amd import gdr_decode_multi
    B, Td, H, d = 3, 12, 4, 128
    q, k, v, la, be, S = _inputs(B, Td, H, d, gate, "f32", seed=60)
    par = synth.draft_tree("chain", B, Td)
    o, D = _gpu_tree(q, k, v, la, be, S, par, "f32")
    Sd = dev(S)
    o_m, s_m = gdr_decode_multi(dev(q), dev(k), dev(v), dev(la), dev(be), Sd, S_out=torch.empty_like(Sd),
                                accepted=dev(np.array([Td, 5, 1], np.int32), torch.int32))
    torch.cuda.synchronize()
    assert rel_err(host(o), host(o_m)) <= 1e-5
    s_t = _commit(k, la, par, D, [Td - 1, 4, 0], S, "f32")
    assert rel_err(host(s_t), host(s_m)) <= 1e-5


def test_parents_out_of_range_read_as_root_children():
    B, Td, H, d = 2, 9, 2, 64
    q, k, v, la, be, S = _inputs(B, Td, H, d, "scalar", "f32", seed=61)
    bad = np.array([[5, 0, 7, 1, -3, 2, 100, 5, 8], [-1, 0, 1, 1, 9, 4, -2, 0, 2]], dtype=np.int32)
    fixed = np.array([[p if -1 <= p < i else -1 for i, p in enumerate(row)] for row in bad], dtype=np.int32)
    o, D = _gpu_tree(q, k, v, la, be, S, bad, "f32")
    o_ref, u_ref, states = oracle.decode_tree(q, k, v, la, be, S, fixed)
    assert rel_err(host(o), o_ref) <= 1e-4 and rel_err(host(D), u_ref) <= 1e-4
    acc = [8, 99]   # 99 is outside [0, Td): keeps S
    s = _commit(k, la, bad, D, acc, S, "f32")
    assert rel_err(host(s), oracle.decode_tree_commit(S, states, [8, -1])) <= 1e-4


def test_outputs_optional():
    torch = torch_mod()
    from linear_attention_sequence_03_amd import gdr_decode_tree
    B, Td, H, d = 1, 6, 2, 64
    q, k, v, la, be, S = _inputs(B, Td, H, d, "channel", "bf16", seed=62)
    par = synth.draft_tree("binary", B, Td)
    bf = io_dtype("bf16")
    args = (dev(q, bf), dev(k, bf), dev(v, bf), dev(la), dev(be), dev(S), dev(par, torch.int32))
    o_only, none_d = gdr_decode_tree(*args, want_D=False)
    none_o, d_only = gdr_decode_tree(*args, want_o=False)
    torch.cuda.synchronize()
    assert none_d is None and none_o is None
    o_ref, u_ref, _ = oracle.decode_tree(q, k, v, la, be, S, par)
    assert rel_err(host(o_only), o_ref) <= TOL_O["bf16"] and rel_err(host(d_only), u_ref) <= TOL_FP32


def test_decode_workload_size_sampled():
    """The decode workload's shape (B=256, H=32, d=128, fp32 state of 512 MiB)
    with a random 16-node tree per sequence; sequences 0, 77 and 255 against
    the oracle, and the accepted state of each."""
    torch = torch_mod()
    w = synth.WORKLOADS[4]
    B, H, d, Td = w.B, w.H, w.d, 16
    q, k, v, la, be, S = _inputs(B, Td, H, d, "scalar", "f32", seed=63)
    par = synth.draft_tree("random", B, Td, seed=63)
    o, D = _gpu_tree(q, k, v, la, be, S, par, "f32")
    acc = np.random.Generator(np.random.PCG64(64)).integers(-1, Td, B).astype(np.int32)
    s = _commit(k, la, par, D, acc, S, "f32")
    o, D, s = host(o), host(D), host(s)
    for b in (0, 77, 255):
        sl = lambda a: a[b:b + 1]  # noqa: E731
        o_ref, u_ref, states = oracle.decode_tree(sl(q), sl(k), sl(v), sl(la), sl(be), sl(S), sl(par))
        assert rel_err(o[b], o_ref[0]) <= 1e-4 and rel_err(D[b], u_ref[0]) <= 1e-4
        s_ref = oracle.decode_tree_commit(sl(S), states, [acc[b]])
        assert rel_err(s[b], s_ref[0]) <= 1e-4
