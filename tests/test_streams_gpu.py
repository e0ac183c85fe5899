"""Calls on several HIP streams at once: the library keeps no state between
calls, so a multi-token decode and a gather running concurrently on separate
streams (each on its own bank and buffers) give the same bits as the same
calls run one after another."""

import pytest
import torch

import gen
from sparse_delta_rule_amd import sdm_decode_steps, sdm_gather, sdm_gather_compact

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _decode_job(wl, seed):
    bank = gen.decode_bank(wl, seed, DEV)
    seq = gen.decode_sequence(wl, seed, DEV)
    return bank, seq


def test_concurrent_streams_match_sequential_calls():
    wa = gen.WORKLOADS["c1"].replace(streams=256, steps=8)
    wb = gen.WORKLOADS["c4"].replace(streams=64, steps=4)
    wg = gen.WORKLOADS["c3"].replace(num_slots=100000, tokens=2048)
    bank_a, seq_a = _decode_job(wa, 51)
    bank_b, seq_b = _decode_job(wb, 52)
    gbank = gen.gather_bank(wg, 53, DEV)
    gi = gen.gather_inputs(wg, 53, DEV)
    kpos = gen.compact_positions(gi["idx0"], wg.chunk, gi["chunk_valid"])
    gkw = dict(chunk=wg.chunk, chunk_valid=gi["chunk_valid"], idx1=gi["idx1"], w1=gi["w1"])

    # one after another, on the current stream
    ra_bank, rb_bank = bank_a.clone(), bank_b.clone()
    ra = sdm_decode_steps(ra_bank, **seq_a)
    rb = sdm_decode_steps(rb_bank, **seq_b)
    g0, gs, g1 = sdm_gather(gbank, gi["idx0"], gi["w0"], **gkw)
    c0, cs, c1 = sdm_gather_compact(gbank, gi["idx0"], gi["w0"], kpos, **gkw)
    torch.cuda.synchronize()

    # the same calls issued on three streams at once, repeated to interleave them
    streams = [torch.cuda.Stream(DEV) for _ in range(3)]
    for rep in range(3):
        xa_bank, xb_bank = bank_a.clone(), bank_b.clone()
        outs = {}
        torch.cuda.synchronize()
        with torch.cuda.stream(streams[0]):
            outs["a"] = sdm_decode_steps(xa_bank, **seq_a)
        with torch.cuda.stream(streams[1]):
            outs["b"] = sdm_decode_steps(xb_bank, **seq_b)
        with torch.cuda.stream(streams[2]):
            outs["g"] = sdm_gather(gbank, gi["idx0"], gi["w0"], **gkw)
            outs["c"] = sdm_gather_compact(gbank, gi["idx0"], gi["w0"], kpos, **gkw)
        torch.cuda.synchronize()
        same = lambda x, y: torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))
        assert same(outs["a"], ra) and same(xa_bank, ra_bank), f"stream 0 decode, repeat {rep}"
        assert same(outs["b"], rb) and same(xb_bank, rb_bank), f"stream 1 decode, repeat {rep}"
        x0, xs, x1 = outs["g"]
        assert same(x0, g0) and same(xs, gs) and same(x1, g1), f"stream 2 gather, repeat {rep}"
        y0, ys, y1 = outs["c"]
        assert same(y0, c0) and same(ys, cs) and same(y1, c1), f"stream 2 compact gather, repeat {rep}"
