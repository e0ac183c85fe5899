"""The seeded input generator: determinism, private slot ranges, distinctness."""

import torch

import gen


def _small(name):
    wl = gen.WORKLOADS[name]
    return wl.replace(streams=min(wl.streams, 8), slots_per_stream=min(wl.slots_per_stream, 512))


def test_decode_inputs_are_seeded_and_private():
    for name in ("c0", "c1", "c2", "c4"):
        wl = _small(name)
        a = gen.decode_step_inputs(wl, 0, 3)
        b = gen.decode_step_inputs(wl, 0, 3)
        c = gen.decode_step_inputs(wl, 1, 3)
        for k in a:
            assert torch.equal(a[k], b[k])
        assert not torch.equal(a["k_val"], c["k_val"])
        P = wl.slots_per_stream
        for key, width in (("k_idx", wl.W), ("q_idx", wl.R)):
            idx = a[key].long()
            assert idx.dtype == torch.int64 and a[key].dtype == wl.idx_dtype
            assert idx.shape == (wl.streams, width)
            owner = torch.div(idx, P, rounding_mode="floor")
            assert torch.equal(owner, torch.arange(wl.streams)[:, None].expand_as(owner))
            for s in range(wl.streams):
                assert idx[s].unique().numel() == width
        assert a["g"].shape == (wl.streams, wl.G) and (a["g"] <= 0).all()
        assert (a["g"] >= wl.g_low).all()
        assert a["beta"].shape == (wl.streams, 1) and (a["beta"] >= 0).all() and (a["beta"] <= 1).all()


def test_bank_is_seeded():
    wl = _small("c0")
    b0 = gen.decode_bank(wl, 0)
    assert torch.equal(b0, gen.decode_bank(wl, 0))
    assert not torch.equal(b0, gen.decode_bank(wl, 1))
    assert 0.015 < b0.float().std().item() < 0.025


def test_gather_inputs():
    wl = gen.WORKLOADS["c3"].replace(num_slots=1000, tokens=256)
    a = gen.gather_inputs(wl, 0)
    assert a["idx0"].shape == (256, 64) and a["idx1"].shape == (256, 64)
    assert a["idx0"].dtype == torch.int32 and a["w0"].dtype == torch.bfloat16
    assert a["chunk_valid"].shape == (4,)
    assert (a["chunk_valid"] >= 32).all() and (a["chunk_valid"] <= 64).all()
    assert int(a["idx0"].min()) >= 0 and int(a["idx0"].max()) < 1000
    b = gen.gather_inputs(wl, 0)
    assert all(torch.equal(a[k], b[k]) for k in a)


def test_sub_seed_separates_keys():
    seen = {gen.sub_seed(0, "k_idx", t) for t in range(100)}
    seen |= {gen.sub_seed(0, "q_idx", t) for t in range(100)}
    assert len(seen) == 200


def test_compact_positions_are_first_positions_in_each_chunks_sorted_slots():
    """Within a chunk, live entries with one slot share a position, a smaller slot
    gets a smaller position, a slot's position counts the live entries of smaller
    slots in the chunk, and padding entries get -1."""
    import torch
    g = torch.Generator().manual_seed(5)
    T, chunk, W0 = 48, 16, 7
    idx0 = torch.randint(0, 40, (T, W0), generator=g)  # many repeats
    cv = torch.tensor([16, 9, 0], dtype=torch.int32)
    kp = gen.compact_positions(idx0, chunk, cv)
    assert kp.dtype == torch.int32 and kp.shape == (T, W0)
    for c in range(T // chunk):
        rows = range(c * chunk, (c + 1) * chunk)
        live = [t for t in rows if t - c * chunk < int(cv[c])]
        slots = [int(idx0[t, n]) for t in live for n in range(W0)]
        for t in rows:
            for n in range(W0):
                if t not in live:
                    assert kp[t, n] == -1
                else:
                    s = int(idx0[t, n])
                    assert kp[t, n] == sum(1 for x in slots if x < s), (t, n)
    # the worked example of the oracle's pins
    ex = gen.compact_positions(torch.tensor([[3, 1], [1, 0], [2, 2], [0, 3]]), 2, torch.tensor([2, 1], dtype=torch.int32))
    assert ex.tolist() == [[3, 1], [1, 0], [0, 0], [-1, -1]]
