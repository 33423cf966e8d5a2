"""The V4.1 CSA2 layer schedule as the workloads define it, against the counts
the page states ("DeepSeek-V4.1 架构解析" §02: 18 CSA2 encoder layers in three groups of six, each
led by its only Full layer; 20 decoder layers: one Full and three Reuse, then
four groups of one Reindex and three Reuse; the decoder's first Full layer
builds the 2,048-block pool its Reindex layers search).  CPU only."""

import workloads as W


def test_v41_schedule_counts():
    cfgs = W.v41_schedule("decode", n_seq=1, ctx_tokens=4096)
    layers = [m for c in cfgs for m in c.layers]
    assert len(layers) == 38
    enc, dec = cfgs[:3], cfgs[3]
    assert all(c.layers == ["F", "U", "U", "U", "U", "U"] and not c.build_pool for c in enc)
    assert sum(len(c.layers) for c in enc) == 18
    assert len(dec.layers) == 20 and dec.build_pool
    assert dec.layers[:4] == ["F", "U", "U", "U"]
    assert all(dec.layers[4 + 4 * g: 8 + 4 * g] == ["I", "U", "U", "U"] for g in range(4))
    assert layers.count("F") == 4 and layers.count("I") == 4 and layers.count("U") == 30


def test_v41_schedule_inputs_are_per_group_and_per_layer():
    cfgs = W.v41_schedule("decode", n_seq=1, ctx_tokens=4 * 40, cid=250)
    wls = [W.make_workload(c) for c in cfgs]
    # own global KV per group (indexer keys drawn from the group's own seed)
    assert not (wls[0].tensors["k_fp8"] == wls[1].tensors["k_fp8"]).all()
    for wl in wls:
        xw = wl.tensors["x_win"]
        assert tuple(xw.shape) == (len(wl.cfg.layers), 1, 128, 512)
        assert not (xw[0] == xw[1]).all()
