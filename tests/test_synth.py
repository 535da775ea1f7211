"""The seeded input generator: determinism, shapes, ranges and the Zipf popularity."""
import numpy as np

import oracle
import synth


def test_deterministic_and_seed_sensitive():
    cfg = synth.PRESETS["tiny"]
    a = synth.SynthLayer(cfg)
    b = synth.SynthLayer(cfg)
    assert a.fingerprint() == b.fingerprint()
    assert np.array_equal(a.x(), b.x())
    c = synth.SynthLayer(cfg, seed=cfg.seed + 1)
    assert a.fingerprint() != c.fingerprint()
    assert not np.array_equal(a.x(stream=0), a.x(stream=1))


def test_shapes_and_ranges():
    cfg = synth.PRESETS["b8mx"]
    fm = synth.expert_formats(cfg)
    assert (fm == synth.FMT_MXFP4).sum() == 52 and (fm == synth.FMT_VQ2).sum() == 204
    rank = synth.zipf_rank(cfg)
    assert np.all(fm[rank < 52] == synth.FMT_MXFP4)
    e_vq = int(np.nonzero(fm == synth.FMT_VQ2)[0][0])
    e_mx = int(np.nonzero(fm == synth.FMT_MXFP4)[0][0])
    v = synth.draw_expert(cfg, e_vq, synth.FMT_VQ2)
    assert v["codes_g"].shape == (2048, 1792) and v["codes_d"].shape == (7168, 512)
    assert v["scales_g"].shape == (2048, 56) and v["scales_d"].shape == (7168, 16)
    s = v["scales_g"].astype(np.float64)
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    m = synth.draw_expert(cfg, e_mx, synth.FMT_MXFP4)
    assert m["nib_g"].shape == (2048, 3584) and m["e8m0_d"].shape == (7168, 64)
    assert set(np.unique(m["e8m0_g"]).tolist()) == {118, 119, 120}


def test_codebook_nondegenerate():
    cb = synth.draw_codebook(1002)
    scb = oracle.signed_codebook(cb)
    assert len({tuple(r) for r in scb.tolist()}) == 256
    assert not np.any(np.all(scb == 0, axis=1))


def test_zipf_popularity():
    """Router logits drawn for a Zipf(1.1) popularity: the most popular ranks are
    selected most often, and the top-ranked expert appears in most tokens."""
    cfg = synth.PRESETS["b32"]
    rw = synth.draw_router(cfg)
    x = synth.draw_x(cfg, n=128, router_bits=rw)
    x64 = oracle.x_value(x, "bf16")
    assert abs(x64.std() - 1.0) < 0.3
    _, ids, _ = oracle.route(rw, x64, cfg.top_k)
    rank = synth.zipf_rank(cfg)
    counts = np.bincount(rank[ids.reshape(-1)], minlength=cfg.n_experts)
    assert counts[0] >= 0.7 * 128
    assert counts[:8].sum() > counts[8:64].sum() * 0.5
    assert counts[:16].mean() > counts[128:].mean() * 10
