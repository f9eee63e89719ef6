"""The oracle's row-range / unit-subset / chunked evaluation (used to check
sampled outputs at full sizes) gives bitwise the rows of the full evaluation."""
import numpy as np

import oracle
from transformer_attention_variant_amd import inputs as I


def test_rows_units_chunks_bitwise():
    for kq in (I.PRE, I.POST, I.PRE_EXACT):
        cfg = I.small(B=2, H=4, T=45, d=8, c_q=4, c_k=7, c_h=2, kq_place=kq, seed=41)
        inp = I.generate(cfg)
        full = oracle.forward_cfg(cfg, inp, threads=1, chunk=0)
        chunked = oracle.forward_cfg(cfg, inp, threads=3, chunk=7)
        assert np.array_equal(full, chunked)
        part = oracle.forward_cfg(cfg, inp, threads=2, rows=(20, 33), units=[3, 0], chunk=5)
        for u in (3, 0):
            b, g = divmod(u, cfg.groups)
            hs = slice(g * cfg.c_h, (g + 1) * cfg.c_h)
            assert np.array_equal(part[b, hs, 20:33], full[b, hs, 20:33])
        # everything outside the requested rows and units stays NaN
        assert np.isnan(part[1, 0:2]).all() and np.isnan(part[0, 0:2, :20]).all()


def test_layer_rows_units_chunks_bitwise():
    """Same for the general layer: the repeated form reads c_q2-1 probability
    rows and c_q-1 + c_q2-1 logit rows above each chunk."""
    for form, kq in (("repeat", I.PRE), ("repeat", I.PRE_EXACT), ("3d", I.PRE)):
        cfg = I.small(B=2, H=4, T=41, d=8, c_q=4, c_k=5, c_h=2, kq_place=kq, form=form, c_q2=3, c_k2=4,
                      head_place=I.PRE if form == "3d" else I.POST, seed=43)
        inp = I.generate(cfg)
        full = oracle.forward_cfg(cfg, inp, threads=1, chunk=0)
        chunked = oracle.forward_cfg(cfg, inp, threads=3, chunk=6)
        assert np.array_equal(full, chunked)
        part = oracle.forward_cfg(cfg, inp, threads=2, rows=(17, 30), units=[2], chunk=4)
        b, g = divmod(2, cfg.groups)
        hs = slice(g * cfg.c_h, (g + 1) * cfg.c_h)
        assert np.array_equal(part[b, hs, 17:30], full[b, hs, 17:30])
