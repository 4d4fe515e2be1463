"""The test-side reader of the cache layout against the byte formulas that
include/nvfp4kv.h states, written out element by element."""
import numpy as np

from layout import Planes


def test_reader_matches_header_formulas():
    rng = np.random.default_rng(0)
    P_, H = 2, 3
    kc = rng.integers(0, 16, (P_, H, 16, 128), dtype=np.uint8)
    ks = rng.integers(0, 256, (P_, H, 16, 8), dtype=np.uint8)
    vc = rng.integers(0, 16, (P_, H, 16, 128), dtype=np.uint8)
    vs = rng.integers(0, 256, (P_, H, 16, 8), dtype=np.uint8)
    kb = np.zeros((P_, H, 1024), np.uint8)
    ksb = np.zeros((P_, H, 128), np.uint8)
    vb = np.zeros((P_, H, 1024), np.uint8)
    vsb = np.zeros((P_, H, 128), np.uint8)
    for p in range(P_):
        for h in range(H):
            for t in range(16):
                for j in range(64):       # K: byte j of token row t = elements 2j, 2j+1
                    kb[p, h, t * 64 + j] = kc[p, h, t, 2 * j] | (kc[p, h, t, 2 * j + 1] << 4)
                for blk in range(8):
                    ksb[p, h, t * 8 + blk] = ks[p, h, t, blk]
                    vsb[p, h, blk * 16 + t] = vs[p, h, t, blk]
                for d in range(128):      # V: element d of the pair (t & ~1, t | 1)
                    off = (t // 4) * 256 + (d // 8) * 16 + ((t // 2) % 2) * 8 + d % 8
                    vb[p, h, off] |= vc[p, h, t, d] << (4 * (t % 2))
    R = Planes(kb.ravel(), ksb.ravel(), vb.ravel(), vsb.ravel(), P_, H)
    pages = np.repeat(np.arange(P_), 16)
    slots = np.tile(np.arange(16), P_)
    gk, gks, gv, gvs = R.gather(pages, slots)
    assert np.array_equal(gk, kc.transpose(0, 2, 1, 3).reshape(-1, H, 128))
    assert np.array_equal(gks, ks.transpose(0, 2, 1, 3).reshape(-1, H, 8))
    assert np.array_equal(gv, vc.transpose(0, 2, 1, 3).reshape(-1, H, 128))
    assert np.array_equal(gvs, vs.transpose(0, 2, 1, 3).reshape(-1, H, 8))
    # fill: a byte 0xA5 reads 5 for even tokens, 0xA for odd tokens in V
    R2 = Planes(np.full(P_ * H * 1024, 0xA5, np.uint8), np.zeros(P_ * H * 128, np.uint8),
                np.full(P_ * H * 1024, 0xA5, np.uint8), np.zeros(P_ * H * 128, np.uint8), P_, H)
    f = R2.untouched_fill(0xA5)
    assert np.array_equal(R2.vc, f[2])
    assert np.all(R2.vc[:, :, 0::2] == 5) and np.all(R2.vc[:, :, 1::2] == 0xA)


def test_cmp_reader_matches_header_formulas():
    from layout import CmpPlanes
    rng = np.random.default_rng(1)
    P_, H = 2, 3
    for fmt, dt in ((1, np.uint8), (2, np.uint16)):
        k = rng.integers(0, np.iinfo(dt).max, (P_, H, 16, 128), dtype=dt)
        v = rng.integers(0, np.iinfo(dt).max, (P_, H, 16, 128), dtype=dt)
        kb = np.zeros((P_, H, 16 * 128), dt)
        vb = np.zeros((P_, H, 16 * 128), dt)
        for p in range(P_):
            for h in range(H):
                for t in range(16):
                    for d in range(128):
                        kb[p, h, t * 128 + d] = k[p, h, t, d]                      # [token][element]
                        vb[p, h, ((t // 4) * 128 + d) * 4 + t % 4] = v[p, h, t, d]  # [quad][element][t%4]
        R = CmpPlanes(kb.ravel().view(np.uint8), vb.ravel().view(np.uint8), P_, H, fmt)
        assert np.array_equal(R.k, k) and np.array_equal(R.v, v)
        gk, gv = R.gather([1, 0], [5, 14])
        assert np.array_equal(gk, k[[1, 0], :, [5, 14]]) and np.array_equal(gv, v[[1, 0], :, [5, 14]])
