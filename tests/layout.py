"""Reader of the paged device layout documented in include/nvfp4kv.h.

Written independently of the kernels from the header's description, so the
tests can compare the library's bytes with the oracle's logical codes.
Works on numpy copies of the four planes.
"""
import numpy as np

D, PAGE, NBLK = 128, 16, 8


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[..., 64] bytes -> [..., 128] codes (element 2j = low nibble of byte j)."""
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


class Planes:
    def __init__(self, k_codes, k_scales, v_codes, v_scales, num_pages, hkv):
        self.kc = np.asarray(k_codes).reshape(num_pages, hkv, PAGE, 64)
        self.ks = np.asarray(k_scales).reshape(num_pages, hkv, PAGE, NBLK)
        # v codes: [page][head][group 4][byte 64][token 4]
        self.vc = np.asarray(v_codes).reshape(num_pages, hkv, 4, 64, 4)
        # v scales: [page][head][block 8][token 16]
        self.vs = np.asarray(v_scales).reshape(num_pages, hkv, NBLK, PAGE)

    def k_row(self, page, slot):
        """codes [Hkv][128], scales [Hkv][8] of the K row at (page, slot)."""
        return unpack_nibbles(self.kc[page, :, slot]), self.ks[page, :, slot]

    def v_row(self, page, slot):
        return unpack_nibbles(self.vc[page, :, slot // 4, :, slot % 4]), self.vs[page, :, :, slot]

    def gather(self, pages, slots):
        """Logical (kcodes, kscales, vcodes, vscales) for token lists, each
        [n][Hkv][...]."""
        pages = np.asarray(pages)
        slots = np.asarray(slots)
        kc = unpack_nibbles(self.kc[pages, :, slots])
        ks = self.ks[pages, :, slots]
        vb = self.vc[pages, :, slots // 4, :, slots % 4]       # [n][Hkv][64]
        vc = unpack_nibbles(vb)
        vs = self.vs[pages, :, :, slots]                        # [n][Hkv][8]
        return kc, ks, vc, vs

    def touched_mask(self, pages, slots):
        """Boolean masks over the four planes marking the bytes that the rows
        (page, slot) own; everything else must keep its fill value."""
        m = [np.zeros(self.kc.shape, bool), np.zeros(self.ks.shape, bool),
             np.zeros(self.vc.shape, bool), np.zeros(self.vs.shape, bool)]
        for p, s in zip(np.asarray(pages), np.asarray(slots)):
            m[0][p, :, s] = True
            m[1][p, :, s] = True
            m[2][p, :, s // 4, :, s % 4] = True
            m[3][p, :, :, s] = True
        return m

    def arrays(self):
        return self.kc, self.ks, self.vc, self.vs


def sequence_tokens(page_table_row, L):
    """(pages, slots) of positions 0..L-1 of one sequence."""
    pos = np.arange(L)
    return np.asarray(page_table_row)[pos // PAGE], pos % PAGE
