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
    """nblk: scale blocks per row, 8 for NVFP4 (16 elements each), 4 for
    MXFP4 (32 each); the code planes are the same."""

    def __init__(self, k_codes, k_scales, v_codes, v_scales, num_pages, hkv, nblk=NBLK):
        self.kc = np.asarray(k_codes).reshape(num_pages, hkv, PAGE, 64)
        self.ks = np.asarray(k_scales).reshape(num_pages, hkv, PAGE, nblk)
        # v codes: [page][head][token quad 4][element group 16][token pair 2]
        # [element 8]; each byte holds the even token of its pair in the low
        # nibble and the odd token in the high nibble.  self.vc is the
        # logical code array [page][head][token 16][element 128].
        vb = np.asarray(v_codes).reshape(num_pages, hkv, 4, 16, 2, 8)
        nib = np.stack([vb & 0xF, vb >> 4], axis=-1)        # [..][quad][group][pair][e][nibble]
        nib = nib.transpose(0, 1, 2, 4, 6, 3, 5)             # [..][quad][pair][nibble][group][e]
        self.vc = np.ascontiguousarray(nib).reshape(num_pages, hkv, PAGE, D)
        # v scales: [page][head][block][token 16]
        self.vs = np.asarray(v_scales).reshape(num_pages, hkv, nblk, PAGE)

    def k_row(self, page, slot):
        """codes [Hkv][128], scales [Hkv][8] of the K row at (page, slot)."""
        return unpack_nibbles(self.kc[page, :, slot]), self.ks[page, :, slot]

    def v_row(self, page, slot):
        return self.vc[page, :, slot], self.vs[page, :, :, slot]

    def gather(self, pages, slots):
        """Logical (kcodes, kscales, vcodes, vscales) for token lists, each
        [n][Hkv][...]."""
        pages = np.asarray(pages)
        slots = np.asarray(slots)
        kc = unpack_nibbles(self.kc[pages, :, slots])
        ks = self.ks[pages, :, slots]
        vc = self.vc[pages, :, slots]                          # [n][Hkv][128]
        vs = self.vs[pages, :, :, slots]                        # [n][Hkv][8]
        return kc, ks, vc, vs

    def touched_mask(self, pages, slots):
        """Boolean masks over the four planes (V codes as the logical nibble
        array) marking what the rows (page, slot) own; everything else must
        keep its fill value (see untouched_fill)."""
        m = [np.zeros(self.kc.shape, bool), np.zeros(self.ks.shape, bool),
             np.zeros(self.vc.shape, bool), np.zeros(self.vs.shape, bool)]
        for p, s in zip(np.asarray(pages), np.asarray(slots)):
            m[0][p, :, s] = True
            m[1][p, :, s] = True
            m[2][p, :, s] = True
            m[3][p, :, :, s] = True
        return m

    def arrays(self):
        return self.kc, self.ks, self.vc, self.vs

    def untouched_fill(self, fill: int):
        """Per-plane arrays of what a byte fill value reads as: the byte for
        three planes, its low (even token) or high (odd token) nibble for the
        V codes."""
        tok = np.arange(PAGE)[None, None, :, None]
        vfill = np.where(tok % 2 == 0, fill & 0xF, fill >> 4) + np.zeros(self.vc.shape, np.uint8)
        return (np.full(self.kc.shape, fill, np.uint8), np.full(self.ks.shape, fill, np.uint8),
                vfill.astype(np.uint8), np.full(self.vs.shape, fill, np.uint8))


def sequence_tokens(page_table_row, L):
    """(pages, slots) of positions 0..L-1 of one sequence."""
    pos = np.arange(L)
    return np.asarray(page_table_row)[pos // PAGE], pos % PAGE


class CmpPlanes:
    """Reader of a comparison-format cache (FP8 or BF16), from the header's
    description: k slab [token 16][element 128]; v slab [token quad 4]
    [element 128][token 4].  Elements are uint8 codes (FP8) or uint16 bf16
    bit patterns (BF16).  self.k, self.v: [page][head][token 16][element 128]."""

    def __init__(self, k_bytes, v_bytes, num_pages, hkv, fmt):
        dt = np.uint8 if fmt == 1 else np.uint16
        k = np.asarray(k_bytes).view(dt).reshape(num_pages, hkv, PAGE, D)
        v = np.asarray(v_bytes).view(dt).reshape(num_pages, hkv, 4, D, 4)     # [..][quad][d][t%4]
        self.k = k
        self.v = np.ascontiguousarray(v.transpose(0, 1, 2, 4, 3)).reshape(num_pages, hkv, PAGE, D)

    def gather(self, pages, slots):
        """(k, v) of token lists, each [n][Hkv][128]."""
        pages = np.asarray(pages)
        slots = np.asarray(slots)
        return self.k[pages, :, slots], self.v[pages, :, slots]
