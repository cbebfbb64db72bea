"""The KV pool's block layout, built by enumerating the attention kernel's
operand loads (as the boundary documents them): lane l of a 16-byte load
of 32-dim chunk c carries 8 elements.  Used by tests to address pool slots;
written from the lane layout of the instructions, independently of the
library's closed-form offsets; a GPU test checks pool import against it."""
import numpy as np


def maps(head_dim: int, page_size: int = 16):
    """(kmap, vmap): [page_size, head_dim] arrays of element positions."""
    assert page_size == 16 and head_dim % 32 == 0
    kmap = np.full((16, head_dim), -1, np.int64)
    vmap = np.full((16, head_dim), -1, np.int64)
    for c in range(head_dim // 32):
        for lane in range(64):
            for e in range(8):
                pos = c * 512 + lane * 8 + e
                # K operand: lane holds key lane % 16, dims 32c + 8 (lane // 16) + e
                kmap[lane % 16, 32 * c + 8 * (lane // 16) + e] = pos
                # V operands: first 4 elements dim block 2c, last 4 block 2c + 1;
                # keys 4 (lane // 16) + e % 4 of dim lane % 16 of that block
                vmap[4 * (lane // 16) + e % 4, 32 * c + 16 * (e // 4) + lane % 16] = pos
    assert (kmap >= 0).all() and (vmap >= 0).all()
    assert len(set(kmap.ravel())) == 16 * head_dim and len(set(vmap.ravel())) == 16 * head_dim
    return kmap, vmap
