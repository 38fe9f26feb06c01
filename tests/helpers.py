"""Shared test set-up: seeded inputs from `synth`, expected values from `oracle`,
device copies quantised by the library's own kernel."""
from __future__ import annotations

import numpy as np


def rel_l2_rows(y_gpu, y_ref) -> np.ndarray:
    """Per-row relative L2 error ||a - b|| / ||b|| (rows with ||b|| = 0 use ||a||)."""
    a = np.asarray(y_gpu, dtype=np.float64).reshape(len(y_ref), -1)
    b = np.asarray(y_ref, dtype=np.float64).reshape(len(y_ref), -1)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


class ExpertSet:
    """Experts of one layer on both sides: oracle copies (host, quantised by the
    oracle) and device blobs (quantised by coli_quantize_expert from the same
    f32 weights). `which` limits generation to some experts; the others share
    one zero blob on the device and have no oracle copy. `keep_oracle` (set)
    limits the oracle copies further, for large layers checked on samples."""

    def __init__(self, coli, shape, seed=0, layer=0, which=None, dev="cuda", shared=True,
                 keep_oracle=None):
        import torch

        import oracle
        import synth

        self.shape = shape
        H, I, E, G = shape.hidden, shape.inter, shape.n_routed, shape.group
        which = range(E) if which is None else sorted(set(int(e) for e in which))
        nbytes = coli.blob_layout(shape)[1]
        self.zero = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.blobs = [self.zero] * E
        self.oracle = [None] * E
        ids = list(which) + ([E] if shared else [])
        self.shared_blob = None
        self.shared_oracle = None
        for e in ids:
            g, u, d = synth.expert_weights(seed, layer, e, H, I)
            host = keep_oracle is None or e in keep_oracle or e == E
            qe = oracle.QExpert.quantize(g, u, d, G, bits=shape.wbits) if host else None
            blob = coli.quantize_expert(shape, torch.from_numpy(g).to(dev),
                                        torch.from_numpy(u).to(dev), torch.from_numpy(d).to(dev))
            if e == E:
                self.shared_blob, self.shared_oracle = blob, qe
            else:
                self.blobs[e], self.oracle[e] = blob, qe
        self.table = coli.blob_table(self.blobs, dev)

    def oracle_list(self):
        """Oracle experts for the routed ids; ids without a copy get an all-zero expert."""
        import oracle
        H, I, G = self.shape.hidden, self.shape.inter, self.shape.group
        out = []
        zero = None
        for qe in self.oracle:
            if qe is None:
                if zero is None:
                    z = np.zeros((I, H), np.float32)
                    zero = oracle.QExpert.quantize(z, z, np.zeros((H, I), np.float32), G,
                                                   bits=self.shape.wbits)
                qe = zero
            out.append(qe)
        return out


def blob_q_rows(blob, off, part: int, rows: int, row_bytes: int):
    """The weight bytes of blob part `part` (0 gate, 1 up, 2 down) as [rows][row_bytes]
    in row order. Gate and up rows are interleaved in the blob in blocks of 16 rows
    (block b of gate, then block b of up, starting at the gate offset); down rows
    are contiguous."""
    import numpy as np
    if part == 2:
        return blob[off[2]:off[2] + rows * row_bytes].reshape(rows, row_bytes)
    region = blob[off[0]:off[0] + 2 * rows * row_bytes].reshape(2 * rows, row_bytes)
    r = np.arange(rows)
    return region[(r // 16) * 32 + r % 16 + (16 if part == 1 else 0)]
