"""Helpers for the GPU parity tests: host <-> device copies of bf16 bit
patterns, guarded output buffers (a canary past the end of every output
detects writes outside the documented shape), and bitmap decoding."""
import numpy as np
import torch

CANARY = 0xA5


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 (bf16 bits) / float32 / int64 -> CUDA tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


class Guarded:
    """An output tensor followed by 256 canary bytes in the same allocation."""

    def __init__(self, shape, dtype, fill=CANARY):
        n = int(np.prod(shape)) if len(shape) else 1
        esz = torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n * esz
        self.raw = torch.full((self.nbytes + 256,), CANARY, dtype=torch.uint8, device="cuda")
        self.raw[: self.nbytes].fill_(fill)
        self.t = self.raw[: self.nbytes].view(dtype).view(*shape) if n else \
            torch.empty(shape, dtype=dtype, device="cuda")

    def check_tail(self):
        tail = self.raw[self.nbytes:].cpu().numpy()
        assert (tail == CANARY).all(), "write past the end of an output"


def like_bf16_or_f32(a: np.ndarray):
    return torch.bfloat16 if a.dtype == np.uint16 else torch.float32


def unpack_row_bitmap(words: np.ndarray, cols: int) -> np.ndarray:
    """[rows, ceil(cols/32)] uint32 -> bool [rows, cols] (bit b = column 32w+b);
    also returns whether the padding bits are all zero."""
    w = np.ascontiguousarray(words.astype(np.uint32))
    bits = np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1), axis=1, bitorder="little")
    return bits[:, :cols].astype(bool), not bits[:, cols:].any()


def unpack_col_bitmap(words: np.ndarray, rows: int) -> np.ndarray:
    """[ceil(rows/32), cols] uint32 -> bool [rows, cols] (bit b = row 32w+b)."""
    w = words.astype(np.uint32)
    nw, cols = w.shape
    b = ((w[:, None, :] >> np.arange(32, dtype=np.uint32)[None, :, None]) & 1).astype(bool)
    full = b.reshape(nw * 32, cols)
    return full[:rows], not full[rows:].any()


def grouped_rows(counts, block):
    """(start, length) of every block-row, group by group."""
    out = []
    start = 0
    for c in counts:
        c = int(c)
        for r0 in range(start, start + c, block):
            out.append((r0, min(block, start + c - r0)))
        start += c
    return out


def unpack_grouped_bitmap(words: np.ndarray, rows: int, counts, block: int):
    """GROUPED bitmap -> bool [rows, cols]; second value: padding bits zero."""
    w = words.astype(np.uint32)
    cols = w.shape[1]
    out = np.zeros((rows, cols), bool)
    clean = True
    sub = block // 32
    for t, (r0, n) in enumerate(grouped_rows(counts, block)):
        for q in range(sub):
            word = w[t * sub + q]
            for b in range(32):
                r = 32 * q + b
                bit = ((word >> np.uint32(b)) & 1).astype(bool)
                if r < n:
                    out[r0 + r] = bit
                elif bit.any():
                    clean = False
    return out, clean
