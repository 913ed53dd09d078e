"""Helpers for the GPU parity tests: host <-> device copies of the synthetic
inputs (bf16 travels as its uint16 bit pattern) and the error measures."""
import numpy as np

import synth


def torch():
    import torch as _t
    return _t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(t.bfloat16).cuda()


def dev_f32(x: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_bf16_bits(x) -> np.ndarray:
    t = torch()
    return x.detach().contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def host_bf16_f32(x) -> np.ndarray:
    return synth.bf16_to_f32(host_bf16_bits(x))


def host(x) -> np.ndarray:
    return x.detach().cpu().numpy()


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print(f"[gpu case] {msg}", flush=True)


def max_tile_rel(got, ref, tile=(256, 256)) -> float:
    """Largest relative Frobenius error over the tiles of a 2-D result (tiles
    of `tile` rows x columns, clipped at the edges). A wrong tile, column
    strip or tile edge that holds a tiny share of the whole tensor's energy
    still fails this bound. A tile whose reference is zero counts as 0 if the
    result is zero there too, else as infinite."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.ndim == 1:
        got, ref = got[None, :], ref[None, :]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    tr, tc = tile
    worst = 0.0
    for r0 in range(0, ref.shape[0], tr):
        for c0 in range(0, ref.shape[1], tc):
            g = got[r0:r0 + tr, c0:c0 + tc]
            f = ref[r0:r0 + tr, c0:c0 + tc]
            den = np.linalg.norm(f)
            num = np.linalg.norm(g - f)
            e = (0.0 if num == 0.0 else float("inf")) if den == 0.0 else float(num / den)
            worst = max(worst, e)
    return worst
