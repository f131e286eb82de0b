"""Seeded synthetic inputs: the only module both the oracle side and the HIP
side consume.

It draws *logical* quantities (codes, f16/f32 scales, activations) from seeded
numpy generators and lays them out as raw block bytes.  It holds none of the
method's arithmetic: no decoding, no products, no sums.

Raw byte layouts (little-endian; a tensor is [rows][cols/B] blocks, row-major,
block b of a row covering columns [B*b, B*b+B)):
  Q4_0  18 B / 32 weights: f16 d, then 16 bytes; byte l holds the code of
        column l in its low nibble and of column l+16 in its high nibble.
  Q8_0  34 B / 32 weights: f16 d, then 32 int8 codes in column order.
  Q4_K  144 B / 256 weights: f16 d, f16 dmin, 12 bytes of six-bit (scale, min)
        pairs for the eight 32-wide sub-blocks (the packing that
        get_scale_min_k4 in "Building llamini.cpp" unpacks), then 128 bytes;
        byte 32c+l holds element l of sub-block 2c (low nibble) and of
        sub-block 2c+1 (high nibble).
  Q6_K  210 B / 256 weights: ql[128], qh[64], 16 int8 scales (one per 16
        columns), f16 d (the GGUF layout of the Q4_K_M files the pages load).
        Column c = 128h + 32j + l keeps its low four bits in ql[64h + 32(j mod
        2) + l] (low nibble for j < 2, high for j >= 2) and its top two bits in
        bits 2j, 2j+1 of qh[32h + l].
  I8ROW int8 [rows][cols] codes plus one fp32 scale per row.

Distributions follow the five workload descriptions (the quantized FFN of a
stories15M-sized model, a SmolLM2-135M decode layer with a Q8_0 vocab head, a
TinyLlama-1.1B layer in Q4_K, a SmolLM2-1.7B-sized per-row INT8 FFN and head,
and a 27B-class dense FFN), plus TinyLlama-1.1B's Q6_K tensors (the down
projection and the vocab head of a Q4_K_M file).  Every tensor has its own stream:
numpy.random.default_rng(SeedSequence([seed, cfg_id, tensor_idx])).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

FMT_BLOCK = {"q4_0": (32, 18), "q8_0": (32, 34), "q4_k": (256, 144), "q6_k": (256, 210)}


# --------------------------------------------------------------------------
# byte layout of logical arrays (encoding only)
# --------------------------------------------------------------------------
def _f16_bytes(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype="<f2")
    return a.view(np.uint8).reshape(a.shape + (2,))


def pack_q4_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d: float16 [rows][cols/32]; q: codes 0..15 [rows][cols] -> uint8 [rows][cols/32*18]."""
    rows, cols = q.shape
    nb = cols // 32
    assert cols % 32 == 0 and d.shape == (rows, nb)
    qb = np.asarray(q, dtype=np.uint8).reshape(rows, nb, 32)
    assert int(qb.max(initial=0)) < 16
    raw = np.empty((rows, nb, 18), dtype=np.uint8)
    raw[:, :, 0:2] = _f16_bytes(d)
    raw[:, :, 2:18] = qb[:, :, 0:16] | (qb[:, :, 16:32] << 4)
    return raw.reshape(rows, nb * 18)


def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d: float16 [rows][cols/32]; q: int8 [rows][cols] -> uint8 [rows][cols/32*34]."""
    rows, cols = q.shape
    nb = cols // 32
    assert cols % 32 == 0 and d.shape == (rows, nb)
    raw = np.empty((rows, nb, 34), dtype=np.uint8)
    raw[:, :, 0:2] = _f16_bytes(d)
    raw[:, :, 2:34] = np.ascontiguousarray(q, dtype=np.int8).view(np.uint8).reshape(rows, nb, 32)
    return raw.reshape(rows, nb * 34)


def pack_q4_k_scales(sc: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Six-bit (scale, min) pairs [..., 8] -> the 12-byte field [..., 12].

    Sub-blocks 0-3 sit in the low six bits of bytes 0-3 (scale) and 4-7 (min);
    sub-blocks 4-7 keep their low four bits in bytes 8-11 (scale low nibble,
    min high nibble) and their top two bits in the spare bits 6-7 of bytes 0-3
    (scale) and 4-7 (min)."""
    sc = np.asarray(sc, dtype=np.uint8)
    m = np.asarray(m, dtype=np.uint8)
    assert int(sc.max(initial=0)) < 64 and int(m.max(initial=0)) < 64
    out = np.empty(sc.shape[:-1] + (12,), dtype=np.uint8)
    out[..., 0:4] = sc[..., 0:4] | ((sc[..., 4:8] >> 4) << 6)
    out[..., 4:8] = m[..., 0:4] | ((m[..., 4:8] >> 4) << 6)
    out[..., 8:12] = (sc[..., 4:8] & 0x0F) | ((m[..., 4:8] & 0x0F) << 4)
    return out


def pack_q4_k(d, dmin, sc, m, q) -> np.ndarray:
    """d, dmin: float16 [rows][nsb]; sc, m: 0..63 [rows][nsb][8]; q: 0..15 [rows][cols]."""
    rows, cols = q.shape
    nsb = cols // 256
    assert cols % 256 == 0 and d.shape == (rows, nsb) and dmin.shape == (rows, nsb)
    raw = np.empty((rows, nsb, 144), dtype=np.uint8)
    raw[:, :, 0:2] = _f16_bytes(d)
    raw[:, :, 2:4] = _f16_bytes(dmin)
    raw[:, :, 4:16] = pack_q4_k_scales(sc, m)
    qs = np.asarray(q, dtype=np.uint8).reshape(rows, nsb, 8, 32)
    assert int(qs.max(initial=0)) < 16
    raw[:, :, 16:144] = (qs[:, :, 0::2, :] | (qs[:, :, 1::2, :] << 4)).reshape(rows, nsb, 128)
    return raw.reshape(rows, nsb * 144)


def pack_q6_k(d, sc, q) -> np.ndarray:
    """d: float16 [rows][nsb]; sc: int8 [rows][nsb][16]; q: 0..63 [rows][cols]."""
    rows, cols = q.shape
    nsb = cols // 256
    assert cols % 256 == 0 and d.shape == (rows, nsb) and sc.shape == (rows, nsb, 16)
    c = np.asarray(q, dtype=np.uint8).reshape(rows, nsb, 2, 4, 32)   # [h][j][l]
    assert int(c.max(initial=0)) < 64
    lo, hi = c & 0x0F, c >> 4
    raw = np.empty((rows, nsb, 210), dtype=np.uint8)
    ql = np.empty((rows, nsb, 2, 2, 32), dtype=np.uint8)             # [h][j mod 2][l]
    ql[:, :, :, 0, :] = lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4)
    ql[:, :, :, 1, :] = lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)
    raw[:, :, 0:128] = ql.reshape(rows, nsb, 128)
    qh = hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4) | (hi[:, :, :, 3, :] << 6)
    raw[:, :, 128:192] = qh.reshape(rows, nsb, 64)
    raw[:, :, 192:208] = np.ascontiguousarray(sc, dtype=np.int8).view(np.uint8)
    raw[:, :, 208:210] = _f16_bytes(d)
    return raw.reshape(rows, nsb * 210)


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------
def rng_for(seed: int, cfg_id: int, tensor_idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_idx]))


@dataclass
class QTensor:
    """One quantized weight tensor: raw bytes plus the logical values it encodes."""
    name: str
    fmt: str
    rows: int
    cols: int
    raw: np.ndarray                      # uint8 raw blocks (int8 codes for i8row)
    row_scale: Optional[np.ndarray] = None  # fp32 [rows] for i8row
    logical: Dict[str, np.ndarray] = field(default_factory=dict)

    @property
    def weight_bytes(self) -> int:
        return algorithmic_bytes(self.fmt, self.rows, self.cols)


def algorithmic_bytes(fmt: str, rows: int, cols: int) -> int:
    """Bytes the method must stream for one pass over the tensor."""
    if fmt == "i8row":
        return rows * cols + 4 * rows
    per, nbytes = FMT_BLOCK[fmt]
    return rows * (cols // per) * nbytes


def draw_q4_0(rng, rows, cols, d_lo=0.005, d_hi=0.05):
    d = rng.uniform(d_lo, d_hi, (rows, cols // 32)).astype(np.float16)
    q = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    return d, q


def draw_q8_0(rng, rows, cols, d_lo=0.001, d_hi=0.02):
    d = rng.uniform(d_lo, d_hi, (rows, cols // 32)).astype(np.float16)
    q = rng.integers(-127, 128, (rows, cols), dtype=np.int8)
    return d, q


def draw_q4_k(rng, rows, cols, d_lo=1e-4, d_hi=1e-3):
    nsb = cols // 256
    d = rng.uniform(d_lo, d_hi, (rows, nsb)).astype(np.float16)
    dmin = rng.uniform(d_lo, d_hi, (rows, nsb)).astype(np.float16)
    sc = rng.integers(0, 64, (rows, nsb, 8), dtype=np.uint8)
    m = rng.integers(0, 64, (rows, nsb, 8), dtype=np.uint8)
    q = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    return d, dmin, sc, m, q


def draw_q6_k(rng, rows, cols, d_lo=1e-4, d_hi=1e-3):
    nsb = cols // 256
    d = rng.uniform(d_lo, d_hi, (rows, nsb)).astype(np.float16)
    sc = rng.integers(-128, 128, (rows, nsb, 16), dtype=np.int8)
    q = rng.integers(0, 64, (rows, cols), dtype=np.uint8)
    return d, sc, q


def draw_i8row(rng, rows, cols, s_lo=1e-4, s_hi=1e-3):
    q = np.clip(np.rint(rng.normal(0.0, 40.0, (rows, cols))), -127, 127).astype(np.int8)
    s = rng.uniform(s_lo, s_hi, rows).astype(np.float32)
    return q, s


def make_tensor(fmt: str, rows: int, cols: int, rng: np.random.Generator, name: str = "w",
                keep_logical: bool = False) -> QTensor:
    if fmt == "q4_0":
        d, q = draw_q4_0(rng, rows, cols)
        t = QTensor(name, fmt, rows, cols, pack_q4_0(d, q))
        if keep_logical:
            t.logical = {"d": d, "q": q}
    elif fmt == "q8_0":
        d, q = draw_q8_0(rng, rows, cols)
        t = QTensor(name, fmt, rows, cols, pack_q8_0(d, q))
        if keep_logical:
            t.logical = {"d": d, "q": q}
    elif fmt == "q4_k":
        d, dmin, sc, m, q = draw_q4_k(rng, rows, cols)
        t = QTensor(name, fmt, rows, cols, pack_q4_k(d, dmin, sc, m, q))
        if keep_logical:
            t.logical = {"d": d, "dmin": dmin, "sc": sc, "m": m, "q": q}
    elif fmt == "q6_k":
        d, sc, q = draw_q6_k(rng, rows, cols)
        t = QTensor(name, fmt, rows, cols, pack_q6_k(d, sc, q))
        if keep_logical:
            t.logical = {"d": d, "sc": sc, "q": q}
    elif fmt == "i8row":
        q, s = draw_i8row(rng, rows, cols)
        t = QTensor(name, fmt, rows, cols, q, row_scale=s)
        if keep_logical:
            t.logical = {"q": q, "s": s}
    else:
        raise ValueError(fmt)
    return t


def draw_x(rng, n_tok, cols) -> np.ndarray:
    return rng.standard_normal((n_tok, cols)).astype(np.float32)


# --------------------------------------------------------------------------
# workload registry
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    kind: str                                    # "ffn" or "gemvs"
    tensors: Tuple[Tuple[str, str, int, int], ...]  # (name, fmt, rows, cols)
    n_tok: Tuple[int, ...] = (1,)
    d_model: int = 0
    ffn: int = 0


WORKLOADS: Dict[str, Workload] = {}


def _reg(w: Workload):
    WORKLOADS[w.name] = w
    return w


CFG1 = _reg(Workload(1, "ffn_q4_0_288x768", "ffn",
                     (("gate", "q4_0", 768, 288), ("up", "q4_0", 768, 288), ("down", "q4_0", 288, 768)),
                     d_model=288, ffn=768))
CFG2 = _reg(Workload(2, "smollm2_135m_layer_q4_0_head_q8_0", "gemvs",
                     (("q", "q4_0", 576, 576), ("o", "q4_0", 576, 576),
                      ("k", "q4_0", 192, 576), ("v", "q4_0", 192, 576),
                      ("gate", "q4_0", 1536, 576), ("up", "q4_0", 1536, 576),
                      ("down", "q4_0", 576, 1536), ("head", "q8_0", 49152, 576)),
                     d_model=576, ffn=1536))
CFG3 = _reg(Workload(3, "tinyllama_1.1b_layer_q4_k", "gemvs",
                     (("attn_2048x2048", "q4_k", 2048, 2048),
                      ("k", "q4_k", 256, 2048), ("v", "q4_k", 256, 2048),
                      ("gate", "q4_k", 5632, 2048), ("up", "q4_k", 5632, 2048),
                      ("down", "q4_k", 2048, 5632)),
                     d_model=2048, ffn=5632))
CFG4 = _reg(Workload(4, "smollm2_1.7b_i8row_ffn_head", "gemvs",
                     (("gate", "i8row", 8192, 2048), ("up", "i8row", 8192, 2048),
                      ("down", "i8row", 2048, 8192), ("head", "i8row", 49152, 2048)),
                     d_model=2048, ffn=8192))
CFG5 = _reg(Workload(5, "dense27b_ffn_q4_0_5120x17408", "ffn",
                     (("gate", "q4_0", 17408, 5120), ("up", "q4_0", 17408, 5120),
                      ("down", "q4_0", 5120, 17408)),
                     n_tok=(1, 8, 128), d_model=5120, ffn=17408))
CFG6 = _reg(Workload(6, "tinyllama_1.1b_q6_k_down_head", "gemvs",
                     (("down", "q6_k", 2048, 5632), ("head", "q6_k", 32000, 2048)),
                     d_model=2048, ffn=5632))


def gen_tensor(w: Workload, idx: int, seed: int = 0, keep_logical: bool = False) -> QTensor:
    name, fmt, rows, cols = w.tensors[idx]
    return make_tensor(fmt, rows, cols, rng_for(seed, w.cfg_id, idx), name, keep_logical)


def gen_x(w: Workload, cols: int, n_tok: int = 1, seed: int = 0, which: int = 0) -> np.ndarray:
    """Activations: drawn after every weight tensor (tensor index len(tensors)+which).
    Independent of n_tok in the sense that the first token is the same row for
    every n_tok only when drawn with the largest n_tok; each (cols, n_tok) call
    is its own stream slot, selected by `which`."""
    return draw_x(rng_for(seed, w.cfg_id, len(w.tensors) + which), n_tok, cols)


def gen_workload(w: Workload, seed: int = 0, keep_logical: bool = False) -> List[QTensor]:
    return [gen_tensor(w, i, seed, keep_logical) for i in range(len(w.tensors))]
