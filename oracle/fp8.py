"""CPU float64 oracle of the FP8 forward: block quantisation, the incoherent
rotation, and attention on the quantised operands.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product path.

Sources (cited by page title and section):

* FlashAttention: Part 2, section 1.6 "FA3 FP8": the FP8 path controls the
  error with block quantisation (each tile scaled relative to its own
  values, not one global scale) and incoherent processing (Q and K
  multiplied by a random orthogonal matrix before quantisation, spreading
  outliers over the head dimension); the algorithm is still
  softmax(Q K^T) V, only the arithmetic is FP8.
* The e4m3 format itself (OCP 8-bit floating point, "E4M3"): 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits, subnormals at exponent field
  0, largest finite value 448, no infinities.

Readings where the pages are silent (each one listed in the design notes):

* Blocks are 64 consecutive rows of one (batch, head), all head_dim
  columns; the last block of a sequence is padded with zero rows.
* A block's scale is a power of two 2^e, e the smallest integer with
  amax <= 448 * 2^e (e = 0 for an all-zero block), clamped to [-127, 127];
  codes are round-to-nearest-even e4m3 of x * 2^-e.
* The random orthogonal matrix is the randomised Hadamard transform
  R = H_d diag(s) / sqrt(d) (H_d the Sylvester Hadamard matrix, s a given
  vector of signs), applied to every row of Q and K: Q K^T is unchanged.
* Both products run on FP8: S from the quantised Q and K, and P V from the
  quantised V and P quantised as e4m3 of 2^(t - M + 6), t = scale log2(e) S
  and M = ceil(max t) of the row (an integer, so the code of a probability
  does not depend on which reference the online recurrence used); the
  softmax denominator uses the unquantised probabilities. O = 2^-6
  sum_j P'_j V_j / sum_j 2^(t_j - M), LSE = ln 2 (M + log2 sum_j 2^(t_j - M)).
"""

import math

import numpy as np

__all__ = [
    "E4M3_MAX",
    "BLOCK",
    "P_BIAS",
    "e4m3_decode",
    "e4m3_encode",
    "hadamard",
    "rotate",
    "block_exponent",
    "quantize_rows",
    "quantize_bhnd",
    "dequantize_bhnd",
    "attention_fp8",
]

E4M3_MAX = 448.0
BLOCK = 64     # rows per quantisation block
P_BIAS = 6     # probabilities are quantised as e4m3(2^(t - M + P_BIAS))


def e4m3_decode(codes):
    """Values of e4m3 codes (uint8 array) from the format definition; the
    two NaN codes (exponent and mantissa all ones) decode to NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (ex - 7))
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return sign * val


_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)           # +0 .. 448, increasing
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x):
    """Round-to-nearest-even e4m3 codes of finite values with |x| <= 448.

    The nearest representable magnitude is found among all 127 finite
    non-negative codes; at an exact tie the code with an even mantissa wins.
    Zero and negative zero both give 0x00 and 0x80 by sign.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: values must be finite and within +-448")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def hadamard(d):
    """Sylvester Hadamard matrix H_d (entries +-1), d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs):
    """Rows of x (..., d) times R^T with R = H_d diag(signs) / sqrt(d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    R = hadamard(d) * np.asarray(signs, dtype=np.float64)[None, :] / math.sqrt(d)
    return x @ R.T


def block_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 for amax = 0), clamped
    to [-127, 127]."""
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    # log2 rounding near a power of two: settle on the exact inequality
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(-127, min(127, e))


def quantize_rows(x):
    """Block quantisation of one (rows, d) head: returns codes (rows_padded,
    d) uint8 and block exponents (rows_padded / 64,) int, rows_padded the
    row count rounded up to 64 (padding rows are zero)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    npad = -(-n // BLOCK) * BLOCK
    xp = np.zeros((npad, d))
    xp[:n] = x
    codes = np.zeros((npad, d), dtype=np.uint8)
    exps = np.zeros(npad // BLOCK, dtype=np.int64)
    for blk in range(npad // BLOCK):
        rows = xp[blk * BLOCK:(blk + 1) * BLOCK]
        e = block_exponent(float(np.max(np.abs(rows))))
        exps[blk] = e
        codes[blk * BLOCK:(blk + 1) * BLOCK] = e4m3_encode(rows * 2.0 ** (-e))
    return codes, exps


def quantize_bhnd(x, signs=None):
    """Quantise a (B, N, H, d) tensor head by head, rotating rows first when
    ``signs`` is given. Returns codes (B, H, N_padded, d) and exponents
    (B, H, N_padded / 64)."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, d = x.shape
    npad = -(-N // BLOCK) * BLOCK
    codes = np.zeros((B, H, npad, d), dtype=np.uint8)
    exps = np.zeros((B, H, npad // BLOCK), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rows = x[b, :, h, :]
            if signs is not None:
                rows = rotate(rows, signs)
            codes[b, h], exps[b, h] = quantize_rows(rows)
    return codes, exps


def dequantize_bhnd(codes, exps):
    """Values of (B, H, N_padded, d) codes with per-64-row exponents."""
    vals = e4m3_decode(codes)
    return vals * np.repeat(2.0 ** np.asarray(exps, dtype=np.float64), BLOCK, axis=2)[..., None]


def attention_fp8(q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, Nq, Nk, causal, scale):
    """Attention on quantised operands, probabilities quantised as stated in
    the module docstring. Codes are (B, H, N_padded, d) as from
    ``quantize_bhnd`` (V in the same row layout); only the first Nq / Nk rows
    take part. Causal is top-left (key j visible to query i iff j <= i).
    Returns O (B, Nq, Hq, d) and LSE (B, Hq, Nq) in float64; a query that
    sees no key gets O = 0 and LSE = -inf.
    """
    Q = dequantize_bhnd(q_codes, q_exps)[:, :, :Nq]
    K = dequantize_bhnd(k_codes, k_exps)[:, :, :Nk]
    V = dequantize_bhnd(v_codes, v_exps)[:, :, :Nk]
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    c = scale * math.log2(math.e)
    O = np.zeros((B, Nq, Hq, V.shape[3]))
    L = np.full((B, Hq, Nq), -np.inf)
    j = np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            t = c * (Q[b, h] @ K[b, kv].T)
            for i in range(Nq):
                vis = (j <= i) if causal else np.ones(Nk, dtype=bool)
                if not vis.any():
                    continue
                ti = t[i, vis]
                M = math.ceil(float(np.max(ti)))
                p = 2.0 ** (ti - M)
                pq = e4m3_decode(e4m3_encode(2.0 ** (ti - M + P_BIAS)))
                den = float(np.sum(p))
                O[b, i, h] = 2.0 ** (-P_BIAS) * (pq @ V[b, kv][vis]) / den
                L[b, h, i] = math.log(2.0) * (M + math.log2(den))
    return O, L
