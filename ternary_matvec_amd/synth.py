"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no arithmetic of the method (no quantisation, packing or
dot products): it only draws numbers.  Both the HIP path and the CPU oracle
receive its outputs as plain arrays.

Generator: splitmix64 used as a counter-based stream (output i of a stream
with seed s is mix(s + (i + 1) * 0x9E3779B97F4A7C15)), the RNG the cpp20gemma
README uses for reproducible tests, with base seed 42.  Draws:

* uniform u in [0, 1): the top 53 bits of an output times 2^-53;
* normal: Box-Muller on two uniforms, cos branch, then cast to fp32;
* trit: r = (z >> 32) % 10; -1 if r < 3, 0 if r < 7, +1 otherwise, so
  P(-1, 0, +1) = (0.3, 0.4, 0.3);
* bf16: fp32 rounded to nearest even (NaN-free inputs only).
"""
import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
BASE_SEED = 42

# Stream tags: one per kind of tensor, so independent streams never overlap.
TAG_WEIGHT = 1
TAG_ACT = 2
TAG_SCALE = 3
TAG_HEAD = 4
TAG_MISC = 5


def _mix_inplace(z, tmp):
    np.right_shift(z, np.uint64(30), out=tmp)
    z ^= tmp
    z *= _M1
    np.right_shift(z, np.uint64(27), out=tmp)
    z ^= tmp
    z *= _M2
    np.right_shift(z, np.uint64(31), out=tmp)
    z ^= tmp
    return z


def splitmix64_scalar(x: int) -> int:
    """One splitmix64 step on a Python int (used to derive stream seeds)."""
    m = (1 << 64) - 1
    z = (x + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def stream_seed(config_id: int, layer: int, matrix_id: int, tag: int, base: int = BASE_SEED) -> int:
    m = (1 << 64) - 1
    return splitmix64_scalar((base ^ (config_id << 48) ^ (layer << 16) ^ matrix_id ^ (tag << 40)) & m)


def raw(seed: int, count: int, start: int = 0):
    """Outputs start .. start+count-1 of the stream with this seed (uint64)."""
    out = np.empty(count, dtype=np.uint64)
    block = 1 << 16
    tmp = np.empty(block, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for b0 in range(0, count, block):
            b1 = min(count, b0 + block)
            z = out[b0:b1]
            z[:] = np.arange(start + b0 + 1, start + b1 + 1, dtype=np.uint64)
            z *= GOLDEN
            z += np.uint64(seed)
            _mix_inplace(z, tmp[: b1 - b0])
    return out


def uniform(seed: int, count: int, start: int = 0):
    return (raw(seed, count, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, shape, std: float = 1.0):
    count = int(np.prod(shape))
    u = uniform(seed, 2 * count).reshape(count, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    z = r * np.cos(2.0 * np.pi * u[:, 1])
    return (z * std).astype(np.float32).reshape(shape)


_TRIT_OF_DECILE = np.array([-1, -1, -1, 0, 0, 0, 0, 1, 1, 1], dtype=np.int8)


def trits(seed: int, shape, start: int = 0):
    """Trits for outputs start .. start+count-1 of the stream (row-major shape)."""
    count = int(np.prod(shape))
    r = (raw(seed, count, start) >> np.uint64(32)) % np.uint64(10)
    return _TRIT_OF_DECILE[r.astype(np.intp)].reshape(shape)


def zero_groups(seed: int, shape, p_zero: float = 0.8, group: int = 4):
    """A boolean mask of `shape` (last axis = columns) that is True on whole
    groups of `group` consecutive columns, each group independently with
    probability p_zero: the sparse activations of zero-group skipping (the
    ternary page's "What is next": 80% of groups of 4 inputs zero)."""
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    k = shape[-1]
    ng = (k + group - 1) // group
    u = uniform(seed, rows * ng).reshape(rows, ng) < p_zero
    mask = np.repeat(u, group, axis=1)[:, :k]
    return mask.reshape(shape)


def ternary_scale(seed: int) -> float:
    """One per-matrix scale, uniform in [0.01, 0.03)."""
    return float(np.float32(0.01 + 0.02 * uniform(seed, 1)[0]))


def to_bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    b = b + np.uint64(0x7FFF) + lsb
    return (b >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# The workloads named on the pages, as shapes.
# --------------------------------------------------------------------------

# Gemma-3-1B decoder block (d=1152, 4 query heads x 256, 1 kv head x 256,
# ffn 6912): (name, N=out rows, K=in columns).  o_proj is listed apart.
GEMMA_MATS = [("q", 1024, 1152), ("k", 256, 1152), ("v", 256, 1152),
              ("gate", 6912, 1152), ("up", 6912, 1152), ("down", 1152, 6912)]
GEMMA_O = ("o", 1152, 1024)
GEMMA_LAYERS = 26

# BitNet-b1.58-large block (d=1536, ffn 4096), 24 blocks.
BITNET_MATS = [("q", 1536, 1536), ("k", 1536, 1536), ("v", 1536, 1536), ("o", 1536, 1536),
               ("gate", 4096, 1536), ("up", 4096, 1536), ("down", 1536, 4096)]
BITNET_LAYERS = 24

# Output layer: 262144 vocabulary rows x 1152.
HEAD_V, HEAD_K = 262144, 1152

# int8 per-tensor matvec: W 768x288.
INT8_N, INT8_K = 768, 288

CONFIG_INT8, CONFIG_GEMMA_DECODE, CONFIG_GEMMA_PREFILL, CONFIG_HEAD, CONFIG_BITNET = 0, 1, 2, 3, 4


def decode_stack(mats, layers, config_id, m=1, act_seed_config=None):
    """Yield (layer, index, name, N, K, trits, scale, x) for every matrix of a stack.

    trits are int8 [N][K]; x is fp32 [m][K] ~ N(0,1)."""
    acfg = config_id if act_seed_config is None else act_seed_config
    for layer in range(layers):
        for mid, (name, n, k) in enumerate(mats):
            t = trits(stream_seed(config_id, layer, mid, TAG_WEIGHT), (n, k))
            s = ternary_scale(stream_seed(config_id, layer, mid, TAG_SCALE))
            x = normal(stream_seed(acfg, layer, mid, TAG_ACT), (m, k))
            yield layer, mid, name, n, k, t, s, x


# --------------------------------------------------------------------------
# The same counter-based streams drawn with torch (on any device), for inputs
# too large to draw quickly on the host.  Integer draws (raw, trits) are
# bit-identical to the NumPy ones above.  Normal draws use the device's own
# log/cos, so their last bits may differ from the NumPy draw: code that hands
# a torch-drawn tensor to the oracle copies that very tensor to the host.
# --------------------------------------------------------------------------

def _i64(u: int) -> int:
    u &= (1 << 64) - 1
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(z, s: int):
    import torch
    return torch.bitwise_and(torch.bitwise_right_shift(z, s), (1 << (64 - s)) - 1)


def raw_torch(seed: int, count: int, start: int = 0, device="cpu"):
    """int64 tensor holding the uint64 stream outputs (two's complement)."""
    import torch
    z = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z.mul_(_i64(0x9E3779B97F4A7C15)).add_(_i64(seed))
    z.bitwise_xor_(_lsr(z, 30)).mul_(_i64(0xBF58476D1CE4E5B9))
    z.bitwise_xor_(_lsr(z, 27)).mul_(_i64(0x94D049BB133111EB))
    z.bitwise_xor_(_lsr(z, 31))
    return z


def trits_torch(seed: int, shape, device="cpu", start: int = 0, block: int = 1 << 24):
    """Same trits as `trits` (bit-identical), drawn with torch."""
    import torch
    count = int(np.prod(shape))
    lut = torch.tensor(_TRIT_OF_DECILE, dtype=torch.int8, device=device)
    out = torch.empty(count, dtype=torch.int8, device=device)
    for b0 in range(0, count, block):
        b1 = min(count, b0 + block)
        z = raw_torch(seed, b1 - b0, start + b0, device)
        r = torch.remainder(_lsr(z, 32), 10)
        out[b0:b1] = lut[r]
    return out.reshape(shape)


def normal_torch(seed: int, shape, std: float = 1.0, device="cpu", block: int = 1 << 23):
    """N(0, std^2) fp32 draws from the same stream layout as `normal` (device math)."""
    import torch
    count = int(np.prod(shape))
    out = torch.empty(count, dtype=torch.float32, device=device)
    for b0 in range(0, count, block):
        b1 = min(count, b0 + block)
        z = raw_torch(seed, 2 * (b1 - b0), 2 * b0, device)
        u = _lsr(z, 11).to(torch.float64) * (2.0 ** -53)
        u = u.reshape(-1, 2)
        r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
        out[b0:b1] = (r * torch.cos(2.0 * np.pi * u[:, 1]) * std).to(torch.float32)
    return out.reshape(shape)
