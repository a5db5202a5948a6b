"""Seeded synthetic inputs shaped like diffusion-transformer linear layers.

This module only draws random numbers; it holds none of the quantizer's
arithmetic.  Both the HIP path's tests/benchmark and the CPU oracle take
their inputs from here, so the two sides see the same bytes.

Stand-ins: the pages evaluate on FLUX.1, Z-Image-Turbo, Wan 2.1 and
CogVideoX activations under GenEval / VBench prompts.  None of those models,
weights or suites exist here; these generators reproduce only the *shapes*
and the qualitative structure the pages attribute to DiT activations
(channel-wise outliers, per-token scale drift, GELU-skewed MLP inputs,
heavy tails, all-zero tokens).

Generation is addressable by row: rows are produced in blocks of
``BLOCK_ROWS`` and block ``b`` of an instance uses its own generator
``numpy.random.default_rng([data_seed, instance_tag, 1, b])``, so a sampled
subset of rows can be regenerated without drawing the whole matrix.
"""
import numpy as np

BLOCK_ROWS = 256

F32, BF16 = 0, 1


def f32_to_bf16_bits(a):
    """Round fp32 -> bf16 to nearest even; returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ recipes --

class ActRecipe:
    """One activation matrix [M, d]."""

    def __init__(self, tag, M, d, dtype, base, n_out, out_factor, sigma_s,
                 zero_frac=0.0, zero_rows=()):
        self.tag, self.M, self.d, self.dtype = tag, M, d, dtype
        self.base, self.n_out, self.out_factor = base, n_out, out_factor
        self.sigma_s, self.zero_frac, self.zero_rows = sigma_s, zero_frac, tuple(zero_rows)


class WeightRecipe:
    """One weight matrix [N, K] (torch Linear convention), N(0, std^2)."""

    def __init__(self, tag, N, K, dtype, std=0.02):
        self.tag, self.N, self.K, self.dtype, self.std = tag, N, K, dtype, std


class Linear:
    def __init__(self, name, act, weight, seed, bit_pairs):
        self.name, self.act, self.weight, self.seed = name, act, weight, seed
        self.bit_pairs = bit_pairs  # list of (w_bits, a_bits)


def _n_out(frac, d):
    return max(1, int(round(frac * d)))


def _configs():
    c = {}
    # 1. tiny single linear, fp32 (parity-only case the oracle finishes in seconds)
    a1 = ActRecipe(101_0, 64, 256, F32, "normal", 2, 20.0, 1.0)
    c["tiny"] = dict(seed=101, linears=[
        Linear("tiny", a1, WeightRecipe(101_1, 256, 256, F32), 11, [(4, 4)])])
    # 2. image-DiT fused QKV projection: 2 CFG branches x (4096 latent + 512 text)
    a2 = ActRecipe(102_0, 9216, 3072, BF16, "normal", _n_out(0.01, 3072), 50.0, 1.5)
    c["image_qkv"] = dict(seed=102, linears=[
        Linear("qkv", a2, WeightRecipe(102_1, 9216, 3072, BF16), 21, [(4, 4)])])
    # 3. image-DiT MLP pair
    a3u = ActRecipe(103_0, 9216, 3072, BF16, "normal", 2, 20.0, 1.0)
    a3d = ActRecipe(103_1, 9216, 12288, BF16, "gelu", _n_out(0.005, 12288), 80.0, 0.0)
    c["image_mlp"] = dict(seed=103, linears=[
        Linear("up", a3u, WeightRecipe(103_2, 12288, 3072, BF16), 31, [(4, 4), (2, 4)]),
        Linear("down", a3d, WeightRecipe(103_3, 3072, 12288, BF16), 32, [(4, 4), (2, 4)])])
    # 4. video-DiT block: 21 x 30 x 52 latent tokens
    a4q = ActRecipe(104_0, 32760, 5120, BF16, "normal", _n_out(0.01, 5120), 50.0, 2.0)
    a4u = ActRecipe(104_1, 32760, 5120, BF16, "normal", _n_out(0.01, 5120), 50.0, 2.0)
    a4d = ActRecipe(104_2, 32760, 13824, BF16, "normal", _n_out(0.01, 13824), 50.0, 2.0)
    c["video_block"] = dict(seed=104, linears=[
        Linear("qkv", a4q, WeightRecipe(104_3, 15360, 5120, BF16), 41, [(4, 4), (3, 4)]),
        Linear("up", a4u, WeightRecipe(104_4, 13824, 5120, BF16), 42, [(4, 4), (3, 4)]),
        Linear("down", a4d, WeightRecipe(104_5, 5120, 13824, BF16), 43, [(4, 4), (3, 4)])])
    # 5. stress: heavy tails, extreme bits, all-zero tokens
    a5 = ActRecipe(105_0, 65536, 3072, BF16, "student_t3", _n_out(0.005, 3072), 100.0, 2.0,
                   zero_frac=0.01, zero_rows=(0, 65535))
    c["stress"] = dict(seed=105, linears=[
        Linear("proj", a5, WeightRecipe(105_1, 3072, 3072, BF16), 51, [(2, 3), (2, 4)])])
    return c


CONFIGS = _configs()
CONFIG_ORDER = ["tiny", "image_qkv", "image_mlp", "video_block", "stress"]


def get_linear(cfg, name):
    for lin in CONFIGS[cfg]["linears"]:
        if lin.name == name:
            return lin
    raise KeyError((cfg, name))


# --------------------------------------------------------------- generation --

def _outlier_channels(data_seed, rec):
    rng = np.random.default_rng([data_seed, rec.tag, 0])
    return np.sort(rng.choice(rec.d, size=rec.n_out, replace=False))


def _zero_rows(data_seed, rec):
    rows = set(r for r in rec.zero_rows if r < rec.M)
    if rec.zero_frac > 0:
        rng = np.random.default_rng([data_seed, rec.tag, 2])
        n = int(round(rec.zero_frac * rec.M))
        rows.update(int(r) for r in rng.choice(rec.M, size=n, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def _gelu_erf(x):
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def _block_f32(data_seed, rec, b, ch):
    r0 = b * BLOCK_ROWS
    nr = min(BLOCK_ROWS, rec.M - r0)
    rng = np.random.default_rng([data_seed, rec.tag, 1, b])
    if rec.base == "normal":
        x = rng.standard_normal((nr, rec.d), dtype=np.float32)
    elif rec.base == "gelu":
        x = _gelu_erf(rng.standard_normal((nr, rec.d), dtype=np.float32)).astype(np.float32)
    elif rec.base == "student_t3":
        x = rng.standard_t(3.0, size=(nr, rec.d)).astype(np.float32)
    else:
        raise ValueError(rec.base)
    x[:, ch] *= np.float32(rec.out_factor)
    if rec.sigma_s > 0:
        s = np.exp(rec.sigma_s * rng.standard_normal(nr)).astype(np.float32)
        x *= s[:, None]
    return x


def activations(cfg, name, rows=None):
    """Activation matrix of linear `name` in config `cfg`.

    Returns float32 [R, d] (fp32 recipes) or uint16 bf16 bit patterns.
    `rows`: optional sorted array of row indices (default: all rows)."""
    data_seed = CONFIGS[cfg]["seed"]
    rec = get_linear(cfg, name).act
    ch = _outlier_channels(data_seed, rec)
    zr = _zero_rows(data_seed, rec)
    if rows is None:
        rows = np.arange(rec.M, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], rec.d), np.float32 if rec.dtype == F32 else np.uint16)
    blocks = np.unique(rows // BLOCK_ROWS)
    for b in blocks:
        sel = np.nonzero(rows // BLOCK_ROWS == b)[0]
        xb = _block_f32(data_seed, rec, int(b), ch)
        local = rows[sel] - b * BLOCK_ROWS
        xs = xb[local]
        zmask = np.isin(rows[sel], zr)
        xs[zmask] = 0.0
        out[sel] = xs if rec.dtype == F32 else f32_to_bf16_bits(xs)
    return out


def weights(cfg, name):
    """Weight matrix [N, K] of linear `name` (float32 or bf16 bits)."""
    data_seed = CONFIGS[cfg]["seed"]
    rec = get_linear(cfg, name).weight
    out = np.empty((rec.N, rec.K), np.float32 if rec.dtype == F32 else np.uint16)
    for b in range(0, rec.N, BLOCK_ROWS):
        rng = np.random.default_rng([data_seed, rec.tag, 1, b // BLOCK_ROWS])
        nr = min(BLOCK_ROWS, rec.N - b)
        w = rng.standard_normal((nr, rec.K), dtype=np.float32) * np.float32(rec.std)
        out[b:b + nr] = w if rec.dtype == F32 else f32_to_bf16_bits(w)
    return out


def custom_activations(M, d, dtype, seed, base="normal", n_out=0, out_factor=1.0,
                       sigma_s=0.0, zero_rows=()):
    """Small ad-hoc activation matrices for edge-case tests (same recipe family)."""
    rec = ActRecipe(seed, M, d, dtype, base, max(n_out, 1), out_factor if n_out else 1.0,
                    sigma_s, zero_rows=zero_rows)
    ch = _outlier_channels(seed, rec)
    out = np.empty((M, d), np.float32)
    for b in range(0, M, BLOCK_ROWS):
        nr = min(BLOCK_ROWS, M - b)
        out[b:b + nr] = _block_f32(seed, rec, b // BLOCK_ROWS, ch)[:nr]
    for r in zero_rows:
        if r < M:
            out[r] = 0.0
    return out if dtype == F32 else f32_to_bf16_bits(out)


# AdaLN modulation projections (INT4 weight-only, not rotated): one input
# row per sample (2 = the two guidance branches), hidden size K, 6 K outputs
# (shift, scale, gate for attention and MLP).  Input SiLU(N(0, 1)) as the
# conditioning vector after its activation; weights N(0, 0.02^2).  Shapes of
# an image DiT (3072) and a video DiT (5120) block.
ADALN = {"image": (2, 3072, 6 * 3072, 61), "video": (2, 5120, 6 * 5120, 62)}


def adaln_inputs(name):
    """(x bf16 bits [M, K], W bf16 bits [N, K]) of an AdaLN projection."""
    M, K, N, seed = ADALN[name]
    rng = np.random.default_rng([seed, 1])
    c = rng.standard_normal((M, K)).astype(np.float32)
    x = c / (1.0 + np.exp(-c))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return f32_to_bf16_bits(x.astype(np.float32)), f32_to_bf16_bits(W)


def random_codes(rows, K, bits, seed):
    """Uniformly random packed code bytes [rows, K*bits/8] and positive norms."""
    rng = np.random.default_rng([seed, 7])
    codes = rng.integers(0, 256, size=(rows, K * bits // 8), dtype=np.uint8)
    norms = np.exp(rng.standard_normal(rows)).astype(np.float32)
    return codes, norms


def sample_rows(M, n, seed):
    """A seeded sorted sample of n distinct row indices in [0, M), always
    including the first and last row."""
    rng = np.random.default_rng([seed, 9])
    n = min(n, M)
    inner = rng.choice(np.arange(1, M - 1), size=max(0, n - 2), replace=False) if M > 2 else []
    rows = np.unique(np.concatenate([[0, M - 1], np.asarray(inner, dtype=np.int64)]))
    return rows.astype(np.int64)
