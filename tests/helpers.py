"""Shared test helpers: moving storage bits to and from the device, tolerances."""
import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

TORCH_DTYPE = None
if torch is not None:
    TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Tolerances against the fp64 oracle on the same rounded inputs.
MAX_ABS = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
MEAN_ABS = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}
LSE_ABS = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def to_dev(x: np.ndarray, dtype: str, device="cuda"):
    """Storage bits (synth) -> device tensor of the matching torch dtype (bit copy)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device)
    return t.view(TORCH_DTYPE[dtype])


def to_dev_i32(x: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def bits_of(t) -> np.ndarray:
    """Device tensor -> storage bits as numpy (uint16 for 16-bit types, float32 for f32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def values_of(t) -> np.ndarray:
    """Device tensor -> exact fp64 values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of |ref| in a 16-bit storage type (0 for f32)."""
    if dtype == "f32":
        return np.zeros_like(ref)
    frac_bits = {"bf16": 7, "f16": 10}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    return np.exp2(e - frac_bits - 1)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "O", storage_slack: bool = False):
    """max-abs / mean-abs bar against the fp64 oracle.

    ``storage_slack``: the output is stored in a 16-bit type, and rounding the
    exact value to that type alone costs up to half an ulp (0.0156 for |O| in
    [4, 8) in bf16); the bar then applies to the arithmetic and each element may
    carry its own storage rounding on top.  The arithmetic alone is checked
    separately through the kernels' fp32-output mode.
    """
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    lim_max = MAX_ABS[dtype]
    lim_mean = MEAN_ABS[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if storage_slack:
        excess = err - half_ulp(ref, dtype)
        assert float(excess.max()) <= lim_max, \
            f"{what}: max-abs beyond storage rounding {float(excess.max()):.3e} > {lim_max:.0e}"
    else:
        assert mx <= lim_max, f"{what}: max-abs {mx:.3e} > {lim_max:.0e} (mean {mean:.3e})"
    assert mean <= lim_mean, f"{what}: mean-abs {mean:.3e} > {lim_mean:.0e}"
    return mx, mean


def assert_lse_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "lse"):
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), f"{what}: -inf pattern differs"
    if finite.any():
        mx = float(np.abs(got[finite] - ref[finite]).max())
        assert mx <= LSE_ABS[dtype], f"{what}: max-abs {mx:.3e} > {LSE_ABS[dtype]:.0e}"


def assert_stored_output(o16, o32, ref: np.ndarray, dtype: str, what: str = "O"):
    """The acceptance rule for every output stored in a 16-bit type.

    ``o32`` is the same call with the fp32-output option: its arithmetic must meet
    the bar on its own (max-abs and mean-abs against the fp64 oracle); the stored
    16-bit output ``o16`` must be exactly ``o32`` rounded to nearest-even; and
    ``o16`` then lies within the bar of the oracle plus its own storage rounding
    (half an ulp of the exact value) in each element.  Returns (max, mean) of the
    fp32 output's error.
    """
    mx, mean = assert_close(values_of(o32), ref, dtype, what=f"{what} (fp32 output)")
    import synth  # storage rounding of the fp32 result (input preparation code, no attention arithmetic)
    assert np.array_equal(bits_of(o16), synth.to_storage(o32.detach().cpu().numpy(), dtype)), \
        f"{what}: 16-bit output is not the round-to-nearest-even of the fp32 result"
    assert_close(values_of(o16), ref, dtype, what=what, storage_slack=True)
    return mx, mean


def poison_table_tail(table, lens, num_blocks):
    """The block table with every entry past each sequence's last block (the
    sequence holds lens[b] keys) replaced by an id outside the pool: a kernel
    that reads one of them raises the bad-block flag.  Numpy in, numpy out."""
    t = table.copy()
    for b in range(t.shape[0]):
        used = -(-int(lens[b]) // 16)
        t[b, used:] = -7 if b % 2 == 0 else num_blocks + 1000
    return t


def extreme_queries(inp, dtype):
    """Edit decode inputs in place so that query heads stress the score path: an
    all-zero head, one dominant channel over tiny ones, a head of tiny values and
    a head of large values (logits near 60); with per-channel key scales, the
    scales of every 7th channel are set to zero as well."""
    import synth
    bits = inp["q"]  # [B, H_q, d] storage bits
    if dtype == "bf16":
        q = (bits.astype(np.uint32) << 16).view(np.float32).copy()
    elif dtype == "f16":
        q = bits.view(np.float16).astype(np.float32)
    else:
        q = np.array(bits, dtype=np.float32)
    q[:, 0, :] = 0.0
    q[:, 1, :] = 1e-3 * np.sign(q[:, 1, :])
    q[:, 1, 5] = 8.0
    q[:, 2, :] = q[:, 2, :] * 1e-20
    q[:, 3, :] = q[:, 3, :] * 40.0
    inp["q"] = synth.to_storage(q, dtype)
    if "k_scales" in inp:
        ks = inp["k_scales"].copy()
        ks[:, ::7] = 0.0
        inp["k_scales"] = ks
