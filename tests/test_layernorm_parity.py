"""GPU parity of the PatchMerger front end (pe_layernorm through the C ABI) against the fp64 oracle.

Tolerances, from the kernel's arithmetic (fp32 statistics, fp32 result, one cast):
  * bf16 output: |err| <= 1e-3 + 1e-2 * |ref| (the final round-to-nearest-even dominates);
  * fp32 output: |err| <= 64u * (|gamma| * rstd * mean|x| + |gamma * xhat| + |beta|), u = 2^-24:
    the row sum is a lane-serial sum of at most 40 values and a 5-6 level tree, so the mean is
    off by at most ~46u * mean|x|; the centred value carries that error times rstd * |gamma|, and
    the product and the affine step add a few u of the result;
  * after a bf16 PatchEmbed, an element whose PatchEmbed value rounded to the other bf16
    neighbour (fp32 vs fp64 sums near a rounding midpoint) moves by one bf16 ulp of that value,
    so |gamma| * rstd * ulp(pe) is added to the bf16 bound there.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def pe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vlm_vision_patch_amd
    return vlm_vision_patch_amd


def say(msg):
    print("[case] " + msg, flush=True)


def gen_rows(seed, n, dim, dtype, scale=1.0, offset=0.0, kind="normal"):
    g = torch.Generator().manual_seed(seed)
    if kind == "constant":
        v = torch.full((n, 1), 0.75) * torch.arange(1, n + 1).reshape(n, 1) / n
        x = v.expand(n, dim).clone()
    else:
        x = torch.randn(n, dim, generator=g) * scale + offset
    return x.to(dtype)


def gen_params(seed, dim, dtype):
    g = torch.Generator().manual_seed(seed + 1000)
    gam = (1.0 + 0.5 * torch.randn(dim, generator=g)).to(dtype)
    bet = (0.5 * torch.randn(dim, generator=g)).to(dtype)
    return gam, bet


def bound(x64, gam, bet, eps, out_dtype, ref):
    if out_dtype == torch.bfloat16:
        return 1e-3 + 1e-2 * np.abs(ref)
    dim = x64.shape[-1]
    mean = x64.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x64 - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    g = np.abs(oracle._f64(gam)) if gam is not None else np.ones(dim)
    b = np.abs(oracle._f64(bet)) if bet is not None else np.zeros(dim)
    xhat = (x64 - mean) * rstd
    return 64 * U32 * (g * rstd * np.abs(x64).mean(axis=1, keepdims=True) + g * np.abs(xhat) + b) + 1e-30


def check(got, ref, tol, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside the bound (max err %.3g, max err/bound %.3g)" % (
        what, bad.sum(), bad.size, err.max(), (err / tol).max())
    return err.max()


CASES = {
    # name: (rows, dim, x dtype, param dtype or None, eps, extra)
    "e1280_bf16_ragged_rows": (1001, 1280, torch.bfloat16, torch.bfloat16, 1e-6, {}),
    "e1024_bf16_f32_params": (777, 1024, torch.bfloat16, torch.float32, 1e-6, {}),
    "e1152_f32": (513, 1152, torch.float32, torch.float32, 1e-6, {}),
    "e1152_bf16_half_lanes_idle": (250, 1152, torch.bfloat16, torch.bfloat16, 1e-5, {}),
    "e1280_f32_bf16_params": (333, 1280, torch.float32, torch.bfloat16, 1e-6, {}),
    "e4096_bf16_64_lanes": (130, 4096, torch.bfloat16, torch.bfloat16, 1e-6, {}),
    "e4096_f32_64_lanes": (66, 4096, torch.float32, torch.float32, 1e-6, {}),
    "e2056_bf16_64_lanes_ragged": (99, 2056, torch.bfloat16, torch.float32, 1e-6, {}),
    "e8_bf16_one_chunk": (300, 8, torch.bfloat16, torch.bfloat16, 1e-3, {}),
    "e16_f32": (47, 16, torch.float32, torch.float32, 1e-6, {}),
    "one_row": (1, 1280, torch.bfloat16, torch.bfloat16, 1e-6, {}),
    "no_affine": (64, 1280, torch.bfloat16, None, 1e-6, {}),
    "in_place_bf16": (200, 1280, torch.bfloat16, torch.bfloat16, 1e-6, {"inplace": True}),
    "in_place_f32": (200, 1024, torch.float32, torch.float32, 1e-6, {"inplace": True}),
    "offset_rows_f32": (128, 1280, torch.float32, torch.float32, 1e-6, {"scale": 1.0, "offset": 100.0}),
    "small_var_rows_f32": (128, 1280, torch.float32, torch.float32, 1e-6, {"scale": 1e-2, "offset": 3.0}),
    "wide_rows_bf16": (128, 1280, torch.bfloat16, torch.bfloat16, 1e-6, {"scale": 40.0, "offset": -5.0}),
    "constant_rows_bf16": (24, 1280, torch.bfloat16, torch.bfloat16, 1e-6, {"kind": "constant"}),
    "constant_rows_f32": (24, 1024, torch.float32, torch.float32, 1e-6, {"kind": "constant"}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layernorm(pe, name):
    n, dim, xdt, pdt, eps, extra = CASES[name]
    say("layernorm %s: rows=%d dim=%d x=%s params=%s eps=%g %s" % (name, n, dim, xdt, pdt, eps, extra))
    seed = zlib.crc32(name.encode()) % 10000
    x = gen_rows(seed, n, dim, xdt, extra.get("scale", 1.0), extra.get("offset", 0.0), extra.get("kind", "normal"))
    gam, bet = gen_params(seed, dim, pdt) if pdt is not None else (None, None)
    xd = x.to(DEV)
    gd = gam.to(DEV) if gam is not None else None
    bd = bet.to(DEV) if bet is not None else None
    y = pe.layer_norm(xd, gd, bd, eps, out=xd if extra.get("inplace") else None)
    torch.cuda.synchronize()
    got = y.cpu().double().numpy()
    ref = oracle.layer_norm(x, gam, bet, eps)
    if extra.get("kind") == "constant":  # constant rows: exactly beta (or 0) on both sides
        want = np.tile(oracle._f64(bet) if bet is not None else np.zeros(dim), (n, 1))
        assert np.array_equal(ref, want)
        assert np.array_equal(got, oracle.round_to(want, "bf16" if xdt == torch.bfloat16 else "f32"))
        return
    e = check(got, ref, bound(oracle._f64(x), gam, bet, eps, xdt, ref), name)
    print("%s: max err %.3g" % (name, e), flush=True)


def test_layernorm_empty_and_errors(pe):
    say("layernorm: zero rows, bad arguments")
    x = torch.empty(0, 1280, dtype=torch.bfloat16, device=DEV)
    assert pe.layer_norm(x).shape == (0, 1280)
    pe.pe_layernorm(0, pe.PE_BF16, None, None, pe.PE_BF16, 1e-6, 0, 1280, 0, None)  # no rows: no-op
    bad = [
        ((pe.PE_BF16, pe.PE_BF16, 1e-6, -1, 1280), pe.PE_ERR_INVALID_ARG),
        ((7, pe.PE_BF16, 1e-6, 0, 1280), pe.PE_ERR_INVALID_ARG),
        ((pe.PE_BF16, pe.PE_BF16, -1.0, 0, 1280), pe.PE_ERR_INVALID_ARG),
        ((pe.PE_BF16, pe.PE_BF16, float("nan"), 0, 1280), pe.PE_ERR_INVALID_ARG),
        ((pe.PE_BF16, pe.PE_BF16, 1e-6, 0, 1284), pe.PE_ERR_UNSUPPORTED),
        ((pe.PE_BF16, pe.PE_BF16, 1e-6, 0, 8192), pe.PE_ERR_UNSUPPORTED),
        ((pe.PE_BF16, pe.PE_BF16, 1e-6, 0, 0), pe.PE_ERR_UNSUPPORTED),
    ]
    for (dt, pdt, eps, n, dim), code in bad:  # rejected before any pointer is used
        with pytest.raises(pe.PEError) as ei:
            pe.pe_layernorm(0, dt, None, None, pdt, eps, n, dim, 0, None)
        assert ei.value.code == code, (dt, pdt, eps, n, dim, ei.value)
    buf = torch.zeros(4, 1280, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pe.PEError) as ei:  # NULL y with rows to write
        pe.pe_layernorm(buf.data_ptr(), pe.PE_BF16, None, None, pe.PE_BF16, 1e-6, 4, 1280, 0, None)
    assert ei.value.code == pe.PE_ERR_INVALID_ARG
    with pytest.raises(pe.PEError) as ei:  # misaligned y
        pe.pe_layernorm(buf.data_ptr(), pe.PE_BF16, None, None, pe.PE_BF16, 1e-6, 1, 1280, buf.data_ptr() + 2, None)
    assert ei.value.code == pe.PE_ERR_INVALID_ARG
    with pytest.raises(pe.PEError) as ei:  # y overlapping x one row on
        pe.pe_layernorm(buf.data_ptr(), pe.PE_BF16, None, None, pe.PE_BF16, 1e-6, 2, 1280,
                        buf.data_ptr() + 2560, None)
    assert ei.value.code == pe.PE_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf).item() == 0  # nothing was written


def test_layernorm_full_size_sampled(pe):
    """The [331776, 1280] bf16 rows of the 64 x 1008^2 batch (the size the benchmark times), seeded
    N(0, 0.6) data; sampled rows (block edges, the last rows, a random sample) against the oracle."""
    n, dim = 331776, 1280
    say("layernorm full size: rows=%d dim=%d bf16" % (n, dim))
    g = torch.Generator().manual_seed(77)
    x = (torch.randn(n, dim, generator=g) * 0.6).to(torch.bfloat16)
    gam, bet = gen_params(77, dim, torch.bfloat16)
    y = pe.layer_norm(x.to(DEV), gam.to(DEV), bet.to(DEV), 1e-6)
    rng = np.random.default_rng(77)
    rows = sorted(set(rng.choice(n, 2000, replace=False).tolist()) | {0, 1, 7, 8, n - 9, n - 8, n - 1})
    ridx = torch.as_tensor(rows)
    got = y[ridx.to(DEV)].cpu().double().numpy()
    ref = oracle.layer_norm(x[ridx], gam, bet, 1e-6)
    check(got, ref, 1e-3 + 1e-2 * np.abs(ref), "full size")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_merger_front_after_patch_embed(pe, out_dtype):
    """PatchEmbed (frames, merge-window order) -> pe_layernorm -> view [N/4, 4E], against the
    oracle's PatchEmbed rounded to the output dtype -> merger_front. Two items, one a video."""
    say("merger front after PatchEmbed: out=%s" % out_dtype)
    g = torch.Generator().manual_seed(21)
    P, E = 14, 1280
    grid, frames = [[1, 16, 20], [2, 8, 12]], [1, 4]
    x = torch.randn(1 * 3 * 16 * P * 20 * P + 4 * 3 * 8 * P * 12 * P, generator=g).to(torch.bfloat16)
    w = (torch.rand(E, 3, 2, P, P, generator=g) * 2 - 1).mul(1176 ** -0.5).to(torch.bfloat16)
    b = (torch.rand(E, generator=g) * 2 - 1).mul(1176 ** -0.5).to(torch.bfloat16)
    gam, bet = gen_params(21, E, torch.bfloat16)
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge", out_dtype=out_dtype)
    rows = mod(x.to(DEV), grid, frames)
    merged = pe.layer_norm(rows, gam.to(DEV), bet.to(DEV), 1e-6, out=rows).view(-1, 4 * E)
    torch.cuda.synchronize()
    got = merged.cpu().double().numpy()
    mod.close()
    pe_ref = oracle.forward(x, w, b, grid=grid, frames=frames, order="merge", m=2)
    pe_ref = oracle.round_via_f32(pe_ref, "bf16" if out_dtype == torch.bfloat16 else "f32")
    ref = oracle.merger_front(pe_ref, gam, bet, 1e-6, m=2)
    assert got.shape == ref.shape == (pe_ref.shape[0] // 4, 4 * E)
    mean = pe_ref.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((pe_ref - mean) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    gabs = np.abs(oracle._f64(gam))
    if out_dtype == torch.bfloat16:
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(pe_ref), 1e-30))) - 7)
        tol = 1e-3 + 1e-2 * np.abs(ref) + (gabs * rstd * ulp).reshape(ref.shape)
    else:  # fp32 PatchEmbed within 5e-4 of the exact value (its parity bound), carried by rstd
        tol = bound(pe_ref, gam, bet, 1e-6, torch.float32, oracle.layer_norm(pe_ref, gam, bet, 1e-6))
        tol = tol.reshape(ref.shape) + (gabs * rstd * 5e-4).reshape(ref.shape)
    e = check(got, ref, tol, "merger front %s" % out_dtype)
    print("merger front %s: max err %.3g" % (out_dtype, e), flush=True)
