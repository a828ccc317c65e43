"""Pins for the oracle (CPU only).

The oracle is checked against what the pages and the mathematics fix, never against itself:
  * Conv3d == flattened dot product, the check on the "Qwen2.5VL-Vision Encode-PatchEmbed"
    page, both in fp64 (to rounding) and in fp32 (the page's printed difference magnitude);
  * the library special case: torch's float64 Conv3d on CPU over the completed volume;
  * the textbook reduction P = 1, Tp = 1 (a per-pixel matrix product);
  * brute force on tiny shapes with slice-based patch extraction, and hand-computed values;
  * linearity in the input and in the weight, and the exact bias shift;
  * the duplicated frame: out = x . (W[:, :, 0] + W[:, :, 1]) (the per-temporal-slice sum of
    the Conv3d -> Conv2d decomposition on the "Optimize VLM PatchEmbed" page);
  * integer inputs give exactly the integer product (that page's R1 == R2 check);
  * row order against the position ids printed on the "Qwen2.5VL语言模型" page and the 2x2
    concatenation of the PatchMerger ("freechatgpt/mytransformer" section 3.2);
  * the shape facts printed on the mytransformer and "patch详解" pages;
  * the PatchMerger front end: LayerNorm against hand values, torch's float64 layer_norm and its
    invariants; the 2x2 concatenation against raster rows gathered by window.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def f64(t):
    return t.detach().to(torch.float64).numpy()


def torch_conv_rows(frames, F, w, b, t, h, wgrid, Tp=2):
    """Library Conv3d (torch, float64, CPU) over one item's completed volume, rows raster."""
    C = frames.shape[1]
    vol = frames.to(torch.float64)  # [F, C, H, W]
    idx = [min(tau, F - 1) for tau in range(t * Tp)]
    vol = vol[idx].permute(1, 0, 2, 3).unsqueeze(0)  # [1, C, T, H, W]
    P = w.shape[-1]
    out = torch.nn.functional.conv3d(vol, w.to(torch.float64),
                                     b.to(torch.float64) if b is not None else None,
                                     stride=(Tp, P, P))
    return out[0].permute(1, 2, 3, 0).reshape(-1, w.shape[0]).numpy()


# ---------------------------------------------------------------------------------------------
# Conv3d == flattened dot product (page 1)
# ---------------------------------------------------------------------------------------------

def test_conv_equals_flattened_dot_fp64(golden):
    g = golden("p1_conv_vs_matmul.txt")
    wl = workloads.WORKLOADS[1]
    x, w, _ = workloads.generate(wl)
    assert tuple(x.shape) == (g["n_patches"], g["k"])
    assert tuple(w.shape) == tuple(g["weight_shape"])
    out = oracle.forward(x, w, None, grid=wl.grid, kind="patches")
    assert out.shape == tuple(g["out_shape"])
    ref = f64(x).reshape(g["n_patches"], -1) @ f64(w).reshape(g["embed"], -1).T
    assert np.max(np.abs(out - ref)) < 1e-12


def test_fp32_evaluation_within_page_magnitude(golden):
    """The page's fp32 conv-vs-matmul gap is ~4e-6 max, ~0.36 summed over 1.31M outputs. An fp32
    evaluation must sit at that order from the fp64 oracle."""
    g = golden("p1_conv_vs_matmul.txt")
    wl = workloads.WORKLOADS[1]
    x, w, _ = workloads.generate(wl)
    out = oracle.forward(x, w, None, grid=wl.grid, kind="patches")
    f32 = (x.reshape(1024, -1) @ w.reshape(1280, -1).T).double().numpy()
    d = np.abs(out - f32)
    assert g["max_abs_diff_f32"] / 10 < d.max() < g["max_abs_diff_f32"] * 5
    assert g["sum_abs_diff_f32"] / 10 < d.sum() < g["sum_abs_diff_f32"] * 5


def test_output_magnitude_closed_form(golden):
    """Var(out) = K * Var(x) * Var(w) = K * 1 * 1/(3K) = 1/3 for N(0,1) inputs and
    U(+-1/sqrt(K)) weights; the page's printed entries have that scale."""
    g = golden("p1_conv_vs_matmul.txt")
    wl = workloads.WORKLOADS[1]
    x, w, _ = workloads.generate(wl)
    out = oracle.forward(x, w, None, grid=wl.grid, kind="patches")
    assert abs(out.std() - 1 / math.sqrt(3)) < 0.01 * (1 / math.sqrt(3))
    assert abs(out.mean()) < 0.01
    # the printed excerpt's largest entry is ~4 sigma; 1.31M draws reach beyond it
    assert np.abs(out).max() > g["max_printed_abs"]


# ---------------------------------------------------------------------------------------------
# library special case: torch Conv3d in float64
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("P,E,F,t,h,w,bias", [
    (14, 32, 1, 1, 3, 5, True),    # single image: duplicated frame
    (14, 16, 4, 2, 2, 3, False),   # video, even frame count
    (14, 16, 3, 2, 2, 2, True),    # odd frame count: last temporal patch repeats frame 2
    (16, 24, 2, 1, 2, 2, True),    # patch 16
])
def test_frames_match_torch_conv3d_f64(P, E, F, t, h, w, bias):
    C = 3
    x = workloads.random_tensor((F, C, h * P, w * P), seed=10 + P + F)
    wt = workloads.random_tensor((E, C, 2, P, P), seed=20 + E, dist="uniform", bound=0.05)
    b = workloads.random_tensor((E,), seed=30, dist="uniform", bound=0.05) if bias else None
    out = oracle.forward(x, wt, b, grid=[[t, h, w]], frames=[F], kind="frames", order="raster")
    ref = torch_conv_rows(x, F, wt, b, t, h, w)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_patch_rows_match_torch_conv3d_f64():
    N, P, E = 37, 14, 40
    x = workloads.random_tensor((N, 3 * 2 * P * P), seed=3)
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=4, dist="uniform", bound=0.05)
    b = workloads.random_tensor((E,), seed=5, dist="uniform", bound=0.05)
    out = oracle.forward(x, wt, b, grid=[[1, 1, N]], kind="patches")
    ref = torch.nn.functional.conv3d(x.double().view(-1, 3, 2, P, P), wt.double(), b.double(),
                                     stride=(2, P, P)).view(-1, E).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_multi_item_concatenation():
    """Items' rows are concatenated in item order; each item equals its own convolution."""
    P, E = 14, 16
    items = [((1, 2, 4), 1), ((2, 2, 2), 4), ((1, 4, 2), 1)]
    xs = [workloads.random_tensor((F, 3, h * P, w * P), seed=40 + i)
          for i, ((t, h, w), F) in enumerate(items)]
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=50, dist="uniform", bound=0.05)
    x = torch.cat([a.reshape(-1) for a in xs])
    out = oracle.forward(x, wt, None, grid=[g for g, _ in items], frames=[F for _, F in items],
                         kind="frames", order="raster")
    ref = np.concatenate([torch_conv_rows(xs[i], F, wt, None, *g)
                          for i, (g, F) in enumerate(items)])
    assert np.max(np.abs(out - ref)) < 1e-12


# ---------------------------------------------------------------------------------------------
# textbook reduction, brute force, hand values
# ---------------------------------------------------------------------------------------------

def test_reduces_to_per_pixel_matmul_when_P1_Tp1():
    C, E, H, W = 3, 7, 4, 5
    x = workloads.random_tensor((1, C, H, W), seed=60)
    wt = workloads.random_tensor((E, C, 1, 1, 1), seed=61)
    out = oracle.forward(x, wt, None, grid=[[1, H, W]], frames=[1], kind="frames")
    pix = f64(x)[0].reshape(C, H * W).T            # [H*W, C], raster pixels
    ref = pix @ f64(wt).reshape(E, C).T
    assert np.max(np.abs(out - ref)) < 1e-13


@pytest.mark.parametrize("C,Tp,P,E,F,t,h,w", [
    (1, 1, 1, 1, 1, 1, 1, 1), (1, 2, 2, 2, 2, 1, 2, 3), (3, 2, 3, 5, 3, 2, 2, 2),
    (3, 1, 2, 2, 2, 2, 3, 1), (3, 2, 1, 5, 1, 1, 4, 4),
])
def test_brute_force_tiny(C, Tp, P, E, F, t, h, w):
    x = workloads.random_tensor((F, C, h * P, w * P), seed=70 + F * 7 + P)
    wt = workloads.random_tensor((E, C, Tp, P, P), seed=80 + E)
    b = workloads.random_tensor((E,), seed=90)
    out = oracle.forward(x, wt, b, grid=[[t, h, w]], frames=[F], kind="frames")
    X, Wn, Bn = f64(x), f64(wt), f64(b)
    r = 0
    for to in range(t):
        frames_used = [min(to * Tp + kt, F - 1) for kt in range(Tp)]
        for ho in range(h):
            for wo in range(w):
                patch = X[frames_used][:, :, ho * P:(ho + 1) * P, wo * P:(wo + 1) * P]  # [Tp,C,P,P]
                patch = patch.transpose(1, 0, 2, 3)                                     # [C,Tp,P,P]
                want = (Wn * patch[None]).sum(axis=(1, 2, 3, 4)) + Bn
                assert np.max(np.abs(out[r] - want)) < 1e-12
                r += 1


def test_hand_values_all_ones():
    """x = 1, W = 1 => every output is K + b."""
    P, E = 14, 4
    x = torch.ones((1, 3, 2 * P, 4 * P))
    wt = torch.ones((E, 3, 2, P, P))
    b = torch.tensor([0.0, 1.0, -2.0, 0.5])
    out = oracle.forward(x, wt, b, grid=[[1, 2, 4]], frames=[1], kind="frames", order="merge")
    K = 3 * 2 * P * P
    assert out.shape == (8, E)
    assert np.all(out == K + b.numpy()[None, :])


def test_hand_values_one_hot():
    """W[e] one-hot at (c, kt, ky, kx) picks exactly that volume element of each patch."""
    P, E = 2, 3
    x = torch.arange(2 * 3 * 4 * 6, dtype=torch.float32).reshape(2, 3, 4, 6)
    wt = torch.zeros((E, 3, 2, P, P))
    wt[0, 0, 0, 0, 0] = 1
    wt[1, 2, 1, 1, 1] = 1
    wt[2, 1, 1, 0, 1] = -1
    out = oracle.forward(x, wt, None, grid=[[1, 2, 3]], frames=[2], kind="frames")
    X = x.numpy()
    r = 0
    for ho in range(2):
        for wo in range(3):
            assert out[r, 0] == X[0, 0, ho * P, wo * P]
            assert out[r, 1] == X[1, 2, ho * P + 1, wo * P + 1]
            assert out[r, 2] == -X[1, 1, ho * P, wo * P + 1]
            r += 1


# ---------------------------------------------------------------------------------------------
# linearity, bias, duplicated frame, integers
# ---------------------------------------------------------------------------------------------

def test_linearity_and_bias_shift():
    P, E, F, t, h, w = 14, 24, 2, 1, 2, 4
    kw = dict(grid=[[t, h, w]], frames=[F], kind="frames", order="merge")
    x = workloads.random_tensor((F, 3, h * P, w * P), seed=100).double()
    y = workloads.random_tensor((F, 3, h * P, w * P), seed=101).double()
    W = workloads.random_tensor((E, 3, 2, P, P), seed=102).double()
    V = workloads.random_tensor((E, 3, 2, P, P), seed=103).double()
    b = workloads.random_tensor((E,), seed=104).double()
    a, c = 0.75, -1.5
    fx, fy = oracle.forward(x, W, **kw), oracle.forward(y, W, **kw)
    assert np.max(np.abs(oracle.forward(a * x + c * y, W, **kw) - (a * fx + c * fy))) < 1e-11
    fv = oracle.forward(x, V, **kw)
    assert np.max(np.abs(oracle.forward(x, a * W + c * V, **kw) - (a * fx + c * fv))) < 1e-11
    assert np.array_equal(oracle.forward(x, W, b, **kw) - fx,
                          np.broadcast_to(b.numpy(), fx.shape)) or \
        np.max(np.abs(oracle.forward(x, W, b, **kw) - fx - b.numpy())) < 1e-13


def test_addend_follows_output_rows():
    """The fused add ("Optimize VLM PatchEmbed", the Model forward: hidden_states + pos_embeds):
    with bias 0, adding the output for x2 to the output for x1 must give the output for x1 + x2
    (linearity), in merge order over items of different sizes, so an addend taken in any other row
    order fails; and a sampled-rows call takes the addend's rows at those positions."""
    g = torch.Generator().manual_seed(14)
    P, E = 2, 6
    grid, frames = [[1, 4, 6], [2, 2, 4]], [1, 4]
    n_x = 1 * 3 * 8 * 12 + 4 * 3 * 4 * 8
    x1 = torch.randn(n_x, generator=g, dtype=torch.float64)
    x2 = torch.randn(n_x, generator=g, dtype=torch.float64)
    w = torch.randn(E, 3, 2, P, P, generator=g, dtype=torch.float64)
    kw = dict(grid=grid, frames=frames, order="merge")
    a2 = oracle.forward(x2, w, **kw)
    got = oracle.forward(x1, w, addend=a2, **kw)
    want = oracle.forward(x1 + x2, w, **kw)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())
    rows = [0, 5, 17, 23, 24, 39]
    sub = oracle.forward(x1, w, addend=a2, rows=rows, **kw)
    assert np.array_equal(sub, got[rows])


def test_duplicated_frame_equals_temporal_weight_sum():
    """A single image frame feeds both temporal slices, so the Conv3d equals a 2-D patch
    product with W[:, :, 0] + W[:, :, 1] (exact in fp64 for bf16 weights)."""
    wl = workloads.WORKLOADS[2]
    x, w, _ = workloads.generate(wl)
    rows = np.arange(0, 1024, 37)
    out = oracle.forward(x, w, None, grid=wl.grid, frames=wl.frames, kind="frames",
                         order="raster", rows=rows)
    X = f64(x)[0]                                          # [3, 224, 896]
    Wf = f64(w)[:, :, 0] + f64(w)[:, :, 1]                 # [E, 3, 14, 14]
    for q, r in enumerate(rows):
        ho, wo = divmod(int(r), 64)
        patch = X[:, ho * 14:(ho + 1) * 14, wo * 14:(wo + 1) * 14]
        want = (Wf * patch[None]).sum(axis=(1, 2, 3))
        assert np.max(np.abs(out[q] - want)) < 1e-12


def test_odd_frame_count_repeats_last_frame():
    """F = 3, Tp = 2 -> t = 2 (rounded up); the second temporal patch sees frame 2 twice."""
    P, E = 14, 8
    x = workloads.random_tensor((3, 3, P, 2 * P), seed=110)
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=111)
    out = oracle.forward(x, wt, None, grid=[[2, 1, 2]], frames=[3], kind="frames")
    X, Wn = f64(x), f64(wt)
    for wo in range(2):
        p2 = X[2][:, :, wo * P:(wo + 1) * P]
        want = ((Wn[:, :, 0] + Wn[:, :, 1]) * p2[None]).sum(axis=(1, 2, 3))
        assert np.max(np.abs(out[2 + wo] - want)) < 1e-12
    with pytest.raises(ValueError):   # t must equal ceil(F / Tp)
        oracle.forward(x, wt, None, grid=[[1, 1, 2]], frames=[3], kind="frames")


def test_integer_inputs_exact():
    """x in {0,1,2}, W in {-2..2}, integer bias: every sum is an integer, equal to the int64
    matrix product exactly (the R1 == R2 check on the "Optimize VLM PatchEmbed" page)."""
    N, P, E = 123, 16, 64
    x = workloads.random_tensor((N, 3 * 2 * P * P), seed=120, dist="int", low=0, high=3)
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=121, dist="int", low=-2, high=3)
    b = workloads.random_tensor((E,), seed=122, dist="int", low=-5, high=6)
    out = oracle.forward(x, wt, b, grid=[[1, 1, N]], kind="patches")
    ref = x.long().numpy() @ wt.long().numpy().reshape(E, -1).T + b.long().numpy()
    assert np.array_equal(out, ref.astype(np.float64))


# ---------------------------------------------------------------------------------------------
# row order and shapes
# ---------------------------------------------------------------------------------------------

def test_merge_order_matches_printed_position_ids(golden):
    g = golden("p3_vision_position_ids.txt")
    t, h, w = g["grid_thw"]
    pos = oracle.row_positions([[t, h, w]], [1], order="merge", m=2)
    assert pos.shape[0] == t * h * w == 4 * g["n_tokens"]
    # every 4 consecutive rows form one merged token; token j sits at merged (hm, wm)
    hm = pos[:, 2].reshape(-1, 4) // 2
    wm = pos[:, 3].reshape(-1, 4) // 2
    assert np.all(hm == hm[:, :1]) and np.all(wm == wm[:, :1])
    h_ids = hm[:, 0] + g["offset"]
    w_ids = wm[:, 0] + g["offset"]
    t_ids = pos[:, 1].reshape(-1, 4)[:, 0] + g["offset"]
    mh, mw = g["merged_grid"][1], g["merged_grid"][2]
    assert np.all(t_ids == g["t_first"]) and g["t_first"] == g["t_last"]
    # printed pattern: h = 15 (x32), 16 (x32), ..., 22; w = 15..46 repeated
    assert np.array_equal(h_ids, np.repeat(np.arange(g["h_first"], g["h_last"] + 1), mw))
    assert np.array_equal(w_ids, np.tile(np.arange(g["w_first"], g["w_last"] + 1), mh))


def test_merge_windows_are_2x2_adjacent_patches():
    pos = oracle.row_positions([[2, 4, 6], [1, 2, 2]], [4, 1], order="merge", m=2)
    for j in range(pos.shape[0] // 4):
        blk = pos[4 * j:4 * j + 4]
        assert len(set(blk[:, 0])) == 1 and len(set(blk[:, 1])) == 1
        hs, ws = sorted(set(blk[:, 2])), sorted(set(blk[:, 3]))
        assert len(hs) == 2 and hs[1] == hs[0] + 1 and hs[0] % 2 == 0
        assert len(ws) == 2 and ws[1] == ws[0] + 1 and ws[0] % 2 == 0
    # every patch appears exactly once
    assert len({tuple(p) for p in pos}) == pos.shape[0]


def test_raster_order_is_conv_view_order():
    """Raster rows are the Conv3d output viewed as (-1, E), the pages' `.view(-1, embed_dim)`."""
    pos = oracle.row_positions([[2, 3, 4]], [4], order="raster")
    want = np.array([(0, a, b, c) for a in range(2) for b in range(3) for c in range(4)])
    assert np.array_equal(pos, want)


def test_shape_facts_mytransformer(golden):
    g = golden("p4_shapes.txt")
    assert oracle.num_rows([g["grid_thw"]]) == g["n_patches"]
    pos = oracle.row_positions([g["grid_thw"]], [1], order="merge")
    assert pos.shape[0] // 4 == g["merged_tokens"]


def test_shape_facts_token_table(golden_table):
    for F, H, W, P, Tp, m, patches, tokens in golden_table("p5_token_table.txt"):
        t = -(-F // Tp)
        grid = [[t, H // P, W // P]]
        assert oracle.num_rows(grid) == patches
        pos = oracle.row_positions(grid, [F], order="merge", m=m, P=P, Tp=Tp)
        windows = {(p[0], p[1], p[2] // m, p[3] // m) for p in pos}
        assert len(windows) == tokens


def test_rejects_bad_shapes():
    x = torch.zeros((1, 3, 14, 42))
    w = torch.zeros((4, 3, 2, 14, 14))
    with pytest.raises(ValueError):  # merge order needs even h and w
        oracle.forward(x, w, grid=[[1, 1, 3]], frames=[1], kind="frames", order="merge")
    with pytest.raises(ValueError):
        oracle.num_rows([[0, 2, 2]])


def test_merge_order_within_window_reading():
    """The pages fix the windows (2x2 adjacent patches, raster over the merged grid) but not the
    order of the four patches inside a window. Reading taken: row-major (dh, dw). Checked here
    against an independent formulation: the raster grid reshaped to (t, h/2, 2, w/2, 2) and
    transposed to (t, h/2, w/2, 2, 2)."""
    t, h, w = 2, 4, 6
    pos = oracle.row_positions([[t, h, w]], [4], order="merge", m=2)
    raster_of_row = (pos[:, 1] * h + pos[:, 2]) * w + pos[:, 3]
    want = np.arange(t * h * w).reshape(t, h // 2, 2, w // 2, 2).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(raster_of_row, want.reshape(-1))


@pytest.mark.parametrize("m,grid,F", [(1, (2, 3, 5), 4), (3, (1, 6, 9), 1), (3, (2, 3, 6), 3), (4, (2, 8, 4), 4)])
def test_merge_order_any_window_size(m, grid, F):
    """Window size m other than 2: the same windows-in-raster, row-major-inside reading, against
    the raster grid reshaped to (t, h/m, m, w/m, m) and transposed; m = 1 is raster order itself."""
    t, h, w = grid
    pos = oracle.row_positions([list(grid)], [F], order="merge", m=m)
    raster_of_row = (pos[:, 1] * h + pos[:, 2]) * w + pos[:, 3]
    want = np.arange(t * h * w).reshape(t, h // m, m, w // m, m).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(raster_of_row, want.reshape(-1))
    if m == 1:
        assert np.array_equal(pos, oracle.row_positions([list(grid)], [F], order="raster"))


# ---------------------------------------------------------------------------------------------
# PatchMerger front end: LayerNorm over E, then the 2x2 concatenation ("freechatgpt/mytransformer"
# section 3.2's vision encoder diagram and section 4.1's PatchMerger bullet)
# ---------------------------------------------------------------------------------------------

def test_layer_norm_hand_values():
    """Row (1, 2, 3, 4): mean 5/2 and biased variance 5/4, so with eps = 0 the row normalizes to
    (-3, -1, 1, 3) / sqrt(5). With eps = 3/4 the root is sqrt(2). The affine step scales by gamma
    and shifts by beta per column. (An unbiased variance, a dropped eps or a sign slip each fail
    one of these.)"""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    y = oracle.layer_norm(x, eps=0.0)
    assert np.allclose(y, np.array([[-3.0, -1.0, 1.0, 3.0]]) / math.sqrt(5.0), rtol=0, atol=1e-15)
    y = oracle.layer_norm(x, eps=0.75)
    assert np.allclose(y, np.array([[-1.5, -0.5, 0.5, 1.5]]) / math.sqrt(2.0), rtol=0, atol=1e-15)
    y = oracle.layer_norm(x, gamma=[2.0, 1.0, -1.0, 0.5], beta=[1.0, 0.0, 0.25, -2.0], eps=0.0)
    want = np.array([-3.0 * 2, -1.0, -1.0, 3.0 * 0.5]) / math.sqrt(5.0) + np.array([1.0, 0.0, 0.25, -2.0])
    assert np.allclose(y[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,eps", [(1280, 1e-6), (1024, 1e-5), (1152, 1e-6), (8, 1e-3)])
def test_layer_norm_matches_torch_f64(E, eps):
    """Library routine: torch.nn.functional.layer_norm in float64 on the CPU."""
    g = torch.Generator().manual_seed(E)
    x = torch.randn(37, E, generator=g, dtype=torch.float64) * 0.7 + 0.3
    gam = torch.randn(E, generator=g, dtype=torch.float64)
    bet = torch.randn(E, generator=g, dtype=torch.float64)
    want = torch.nn.functional.layer_norm(x, (E,), gam, bet, eps).numpy()
    got = oracle.layer_norm(x, gam, bet, eps)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_layer_norm_invariants():
    """Each normalized row (gamma 1, beta 0, eps 0) has mean 0 and mean square 1; the result is
    unchanged by x -> a*x + c for a > 0 and negated for a < 0; a constant row gives beta."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 1280)) * 3.0 + 7.0
    y = oracle.layer_norm(x, eps=0.0)
    assert np.abs(y.mean(axis=1)).max() < 1e-12
    assert np.abs((y * y).mean(axis=1) - 1.0).max() < 1e-12
    np.testing.assert_allclose(oracle.layer_norm(2.5 * x - 4.0, eps=0.0), y, rtol=0, atol=1e-11)
    np.testing.assert_allclose(oracle.layer_norm(-0.5 * x + 1.0, eps=0.0), -y, rtol=0, atol=1e-11)
    beta = rng.standard_normal(1280)
    c = np.full((3, 1280), 0.3125)
    assert np.array_equal(oracle.layer_norm(c, rng.standard_normal(1280), beta, 1e-6), np.tile(beta, (3, 1)))


def test_merger_front_concatenates_2x2_neighbours():
    """merger_front on merge-window rows: row j of the [N/4, 4E] result is the LayerNorm of the
    four patches of window j, side by side. Checked against raster rows (the Conv3d view order)
    gathered by window coordinates: window (t, i, j) holds patches (t, 2i + dh, 2j + dw)."""
    gen = torch.Generator().manual_seed(11)
    P, E, t, h, w = 14, 24, 2, 4, 6
    frames = torch.randn(2 * t, 3, h * P, w * P, generator=gen).to(torch.bfloat16)
    wt = (torch.randn(E, 3, 2, P, P, generator=gen) * 0.03).to(torch.bfloat16)
    b = (torch.randn(E, generator=gen) * 0.1).to(torch.bfloat16)
    gam = torch.randn(E, generator=gen, dtype=torch.float64)
    bet = torch.randn(E, generator=gen, dtype=torch.float64)
    raster = oracle.forward(frames, wt, b, grid=[[t, h, w]], frames=[2 * t], order="raster")
    merge = oracle.forward(frames, wt, b, grid=[[t, h, w]], frames=[2 * t], order="merge", m=2)
    got = oracle.merger_front(merge, gam, bet, 1e-6, m=2)
    assert got.shape == (t * h * w // 4, 4 * E)
    ln_r = oracle.layer_norm(raster, gam, bet, 1e-6).reshape(t, h, w, E)
    want = ln_r.reshape(t, h // 2, 2, w // 2, 2, E).transpose(0, 1, 3, 2, 4, 5).reshape(-1, 4 * E)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the merged token count of the mytransformer shape table: [1944, 1280] rows -> 486 tokens
    assert oracle.merger_front(np.ones((1944, 8)) * np.arange(8), m=2).shape == (486, 32)


# ---- the input cast: round to nearest, ties to even, applied once ("Optimize VLM PatchEmbed",
# the Qwen3VLVisionPatchEmbed forward casts its input to the weight dtype). Expected values are
# written out by hand from the formats: bf16 keeps 8 significant bits, so next to 1 its spacing
# is 2^-7 and 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7; fp32 keeps 24.

def _r(v, dt):
    return float(oracle.round_to(np.array([v]), dt)[0])


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_round_to_bf16_hand_values(sign):
    s = sign
    # ties go to the neighbour with an even last bit
    assert _r(s * (1 + 2 ** -8), "bf16") == s * 1.0                      # 1 (even) vs 1 + 2^-7 (odd)
    assert _r(s * (1 + 3 * 2 ** -8), "bf16") == s * (1 + 2 ** -6)        # 1 + 2^-7 (odd) vs 1 + 2^-6 (even)
    assert _r(s * (2 + 2 ** -7), "bf16") == s * 2.0                      # midpoint one binade up
    # off the midpoint by a little: the nearer neighbour, whatever its last bit
    assert _r(s * (1 + 2 ** -8 + 2 ** -30), "bf16") == s * (1 + 2 ** -7)
    assert _r(s * (1 + 2 ** -8 - 2 ** -30), "bf16") == s * 1.0
    assert _r(s * (1 + 3 * 2 ** -8 - 2 ** -30), "bf16") == s * (1 + 2 ** -7)
    # representable values stay
    assert _r(s * (1 + 5 * 2 ** -7), "bf16") == s * (1 + 5 * 2 ** -7)
    # a value given as fp32 rounds exactly once: 1 + 2^-8 + 2^-20 is an fp32 value above the midpoint
    assert _r(np.float32(s * (1 + 2 ** -8 + 2 ** -20)), "bf16") == s * (1 + 2 ** -7)


def test_round_to_bf16_is_one_rounding_not_two():
    # through fp32 first, 1 + 2^-8 + 2^-30 would land on the bf16 midpoint 1 + 2^-8 and tie to 1
    v = np.array([1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -30)])
    assert list(oracle.round_to(v, "bf16")) == [1 + 2 ** -7, -(1 + 2 ** -7)]
    assert list(oracle.round_via_f32(v, "bf16")) == [1.0, -1.0]


def test_round_to_bf16_range_edges():
    big = (2 - 2 ** -7) * 2.0 ** 127                    # the largest finite bf16
    assert _r(big, "bf16") == big
    assert _r((2 - 2 ** -8 - 2 ** -20) * 2.0 ** 127, "bf16") == big   # below the midpoint to 2^128
    assert _r((2 - 2 ** -8) * 2.0 ** 127, "bf16") == math.inf         # midpoint: even is 2^128, overflow
    assert _r(-(2 - 2 ** -8) * 2.0 ** 127, "bf16") == -math.inf
    # subnormals: spacing 2^-133 below 2^-126
    assert _r(2.0 ** -133, "bf16") == 2.0 ** -133
    assert _r(2.0 ** -134, "bf16") == 0.0                             # tie between 0 (even) and 2^-133
    assert _r(3 * 2.0 ** -134, "bf16") == 2.0 ** -132                 # tie between 2^-133 (odd) and 2^-132
    assert _r(1.5 * 2.0 ** -126 + 2.0 ** -134, "bf16") == 1.5 * 2.0 ** -126   # tie at the normal edge -> even
    z = oracle.round_to(np.array([0.0, -0.0, np.inf, -np.inf, np.nan]), "bf16")
    assert z[0] == 0.0 and not np.signbit(z[0]) and z[1] == 0.0 and np.signbit(z[1])
    assert z[2] == np.inf and z[3] == -np.inf and np.isnan(z[4])


def test_round_to_f32_hand_values():
    assert _r(1 + 2 ** -24, "f32") == 1.0                             # tie, 1 is even
    assert _r(1 + 3 * 2 ** -24, "f32") == 1 + 2 ** -22                # tie, 1 + 2^-22 is even
    assert _r(1 + 2 ** -24 + 2 ** -40, "f32") == 1 + 2 ** -23
    assert _r(-(1 + 2 ** -24 + 2 ** -40), "f32") == -(1 + 2 ** -23)
    assert _r(2.0 ** -149, "f32") == 2.0 ** -149                      # smallest fp32 subnormal
    assert _r(2.0 ** -150, "f32") == 0.0
    assert _r((2 - 2 ** -24) * 2.0 ** 127, "f32") == math.inf


def test_round_to_matches_torch_cast_on_fp32_values():
    # special case that reduces to a library routine: for values that are already fp32, torch's
    # fp32 -> bf16 cast (round to nearest even) must agree bit for bit
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(200000, generator=g) * s for s in (1e-38, 1e-3, 1.0, 1e3, 1e37)])
    x = torch.cat([x, torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38])])
    want = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to(x, "bf16")
    assert np.array_equal(got, want)
