/*
 * pe.h -- C ABI of the MI355X (gfx950) vision PatchEmbed library (libpe.so).
 *
 * The operation. The vision PatchEmbed of Qwen2/2.5/3-VL is a Conv3d with C = 3 input
 * channels, E output channels and kernel = stride = (Tp, P, P), Tp = 2. Because the kernel
 * covers a whole patch and stride equals kernel, each patch meets the kernel exactly once, so
 * the convolution is a dot product of the flattened patch with each flattened filter
 * ("Qwen2.5VL-Vision Encode-PatchEmbed", the bullet list on the convolution and its torch
 * check): out[N, E] = patches[N, K] x W[E, K]^T (+ bias), K = C*Tp*P*P (1176 for P = 14,
 * 1536 for P = 16). The pages' module interfaces are construct-once / forward-many: the candle
 * struct's new() and forward() on that page, the Qwen3VLVisionPatchEmbed class and the vision
 * model's forward(hidden_states, grid_thw) on "Optimize VLM PatchEmbed". This header mirrors
 * them with pe_create / pe_forward / pe_destroy.
 *
 * All device pointers are HIP device memory on the device that was current at pe_create.
 * Streams are hipStream_t passed as void* (NULL = the null stream). No call throws; every
 * call returns a pe_status (or a count) and leaves a message for pe_last_error() on failure.
 */
#ifndef PE_H_
#define PE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PE_OK = 0,
    PE_ERR_INVALID_ARG = -1,  /* null pointer, bad enum value, negative count            */
    PE_ERR_SHAPE = -2,        /* grid / frame counts inconsistent with the operation      */
    PE_ERR_UNSUPPORTED = -3,  /* valid request outside what the kernels implement         */
    PE_ERR_HIP = -4,          /* a HIP runtime call failed (message has hipGetErrorString) */
    PE_ERR_OOM = -5           /* device allocation failed in pe_create                    */
} pe_status;

typedef enum { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Output row order for frames input.
 *  RASTER:        rows follow the Conv3d output viewed as (-1, E), i.e. (t, h, w) raster
 *                 order per item (the `.view(-1, embed_dim)` of the pages' PatchEmbed classes).
 *  MERGE_WINDOW:  the rows of each m x m window of neighbouring patches are consecutive, as the
 *                 PatchMerger concatenates them ("freechatgpt/mytransformer" section 3.2);
 *                 windows follow the merged grid (t, h/m, w/m) in raster order (the vision
 *                 position ids on the "Qwen2.5VL语言模型" page); inside a window the patches
 *                 are in row-major (dh, dw) order (the pages leave this open; reading taken).
 *  Pre-flattened patch rows keep their input order whatever this says. */
typedef enum { PE_ORDER_RASTER = 0, PE_ORDER_MERGE_WINDOW = 1 } pe_order;

/* What pe_forward receives.
 *  PATCHES: rows x[N, K] row-major, each row flattened in (c, t, py, px) order, the
 *           processor's pixel_values [N, 1176] (the `view(-1, 3, 2, 14, 14)` on the pages).
 *  FRAMES:  raw frames. Item i is F_i frames of [C, h_i*P, w_i*P] row-major, items back to back
 *           in one buffer. Temporal patch tp of item i reads frames min(tp*Tp + tt, F_i - 1),
 *           tt < Tp: a single image frame fills both temporal slots ("patch详解" section 4.5
 *           rounds 1/2 up to one temporal patch; repeating the frame is the reading taken). */
typedef enum { PE_INPUT_PATCHES = 0, PE_INPUT_FRAMES = 1 } pe_input_kind;

typedef struct {
    int32_t in_channels;          /* C. Only 3 is supported.                                 */
    int32_t temporal_patch_size;  /* Tp. Only 2 is supported.                                */
    int32_t patch_size;           /* P. 14 or 16.                                            */
    int32_t embed_dim;            /* E. Positive multiple of 16, at most 65536.              */
    int32_t spatial_merge_size;   /* m, used by PE_ORDER_MERGE_WINDOW (>= 1; the models: 2).  */
    int32_t weight_dtype;         /* pe_dtype of weight and bias.                            */
    int32_t out_dtype;            /* pe_dtype of the output.                                 */
    int32_t out_order;            /* pe_order, applied to FRAMES input.                      */
    int32_t image_fold;           /* 0: exact (default). 1: APPROXIMATE mode for single-frame   */
                                  /* items, see below. Needs a bf16 weight.                   */
    int32_t stage_images;         /* 0: default. 1: single images gathered through LDS, see   */
                                  /* below (exact; slower on MI355X, kept for comparison).    */
} pe_config;

/* stage_images. With stage_images = 1, frames launches whose items are all single images of one
 * frame size, with bf16 input and weight, P = 14 and the large tiles, stage the tile's pixel rows
 * through LDS (each wave loads whole pixel rows of 32 patches and the waves share them, as the
 * LDS-staged A tiles of a classic GEMM) instead of each wave gathering its own patches' pixels
 * into registers. Same sum in a different k order (fp32 accumulation, so the
 * last bits may differ). On MI355X it measured 3-20 %
 * slower than the default, so it is off unless asked for; pe_forward_plan reports such launches
 * as PE_A_IMAGES_LDS. Other launches are unaffected. */

/* image_fold. An image item repeats its one frame in both temporal slots, so its output is
 * x . (W[:, :, 0] + W[:, :, 1]) over the C*P*P elements of that frame (the per-temporal-slice sum of
 * the Conv3d -> Conv2d decomposition on "Optimize VLM PatchEmbed"). With image_fold = 1, pe_create
 * also packs that folded weight, rounded to bf16 once, and frames launches of single-frame items
 * use it: half the matrix-core work. Approximate: the folded weight's rounding (at most 2^-8 of
 * |W0 + W1| per element) adds up to 2^-8 * sum_k |x_k| |W0_k + W1_k| to each output, beyond the exact
 * path's single output rounding. Video items and patch rows are unaffected (exact). */

typedef struct pe_handle_s *pe_handle;

/*
 * pe_create -- validate the configuration and pre-pack the weight once.
 *   cfg        configuration (read during the call only).
 *   weight     device [E, C, Tp, P, P] row-major in cfg->weight_dtype: the checkpoint's
 *              `visual.patch_embed.proj.weight` (the candle struct flattens and transposes it
 *              once at load; this call re-lays it out once for the matrix cores instead).
 *   bias       device [E] in cfg->weight_dtype, or NULL for no bias (Qwen2/2.5-VL have none,
 *              the Qwen3-VL module has one: "Optimize VLM PatchEmbed").
 *   hip_stream stream the packing runs on; the call synchronizes it before returning, so the
 *              caller may free weight and bias afterwards.
 *   out        receives the handle. The handle owns its packed copy (device memory).
 * Returns PE_OK, PE_ERR_INVALID_ARG (null pointer, bad enum), PE_ERR_UNSUPPORTED (C != 3,
 * Tp != 2, P not 14/16, E not a positive multiple of 16 or above 65536), PE_ERR_OOM or
 * PE_ERR_HIP. On error
 * *out is set to NULL and nothing is leaked.
 */
int pe_create(const pe_config *cfg, const void *weight, const void *bias, void *hip_stream,
              pe_handle *out);

/*
 * pe_forward -- out[N, E] = PatchEmbed(input), asynchronously on hip_stream.
 *   h          handle from pe_create. Immutable: concurrent calls on different streams are safe.
 *   input_kind pe_input_kind (see above).
 *   input      device buffer (PATCHES: [N, K]; FRAMES: the items' frames back to back).
 *   in_dtype   pe_dtype of the input. With a bf16 weight: bf16, or fp32, which is rounded to bf16
 *              (nearest-even) as it is loaded: the cast of the input to the weight dtype that the
 *              Qwen3VLVisionPatchEmbed forward does ("Optimize VLM PatchEmbed"). With an fp32
 *              weight: fp32.
 *   grid_thw   HOST int32 [n_items, 3]: per item (t, h, w) in patches; N = sum t*h*w.
 *   frames     HOST int32 [n_items] frame counts F_i for FRAMES input, or NULL: then an item
 *              with t = 1 is one image frame (F = 1) and an item with t > 1 has F = Tp*t.
 *              Requires ceil(F_i / Tp) == t_i. Ignored for PATCHES.
 *   n_items    number of items, at least 1 (0 items, N = 0, is PE_ERR_SHAPE).
 *   out        device [N, E] in the handle's out dtype; rows of item i follow those of i-1.
 * Arithmetic: products of the input and weight values accumulated in fp32 together with the
 * fp32 bias, one round-to-nearest-even cast to the output dtype. Allocates nothing; does not
 * take ownership of input or out, which must stay valid until the stream work completes. One
 * kernel launch covers up to 64 consecutive items (any number of identical ones), images and
 * videos alike (with image_fold, runs of single images and of videos go to separate launches);
 * their frame sizes may differ.
 * Inputs beyond one launch's 4 GiB buffer range are split into several launches: frames at item
 * boundaries, patch rows at any row.
 * Returns PE_OK, PE_ERR_INVALID_ARG, PE_ERR_SHAPE (a non-positive t/h/w, F_i inconsistent
 * with t_i, merge order with h or w not divisible by m, N >= 2^31), PE_ERR_UNSUPPORTED (bf16
 * input on an fp32 weight; one item's frames beyond 4 GiB) or PE_ERR_HIP (launch failure).
 * Validation happens before any launch.
 */
int pe_forward(pe_handle h, int32_t input_kind, const void *input, int32_t in_dtype,
               const int32_t *grid_thw, const int32_t *frames, int32_t n_items, void *out,
               void *hip_stream);

/*
 * pe_forward_add -- out[N, E] = PatchEmbed(input) + addend, asynchronously on hip_stream.
 *   The next step after the PatchEmbed in the Qwen3-VL vision forward adds the interpolated
 *   position embeddings to its output ("Optimize VLM PatchEmbed", the Model forward:
 *   hidden_states + pos_embeds). This call fuses that add into the PatchEmbed epilogue, saving a
 *   separate pass over [N, E].
 *   addend     device [N, E] row-major in the handle's out dtype, rows in the output order (the
 *              order pe_forward writes); read only. May be the same buffer as out.
 *   All other arguments as pe_forward.
 * Arithmetic: the addend value is added in fp32 to the fp32 sum (products and bias), then one
 * round-to-nearest-even cast to the output dtype (the module rounds twice: after the convolution
 * and after the add). Returns as pe_forward, and PE_ERR_INVALID_ARG for a NULL addend.
 */
int pe_forward_add(pe_handle h, int32_t input_kind, const void *input, int32_t in_dtype,
                   const int32_t *grid_thw, const int32_t *frames, int32_t n_items, const void *addend,
                   void *out, void *hip_stream);

/* How a launch reads its A operand (the patches). */
typedef enum {
    PE_A_FRAMES = 0,         /* frames with two temporal slots (videos, or images mixed with videos) */
    PE_A_IMAGES = 1,         /* frames, every item one image frame (both slots the same pixels)    */
    PE_A_PATCH_ROWS = 2,     /* pre-flattened patch rows                                            */
    PE_A_FOLDED_IMAGES = 3,  /* single images against the folded weight (image_fold = 1)            */
    PE_A_IMAGES_LDS = 4      /* single images, bf16 input, P = 14, large tiles: each wave stages its
                                patches' pixel rows through LDS (whole-row loads)                 */
} pe_a_mode;

/* One kernel launch of a pe_forward call, as pe_forward_plan describes it. */
typedef struct {
    char kernel[32];      /* name of the HIP kernel the launch runs, e.g. "pe_fwd32_kernel"          */
    int32_t tile_rows;    /* output rows x columns of one workgroup's tile                          */
    int32_t tile_cols;
    int64_t workgroups;   /* grid size                                                              */
    int64_t row0;         /* first output row of the launch                                         */
    int64_t n_rows;       /* output rows of the launch                                              */
    int64_t in_offset;    /* byte offset of the launch's input within the input buffer              */
    int64_t in_bytes;     /* bytes of input the launch may read                                     */
    int32_t n_items;      /* items of a frames launch (0 for patch rows)                            */
    int32_t a_mode;       /* pe_a_mode                                                              */
} pe_launch_info;

/*
 * pe_forward_plan -- describe the kernel launches pe_forward (or pe_forward_add) would make for
 *   this request, without launching anything and without touching device memory: the split into
 *   launches, and per launch the kernel and tile chosen for it. Host-only; for profiling and for
 *   callers that size their own timing around the launches.
 *   h, input_kind, in_dtype, grid_thw, frames, n_items   as pe_forward (no device pointers needed).
 *   info       host array of max_info entries (may be NULL when max_info is 0); the first
 *              min(count, max_info) launches are written.
 * Returns the number of launches (at least 1), or a negative pe_status: the same request
 * checks and codes as pe_forward, PE_ERR_INVALID_ARG for max_info < 0 or a NULL info with
 * max_info > 0.
 */
int pe_forward_plan(pe_handle h, int32_t input_kind, int32_t in_dtype, const int32_t *grid_thw,
                    const int32_t *frames, int32_t n_items, pe_launch_info *info, int32_t max_info);

/*
 * pe_layernorm -- y[r, :] = (x[r, :] - mean_r) / sqrt(var_r + eps) * gamma + beta, for every row r
 *   of a row-major [n_rows, dim] tensor, asynchronously on hip_stream, on the current device.
 *   The PatchMerger after the vision tower starts with a LayerNorm over E and then concatenates
 *   the 2x2 neighbouring patches into one 4E row ("freechatgpt/mytransformer", the vision
 *   encoder diagram in section 3.2 and the PatchMerger bullet in section 4.1). On rows that
 *   pe_forward wrote in PE_ORDER_MERGE_WINDOW order with m = 2, y viewed as [n_rows / 4, 4 * dim]
 *   is that concatenation, so this call is the whole front end of the merger.
 *   x, y       device [n_rows, dim] in dtype (pe_dtype). y may be x (in place); otherwise the two
 *              must not overlap. 16-byte aligned.
 *   gamma,beta device [dim] in param_dtype (pe_dtype), 16-byte aligned, or NULL for all ones /
 *              all zeros.
 *   eps        finite, >= 0 (the pages give no value; the Python binding defaults to 1e-6). With
 *              eps = 0 a constant row gives NaN, as the formula does.
 *   n_rows     >= 0; 0 is a no-op that returns PE_OK.
 *   dim        a positive multiple of 8, at most 4096.
 * Arithmetic: mean_r and the biased variance var_r = mean((x - mean_r)^2) in fp32 (the pages
 * compute the language model's norms in fp32 for stability, section 3.3; the same is taken here),
 * y in fp32, one round-to-nearest-even cast to dtype. Allocates nothing.
 * Returns PE_OK, PE_ERR_INVALID_ARG (NULL x/y, bad dtype, bad eps, misalignment, partial
 * overlap), PE_ERR_UNSUPPORTED (dim), PE_ERR_SHAPE (byte count overflow) or PE_ERR_HIP.
 */
int pe_layernorm(const void *x, int32_t dtype, const void *gamma, const void *beta, int32_t param_dtype,
                 float eps, int64_t n_rows, int32_t dim, void *y, void *hip_stream);

/* N = sum over items of t*h*w ("freechatgpt/mytransformer" section 3.2: N = t*h*w), or a
 * negative pe_status: PE_ERR_INVALID_ARG for a NULL grid or negative n_items, PE_ERR_SHAPE for a
 * non-positive entry or a sum beyond int64. */
int64_t pe_num_rows(const int32_t *grid_thw, int32_t n_items);

/* Release the handle and its device memory (synchronizes the device first). NULL -> PE_OK. */
int pe_destroy(pe_handle h);

/* Message of the last failed call on this thread ("" if none). Valid until the next call. */
const char *pe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PE_H_ */
