// pe_plan.h -- the launch plan of pe_forward / pe_forward_add: validation of the request's grid,
// the grouping of items into kernel launches, the split at one launch's 4 GiB buffer range, and
// the choice of kernel and tile for each launch. Host-only code with no HIP header, so it also
// builds with a plain host compiler and runs under the address and undefined-behaviour
// sanitizers without a GPU. The kernel argument struct lives here because the plan fills it.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace pe {

constexpr int kMaxItems = 64;  // items per launch (the item table travels in the kernel arguments)
// bytes one launch may address from its input pointer (32-bit buffer offsets)
constexpr uint64_t kMaxLaunchBytes = 0xFFFFFFF0ull;

// One item (image or video) of a frames launch. Offsets are in input elements relative to the
// launch's input pointer; rows are relative to the launch's first output row.
struct Item {
    int32_t row0;     // first output row of the item
    int32_t t, h, w;  // patch grid
    int32_t F;        // frame count
    uint32_t x_off;   // element offset of the item's first frame
};

struct FwdArgs {
    const void *in;      // launch input base
    const void *wpk;     // packed weight
    const float *bias;   // fp32 [E] or null
    void *out;           // launch output base (row 0 of the launch)
    const void *addend;  // fused add: [rows, E] in the output dtype at the launch's rows, or null
    uint32_t in_bytes;   // bytes addressable from `in` (buffer range; loads beyond read 0)
    int32_t n_rows;      // output rows in this launch
    int32_t E;
    int32_t kind;        // 0 patch rows, 1 frames
    int32_t order;       // 0 raster, 1 merge window
    int32_t m;           // merge size
    int32_t n_items;
    int32_t tiles_m, tiles_n;
    int32_t colmajor;      // tile order within an XCD's run: 1 = column tiles outermost
    int32_t img;           // 1: frames launch whose items are all single images (F = 1)
    int32_t fold;          // 1: such a launch reads the folded weight (kAFold)
    int32_t mixg;          // 1: frames launch whose items differ in frame size (h, w)
    int32_t tiles;         // TileShape::id of the kernel and tile the plan chose
    int32_t staged;        // 1: single images whose pixel rows the kernel stages through LDS
                           //    (bf16 P = 14 large tiles; reads the grouped weight kWeightGrouped)
    uint32_t plane, rstr;  // channel and pixel-row strides (elements) when every item has one frame size
    // every item of the launch the same (t, h, w, F): item of a row by division, no table lookup
    int32_t uni;
    int32_t u_rows;        // rows per item (t*h*w)
    uint32_t u_elems;      // input elements per item
    Item items[kMaxItems];
};

// The forward kernels and their workgroup tiles (output rows x columns).
enum TileId {
    kTileLarge256 = 0,  // bf16 pe_fwd32_kernel, 256 x 256 (8 waves of 32 x 256)
    kTileLarge128 = 1,  // bf16 pe_fwd32_kernel, 256 x 128
    kTileSplitK = 2,    // bf16 pe_fwd32_sk_kernel, 32 x 160 (E % 160 == 0) or 32 x 128
    kTileF32 = 3        // fp32 weight: pe_fwd16_kernel, 32 x 160 (E % 160 == 0) or 32 x 128
};
struct TileShape {
    int id;      // TileId
    int bm, bn;  // workgroup tile
};
const char *kernel_name(int tile_id);

// Packed weights a handle holds (pe_create packs each once).
enum WeightMap { kWeightFrames = 0, kWeightRows = 1, kWeightFold = 2, kWeightGrouped = 3 };

struct PlanRequest {
    int P, E, m;           // patch size, embed dim, merge size
    int weight_esz;        // bytes per weight element (2 bf16, 4 fp32)
    int in_esz, out_esz;   // bytes per input / output element
    int merge;             // frames rows in merge-window order
    int image_fold;        // approximate fold of single-frame items (bf16 weight)
    int stage_images;      // opt-in LDS-staged gather of single images (bf16, P = 14, large tiles)
    int num_cus;           // compute units of the device (0: assume 256)
    int input_kind;        // 0 patch rows, 1 frames (pe_input_kind)
    const int32_t *grid_thw;
    const int32_t *frames;
    int32_t n_items;
};

struct Launch {
    FwdArgs a;          // kernel arguments; the pointers are bound per call (null here)
    uint64_t in_off;    // byte offset of the launch's input in the caller's input buffer
    int64_t row0;       // first output row (the output and addend offsets follow from it)
    int weight_map;     // WeightMap of the packed weight the launch reads
    TileShape tile;
    int64_t workgroups;
};

// Validate the grid and plan the launches. Returns 0 (PE_OK) with the launches in order, or a
// negative pe_status (PE_ERR_INVALID_ARG, PE_ERR_SHAPE, PE_ERR_UNSUPPORTED) with a message in err
// and no launches. n_items == 0 (N = 0) is PE_ERR_SHAPE.
int plan_forward(const PlanRequest &r, std::vector<Launch> &out, std::string &err);

// Tile for a launch of n_rows output rows (see pe_plan.cpp for the cost model).
TileShape choose_tiles(int64_t n_rows, int E, int weight_esz, int num_cus);

}  // namespace pe
