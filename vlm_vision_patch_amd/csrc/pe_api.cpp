// pe_api.cpp -- the C ABI of include/pe.h: validation, the weight pre-pack at create, the
// launch plan of pe_forward / pe_forward_add (item tables, launch splitting) and pe_layernorm's
// checks. No allocation after pe_create.
#include "pe.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include <string>
#include <vector>

#include "pe_internal.h"
#include "pe_plan.h"

struct pe_handle_s {
    pe_config cfg;
    int device;
    int num_cus;    // compute units of the device (tile-size choice)
    int steps;
    void *wpk;      // packed weight for frames, steps * packed_cols(E) * 64 bytes
    void *wpk_rows; // bf16: the same weight packed for patch rows (inside wpk's allocation); fp32: wpk
    void *wpk_fold; // bf16 with image_fold: W[:, :, 0] + W[:, :, 1] in the fold map (inside wpk's allocation)
    void *wpk_grp;  // bf16, P = 14 with stage_images: the frames pack in the grouped order, for
                    // single images staged through LDS (inside wpk's allocation)
    float *bias32;  // fp32 bias or null
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(PE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int esize(int32_t dt) { return dt == PE_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == PE_F32 || dt == PE_BF16; }

// Keeps the caller's current device; switches to the handle's device for the call.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = err == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (switched) (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" {

const char *pe_last_error(void) { return g_err.c_str(); }

int64_t pe_num_rows(const int32_t *grid_thw, int32_t n_items) {
    if (n_items < 0) return fail(PE_ERR_INVALID_ARG, "n_items must be >= 0 (got %d)", n_items);
    if (n_items == 0) return 0;
    if (!grid_thw) return fail(PE_ERR_INVALID_ARG, "grid_thw is NULL");
    int64_t n = 0;
    for (int i = 0; i < n_items; ++i) {
        const int32_t t = grid_thw[3 * i], h = grid_thw[3 * i + 1], w = grid_thw[3 * i + 2];
        if (t <= 0 || h <= 0 || w <= 0)
            return fail(PE_ERR_SHAPE, "item %d: grid (%d, %d, %d) has a non-positive entry", i, t, h, w);
        const int64_t th = (int64_t)t * h;  // < 2^62
        if (th > (INT64_MAX - n) / w)
            return fail(PE_ERR_SHAPE, "item %d: grid (%d, %d, %d): the row count overflows", i, t, h, w);
        n += th * w;
    }
    return n;
}

int pe_create(const pe_config *cfg, const void *weight, const void *bias, void *hip_stream,
              pe_handle *out) {
    if (!out) return fail(PE_ERR_INVALID_ARG, "out (handle pointer) is NULL");
    *out = nullptr;
    if (!cfg) return fail(PE_ERR_INVALID_ARG, "cfg is NULL");
    if (!weight) return fail(PE_ERR_INVALID_ARG, "weight is NULL");
    if (!dtype_ok(cfg->weight_dtype) || !dtype_ok(cfg->out_dtype))
        return fail(PE_ERR_INVALID_ARG, "bad dtype (weight %d, out %d)", cfg->weight_dtype, cfg->out_dtype);
    if (cfg->out_order != PE_ORDER_RASTER && cfg->out_order != PE_ORDER_MERGE_WINDOW)
        return fail(PE_ERR_INVALID_ARG, "bad out_order %d", cfg->out_order);
    if (cfg->out_order == PE_ORDER_MERGE_WINDOW && cfg->spatial_merge_size < 1)
        return fail(PE_ERR_INVALID_ARG, "spatial_merge_size must be >= 1 (got %d)", cfg->spatial_merge_size);
    if (cfg->in_channels != pe::kC)
        return fail(PE_ERR_UNSUPPORTED, "in_channels %d: only 3 is supported", cfg->in_channels);
    if (cfg->temporal_patch_size != pe::kTp)
        return fail(PE_ERR_UNSUPPORTED, "temporal_patch_size %d: only 2 is supported", cfg->temporal_patch_size);
    if (!pe::patch_supported(cfg->patch_size))
        return fail(PE_ERR_UNSUPPORTED, "patch_size %d: only 14 and 16 are supported", cfg->patch_size);
    if (cfg->embed_dim <= 0 || cfg->embed_dim % 16 != 0 || cfg->embed_dim > 65536)
        return fail(PE_ERR_UNSUPPORTED, "embed_dim %d: must be a positive multiple of 16, at most 65536",
                    cfg->embed_dim);
    if (cfg->image_fold != 0 && cfg->image_fold != 1)
        return fail(PE_ERR_INVALID_ARG, "image_fold must be 0 or 1 (got %d)", cfg->image_fold);
    if (cfg->image_fold && cfg->weight_dtype != PE_BF16)
        return fail(PE_ERR_UNSUPPORTED, "image_fold needs a bf16 weight");
    if (cfg->stage_images != 0 && cfg->stage_images != 1)
        return fail(PE_ERR_INVALID_ARG, "stage_images must be 0 or 1 (got %d)", cfg->stage_images);

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int wes = esize(cfg->weight_dtype);
    const int steps = pe::packed_steps(cfg->patch_size, wes);
    const size_t frames_bytes = (size_t)steps * pe::packed_cols(cfg->embed_dim, wes) * 64;
    // bf16 keeps a second pack in the patch-rows order (fp32 uses one map for both inputs)
    const size_t rows_bytes = wes == 2 ? (size_t)pe::rows_steps(cfg->patch_size) * pe::packed_cols(cfg->embed_dim, wes) * 64 : 0;
    // and, with image_fold, a third in the folded map for single-frame items
    const size_t fold_bytes = cfg->image_fold ? (size_t)pe::fold_steps(cfg->patch_size) * pe::packed_cols(cfg->embed_dim, wes) * 64 : 0;
    // and, with stage_images and P = 14, the frames pack again in the grouped order
    const size_t grp_bytes = (cfg->stage_images && wes == 2 && cfg->patch_size == 14) ? frames_bytes : 0;
    const size_t wpk_bytes = frames_bytes + rows_bytes + fold_bytes + grp_bytes;

    pe_handle h = new (std::nothrow) pe_handle_s;
    if (!h) return fail(PE_ERR_OOM, "host allocation failed");
    h->cfg = *cfg;
    h->device = dev;
    h->num_cus = 0;
    if (hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        h->num_cus = 0;  // the tile choice then assumes 256
        (void)hipGetLastError();
    }
    h->steps = steps;
    h->wpk = nullptr;
    h->wpk_rows = nullptr;
    h->wpk_fold = nullptr;
    h->wpk_grp = nullptr;
    h->bias32 = nullptr;
    e = hipMalloc(&h->wpk, wpk_bytes);
    if (e != hipSuccess) {
        delete h;
        (void)hipGetLastError();
        return fail(PE_ERR_OOM, "hipMalloc(%zu) for the packed weight: %s", wpk_bytes, hipGetErrorString(e));
    }
    h->wpk_rows = rows_bytes ? static_cast<char *>(h->wpk) + frames_bytes : h->wpk;
    h->wpk_fold = fold_bytes ? static_cast<char *>(h->wpk) + frames_bytes + rows_bytes : nullptr;
    h->wpk_grp = grp_bytes ? static_cast<char *>(h->wpk) + frames_bytes + rows_bytes + fold_bytes : nullptr;
    if (bias) {
        e = hipMalloc(reinterpret_cast<void **>(&h->bias32), sizeof(float) * cfg->embed_dim);
        if (e != hipSuccess) {
            (void)hipFree(h->wpk);
            delete h;
            (void)hipGetLastError();
            return fail(PE_ERR_OOM, "hipMalloc for the bias: %s", hipGetErrorString(e));
        }
    }
    e = pe::launch_pack(weight, wes, h->wpk, cfg->patch_size, cfg->embed_dim, pe::kPackTT, st);
    if (e == hipSuccess && rows_bytes)
        e = pe::launch_pack(weight, wes, h->wpk_rows, cfg->patch_size, cfg->embed_dim, pe::kPackRows, st);
    if (e == hipSuccess && fold_bytes)
        e = pe::launch_pack(weight, wes, h->wpk_fold, cfg->patch_size, cfg->embed_dim, pe::kPackFold, st);
    if (e == hipSuccess && grp_bytes)
        e = pe::launch_pack(weight, wes, h->wpk_grp, cfg->patch_size, cfg->embed_dim, pe::kPackTTG, st);
    if (e == hipSuccess && bias) e = pe::launch_bias(bias, wes, h->bias32, cfg->embed_dim, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        int rc = hip_fail(e, "weight pre-pack");
        (void)hipFree(h->wpk);
        if (h->bias32) (void)hipFree(h->bias32);
        delete h;
        return rc;
    }
    *out = h;
    g_err.clear();
    return PE_OK;
}

int pe_destroy(pe_handle h) {
    if (!h) return PE_OK;
    DeviceGuard dg(h->device);
    hipError_t e1 = hipFree(h->wpk);
    hipError_t e2 = h->bias32 ? hipFree(h->bias32) : hipSuccess;
    delete h;
    if (e1 != hipSuccess) return hip_fail(e1, "hipFree");
    if (e2 != hipSuccess) return hip_fail(e2, "hipFree");
    return PE_OK;
}

}  // extern "C"

namespace {

void fill_request(pe_handle h, int32_t input_kind, int32_t in_dtype, const int32_t *grid_thw, const int32_t *frames,
                  int32_t n_items, pe::PlanRequest &rq) {
    const pe_config &cfg = h->cfg;
    rq.P = cfg.patch_size;
    rq.E = cfg.embed_dim;
    rq.m = cfg.spatial_merge_size;
    rq.weight_esz = esize(cfg.weight_dtype);
    rq.in_esz = esize(in_dtype);
    rq.out_esz = esize(cfg.out_dtype);
    rq.merge = cfg.out_order == PE_ORDER_MERGE_WINDOW;
    rq.image_fold = cfg.image_fold;
    rq.stage_images = cfg.stage_images;
    rq.num_cus = h->num_cus;
    rq.input_kind = input_kind;
    rq.grid_thw = grid_thw;
    rq.frames = frames;
    rq.n_items = n_items;
}

// checks of pe_forward's handle and dtype arguments (the plan checks the grid)
int check_request(pe_handle h, int32_t input_kind, int32_t in_dtype, int32_t n_items, const int32_t *grid_thw) {
    if (!h) return fail(PE_ERR_INVALID_ARG, "handle is NULL");
    if (n_items < 0) return fail(PE_ERR_INVALID_ARG, "n_items must be >= 0 (got %d)", n_items);
    if (n_items == 0) return fail(PE_ERR_SHAPE, "no items: N = 0");
    if (!grid_thw) return fail(PE_ERR_INVALID_ARG, "grid_thw is NULL");
    if (input_kind != PE_INPUT_PATCHES && input_kind != PE_INPUT_FRAMES)
        return fail(PE_ERR_INVALID_ARG, "bad input_kind %d", input_kind);
    if (!dtype_ok(in_dtype)) return fail(PE_ERR_INVALID_ARG, "bad in_dtype %d", in_dtype);
    const pe_config &cfg = h->cfg;
    // bf16 weight: bf16 input, or fp32 input rounded to bf16 on load; fp32 weight: fp32 input
    if (in_dtype != cfg.weight_dtype && !(cfg.weight_dtype == PE_BF16 && in_dtype == PE_F32))
        return fail(PE_ERR_UNSUPPORTED, "in_dtype %d with weight dtype %d: supported are bf16/bf16, "
                    "fp32/bf16 (rounded on load) and fp32/fp32", in_dtype, cfg.weight_dtype);
    return PE_OK;
}

// pe_forward and pe_forward_add: addend is null for the plain forward
int forward_impl(pe_handle h, int32_t input_kind, const void *input, int32_t in_dtype,
                 const int32_t *grid_thw, const int32_t *frames, int32_t n_items, const void *addend,
                 void *out, void *hip_stream) {
    if (!h) return fail(PE_ERR_INVALID_ARG, "handle is NULL");
    if (n_items < 0) return fail(PE_ERR_INVALID_ARG, "n_items must be >= 0 (got %d)", n_items);
    if (n_items == 0) return fail(PE_ERR_SHAPE, "no items: N = 0");
    if (!grid_thw) return fail(PE_ERR_INVALID_ARG, "grid_thw is NULL");
    if (!input) return fail(PE_ERR_INVALID_ARG, "input is NULL");
    if (!out) return fail(PE_ERR_INVALID_ARG, "out is NULL");
    const int crc = check_request(h, input_kind, in_dtype, n_items, grid_thw);
    if (crc != PE_OK) return crc;
    const pe_config &cfg = h->cfg;

    pe::PlanRequest rq;
    fill_request(h, input_kind, in_dtype, grid_thw, frames, n_items, rq);
    std::vector<pe::Launch> plan;
    std::string err;
    const int rc = pe::plan_forward(rq, plan, err);
    if (rc != PE_OK) return fail(rc, "%s", err.c_str());

    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int64_t row_bytes = (int64_t)cfg.embed_dim * rq.out_esz;
    // every launch's packed weight is bound (and checked) before the first launch is queued
    for (pe::Launch &L : plan) {
        switch (L.weight_map) {
            case pe::kWeightRows: L.a.wpk = h->wpk_rows; break;
            case pe::kWeightFold: L.a.wpk = h->wpk_fold; break;
            case pe::kWeightGrouped: L.a.wpk = h->wpk_grp; break;
            default: L.a.wpk = h->wpk; break;
        }
        if (!L.a.wpk) return fail(PE_ERR_UNSUPPORTED, "the plan asks for a packed weight the handle does not hold");
    }
    for (pe::Launch &L : plan) {
        pe::FwdArgs &a = L.a;
        a.bias = h->bias32;
        a.in = static_cast<const char *>(input) + L.in_off;
        a.out = static_cast<char *>(out) + L.row0 * row_bytes;
        a.addend = addend ? static_cast<const char *>(addend) + L.row0 * row_bytes : nullptr;
        hipError_t e = pe::launch_forward(a, rq.P, rq.weight_esz, rq.in_esz, rq.out_esz, st);
        if (e != hipSuccess) return hip_fail(e, "forward launch");
    }
    return PE_OK;
}

}  // namespace

extern "C" {

int pe_forward(pe_handle h, int32_t input_kind, const void *input, int32_t in_dtype,
               const int32_t *grid_thw, const int32_t *frames, int32_t n_items, void *out,
               void *hip_stream) {
    return forward_impl(h, input_kind, input, in_dtype, grid_thw, frames, n_items, nullptr, out, hip_stream);
}

int pe_forward_add(pe_handle h, int32_t input_kind, const void *input, int32_t in_dtype,
                   const int32_t *grid_thw, const int32_t *frames, int32_t n_items, const void *addend,
                   void *out, void *hip_stream) {
    if (n_items > 0 && !addend) return fail(PE_ERR_INVALID_ARG, "addend is NULL");
    return forward_impl(h, input_kind, input, in_dtype, grid_thw, frames, n_items, addend, out, hip_stream);
}

int pe_forward_plan(pe_handle h, int32_t input_kind, int32_t in_dtype, const int32_t *grid_thw,
                    const int32_t *frames, int32_t n_items, pe_launch_info *info, int32_t max_info) {
    if (max_info < 0 || (max_info > 0 && !info))
        return fail(PE_ERR_INVALID_ARG, "info must hold max_info >= 0 entries");
    const int crc = check_request(h, input_kind, in_dtype, n_items, grid_thw);
    if (crc != PE_OK) return crc;
    pe::PlanRequest rq;
    fill_request(h, input_kind, in_dtype, grid_thw, frames, n_items, rq);
    std::vector<pe::Launch> plan;
    std::string err;
    const int rc = pe::plan_forward(rq, plan, err);
    if (rc != PE_OK) return fail(rc, "%s", err.c_str());
    for (size_t i = 0; i < plan.size() && (int64_t)i < max_info; ++i) {
        const pe::Launch &L = plan[i];
        pe_launch_info &o = info[i];
        memset(&o, 0, sizeof o);
        snprintf(o.kernel, sizeof o.kernel, "%s", pe::kernel_name(L.tile.id));
        o.tile_rows = L.tile.bm;
        o.tile_cols = L.tile.bn;
        o.workgroups = L.workgroups;
        o.row0 = L.row0;
        o.n_rows = L.a.n_rows;
        o.in_offset = (int64_t)L.in_off;
        o.in_bytes = L.a.in_bytes;
        o.n_items = L.a.n_items;
        o.a_mode = L.a.kind == 0 ? PE_A_PATCH_ROWS
                 : L.a.fold      ? PE_A_FOLDED_IMAGES
                 : L.a.staged    ? PE_A_IMAGES_LDS
                 : L.a.img       ? PE_A_IMAGES
                                 : PE_A_FRAMES;
    }
    return plan.size() > (size_t)INT32_MAX ? fail(PE_ERR_SHAPE, "too many launches") : (int)plan.size();
}

int pe_layernorm(const void *x, int32_t dtype, const void *gamma, const void *beta, int32_t param_dtype,
                 float eps, int64_t n_rows, int32_t dim, void *y, void *hip_stream) {
    if (n_rows < 0) return fail(PE_ERR_INVALID_ARG, "n_rows must be >= 0 (got %lld)", (long long)n_rows);
    if (!dtype_ok(dtype) || !dtype_ok(param_dtype))
        return fail(PE_ERR_INVALID_ARG, "dtype %d / param_dtype %d is not a pe_dtype", dtype, param_dtype);
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(PE_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (dim <= 0 || dim % 8 != 0 || dim > pe::kNormMaxDim)
        return fail(PE_ERR_UNSUPPORTED, "dim %d: a positive multiple of 8 up to %d is supported", dim, pe::kNormMaxDim);
    if (n_rows == 0) return PE_OK;
    if (!x || !y) return fail(PE_ERR_INVALID_ARG, "x or y is NULL");
    const int es = esize(dtype);
    if (n_rows > INT64_MAX / ((int64_t)dim * es)) return fail(PE_ERR_SHAPE, "n_rows * dim overflows");
    const uintptr_t al = (uintptr_t)x | (uintptr_t)y | (uintptr_t)gamma | (uintptr_t)beta;
    if (al & 15) return fail(PE_ERR_INVALID_ARG, "x, y, gamma and beta must be 16-byte aligned");
    const uintptr_t bytes = (uintptr_t)(n_rows * dim * es);
    const uintptr_t xb = (uintptr_t)x, yb = (uintptr_t)y;
    if (xb != yb && xb < yb + bytes && yb < xb + bytes)
        return fail(PE_ERR_INVALID_ARG, "y overlaps x without being x");
    hipError_t e = pe::launch_layernorm(x, es, y, gamma, beta, esize(param_dtype), eps, n_rows, dim,
                                        static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "layernorm launch");
    return PE_OK;
}

}  // extern "C"
