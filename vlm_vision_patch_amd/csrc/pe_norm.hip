// pe_norm.hip -- LayerNorm over the last dimension of a row-major [rows, dim] tensor: the first
// step of the PatchMerger that follows the vision tower ("freechatgpt/mytransformer", the vision
// encoder structure in section 3.2 and the PatchMerger bullet of section 4.1: LayerNorm, then the
// 2x2 neighbouring patches concatenated to 4E). With the PatchEmbed rows in merge-window order
// that concatenation is a view of the normalized rows, so this kernel is the whole front end.
//
// y = (x - mean) / sqrt(var + eps) * gamma + beta per row, mean and (biased) variance over the
// dim elements of the row, all arithmetic in fp32, one round-to-nearest-even cast of y.
//
// HBM-bound: every element is read once and written once. L lanes (32 or 64) own one row; each
// lane holds CPL 16-byte chunks of it in registers (chunk j of lane l is chunk j*L + l of the
// row, so a wave's loads of one j are contiguous), the mean comes from a first lane-then-tree
// reduction and the variance from a second one over the centred register values (no
// E[x^2] - mean^2 cancellation), then the row is written back from the registers. Rows are
// independent and each element is read and written by the same lane, so y may be x.
#include "pe_device.h"

namespace pe {

template <int ESZ>
__device__ __forceinline__ void unpack_chunk(const u32x4 &d, float (&v)[16 / ESZ]) {
    if constexpr (ESZ == 2) {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    } else {
        const f32x4 f = __builtin_bit_cast(f32x4, d);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
}

// VPC consecutive parameter values (gamma or beta) starting at element e0, as fp32
template <int PSZ, int VPC>
__device__ __forceinline__ void load_param(const void *p, int e0, float (&o)[VPC]) {
    if constexpr (PSZ == 4) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + e0);
#pragma unroll
        for (int i = 0; i < VPC / 4; ++i) {
            const f32x4 t = q[i];
            o[4 * i] = t.x; o[4 * i + 1] = t.y; o[4 * i + 2] = t.z; o[4 * i + 3] = t.w;
        }
    } else {
        const uint16_t *q = static_cast<const uint16_t *>(p) + e0;
        uint32_t w[VPC / 2];
        if constexpr (VPC == 8) {
            const u32x4 t = *reinterpret_cast<const u32x4 *>(q);
            w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
        } else {
            const u32x2 t = *reinterpret_cast<const u32x2 *>(q);
            w[0] = t.x; w[1] = t.y;
        }
#pragma unroll
        for (int i = 0; i < VPC / 2; ++i) {
            o[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            o[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    }
}

template <int L>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int off = L / 2; off >= 1; off /= 2) v += __shfl_xor(v, off, 64);
    return v;
}

// ESZ: bytes of an x / y element; PSZ: bytes of a gamma / beta element; L lanes per row;
// CPL chunks per lane (CPL * L >= dim * ESZ / 16).
template <int ESZ, int PSZ, int L, int CPL>
__global__ __launch_bounds__(256) void pe_layernorm_kernel(const void *__restrict__ x, void *y,
                                                           const void *__restrict__ gamma,
                                                           const void *__restrict__ beta, float eps,
                                                           int64_t n_rows, int dim) {
    constexpr int VPC = 16 / ESZ;  // values per chunk
    const int64_t row = (int64_t)blockIdx.x * (256 / L) + threadIdx.x / L;
    if (row >= n_rows) return;  // whole L-lane groups leave together; reductions stay in a group
    const int li = threadIdx.x % L;
    const int nch = dim / VPC;
    const char *xr = static_cast<const char *>(x) + row * dim * ESZ;
    char *yr = static_cast<char *>(y) + row * dim * ESZ;

    float v[CPL][VPC];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = j * L + li;
        u32x4 d = u32x4{0u, 0u, 0u, 0u};
        if (c < nch) d = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + c * 16));
        unpack_chunk<ESZ>(d, v[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < VPC; ++e) s += v[j][e];  // chunks past the row hold zeros
    const float mean = row_sum<L>(s) / (float)dim;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        if (j * L + li < nch) {
#pragma unroll
            for (int e = 0; e < VPC; ++e) {
                v[j][e] -= mean;
                q += v[j][e] * v[j][e];
            }
        }
    }
    const float var = row_sum<L>(q) / (float)dim;
    const float rstd = 1.0f / sqrtf(var + eps);

#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = j * L + li;
        if (c >= nch) continue;
        float g[VPC], b[VPC];
        if (gamma) load_param<PSZ, VPC>(gamma, c * VPC, g);
        else
#pragma unroll
            for (int e = 0; e < VPC; ++e) g[e] = 1.f;
        if (beta) load_param<PSZ, VPC>(beta, c * VPC, b);
        else
#pragma unroll
            for (int e = 0; e < VPC; ++e) b[e] = 0.f;
        float o[VPC];
#pragma unroll
        for (int e = 0; e < VPC; ++e) o[e] = __builtin_fmaf(v[j][e] * rstd, g[e], b[e]);
        store_chunk_r<ESZ>(yr, false, u32x4{0u, 0u, 0u, 0u}, (int64_t)c * VPC, o);
    }
}

namespace {

template <int ESZ, int PSZ, int L, int CPL>
hipError_t ln_launch(const void *x, void *y, const void *g, const void *b, float eps, int64_t n_rows, int dim,
                     hipStream_t st) {
    constexpr int rows_per_block = 256 / L;
    const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((pe_layernorm_kernel<ESZ, PSZ, L, CPL>), dim3((unsigned)blocks), dim3(256), 0, st, x, y, g, b,
                       eps, n_rows, dim);
    return hipGetLastError();
}

// chunks per lane for a row of nch 16-byte chunks: 32 lanes per row up to 256 chunks, then 64
template <int ESZ, int PSZ>
hipError_t ln_dispatch(const void *x, void *y, const void *g, const void *b, float eps, int64_t n_rows, int dim,
                       hipStream_t st) {
    const int nch = dim * ESZ / 16;
    if (nch <= 32 * 8) {
        switch ((nch + 31) / 32) {
        case 1: return ln_launch<ESZ, PSZ, 32, 1>(x, y, g, b, eps, n_rows, dim, st);
        case 2: return ln_launch<ESZ, PSZ, 32, 2>(x, y, g, b, eps, n_rows, dim, st);
        case 3: return ln_launch<ESZ, PSZ, 32, 3>(x, y, g, b, eps, n_rows, dim, st);
        case 4: return ln_launch<ESZ, PSZ, 32, 4>(x, y, g, b, eps, n_rows, dim, st);
        case 5: return ln_launch<ESZ, PSZ, 32, 5>(x, y, g, b, eps, n_rows, dim, st);
        case 6: return ln_launch<ESZ, PSZ, 32, 6>(x, y, g, b, eps, n_rows, dim, st);
        case 7: return ln_launch<ESZ, PSZ, 32, 7>(x, y, g, b, eps, n_rows, dim, st);
        default: return ln_launch<ESZ, PSZ, 32, 8>(x, y, g, b, eps, n_rows, dim, st);
        }
    }
    const int cpl = (nch + 63) / 64;  // 5 .. 16 for dim <= kNormMaxDim
    if (cpl <= 6) return ln_launch<ESZ, PSZ, 64, 6>(x, y, g, b, eps, n_rows, dim, st);
    if (cpl <= 8) return ln_launch<ESZ, PSZ, 64, 8>(x, y, g, b, eps, n_rows, dim, st);
    if (cpl <= 12) return ln_launch<ESZ, PSZ, 64, 12>(x, y, g, b, eps, n_rows, dim, st);
    if (cpl <= 16) return ln_launch<ESZ, PSZ, 64, 16>(x, y, g, b, eps, n_rows, dim, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_layernorm(const void *x, int esz, void *y, const void *gamma, const void *beta, int psz,
                            float eps, int64_t n_rows, int dim, hipStream_t st) {
    if (dim <= 0 || dim % 8 != 0 || dim > kNormMaxDim || n_rows <= 0) return hipErrorInvalidValue;
    // at most 2^24 rows per launch: 4M blocks of 256 work-items keeps the grid far below 2^32
    constexpr int64_t kRowsPerLaunch = int64_t(1) << 24;
    for (int64_t r0 = 0; r0 < n_rows; r0 += kRowsPerLaunch) {
        const int64_t nr = n_rows - r0 < kRowsPerLaunch ? n_rows - r0 : kRowsPerLaunch;
        const void *xs = static_cast<const char *>(x) + r0 * dim * esz;
        void *ys = static_cast<char *>(y) + r0 * dim * esz;
        hipError_t e;
        if (esz == 2) e = psz == 2 ? ln_dispatch<2, 2>(xs, ys, gamma, beta, eps, nr, dim, st)
                                   : ln_dispatch<2, 4>(xs, ys, gamma, beta, eps, nr, dim, st);
        else e = psz == 2 ? ln_dispatch<4, 2>(xs, ys, gamma, beta, eps, nr, dim, st)
                          : ln_dispatch<4, 4>(xs, ys, gamma, beta, eps, nr, dim, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pe
