// RMSNorm, fused into one pass and as the four passes of the unfused form
// ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.2 byte ledger and the
// appendix ledger's RMSNorm entry: square, mean, multiply by the reciprocal
// root, multiply by the gain):
//   y[i][j] = x[i][j] / sqrt(mean_j x[i][j]^2 + eps) * g[j]      (fp32)
//
// Fused: one 256-thread workgroup per row.  Thread t holds the row's 16-byte
// vectors t, t + 256, ... (at most 16, so d <= 16384) in registers, loaded
// nontemporally; the sum of squares is reduced across the wave by shuffles
// and across the 4 waves through LDS; one correctly rounded 1/sqrt per row;
// the outputs are written nontemporally.  x is read once and y written once.
//
// Unfused: four launches over a workspace, each a plain streaming kernel:
//   1. s = x * x                    (n -> n)
//   2. m[i] = mean_j s[i][j]        (n -> rows, one workgroup per row)
//   3. t = x * (1 / sqrt(m + eps))  (n + rows -> n, into the buffer of s)
//   4. y = t * g                    (n + d -> n)
#include "fc_internal.h"

namespace fc {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace rms {
constexpr int NT = 256, MAXV = 16;
}

__device__ __forceinline__ float rms_block_sum(float v, float *red)
{
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int NV>
__global__ __launch_bounds__(rms::NT) void rmsnorm_fused_kernel(const float *__restrict__ x,
                                                                const float *__restrict__ g,
                                                                float *__restrict__ y, int d, float eps)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int nvec = d >> 2;
    const f32x4 *xv = reinterpret_cast<const f32x4 *>(x + row * d);
    f32x4 *yv = reinterpret_cast<f32x4 *>(y + row * d);
    const f32x4 *gv = reinterpret_cast<const f32x4 *>(g);
    f32x4 v[NV];
    float ss = 0.0f;
    // unconditional loads from clamped indices, out-of-row vectors zeroed by a
    // select: a load behind a branch would be waited for before the next one
#pragma unroll
    for (int u = 0; u < NV; ++u) v[u] = __builtin_nontemporal_load(xv + min((int)threadIdx.x + u * rms::NT, nvec - 1));
#pragma unroll
    for (int u = 0; u < NV; ++u)
        if ((int)threadIdx.x + u * rms::NT >= nvec) v[u] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < NV; ++u)
        ss += (v[u].x * v[u].x + v[u].y * v[u].y) + (v[u].z * v[u].z + v[u].w * v[u].w);
    const float total = rms_block_sum(ss, red);
    const float r = 1.0f / sqrtf(total / (float)d + eps);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int i = threadIdx.x + u * rms::NT;
        if (i < nvec) __builtin_nontemporal_store(v[u] * r * gv[i], yv + i);
    }
}

// pass 1 and pass 4: elementwise over n/4 vectors (grid-stride)
__global__ __launch_bounds__(rms::NT) void rms_square_kernel(const f32x4 *__restrict__ x, f32x4 *__restrict__ s,
                                                             int64_t nvec)
{
    for (int64_t i = (int64_t)blockIdx.x * rms::NT + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * rms::NT) {
        const f32x4 a = x[i];
        s[i] = a * a;
    }
}

__global__ __launch_bounds__(rms::NT) void rms_mean_kernel(const float *__restrict__ s, float *__restrict__ m,
                                                           int d)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const f32x4 *sv = reinterpret_cast<const f32x4 *>(s + row * d);
    float acc = 0.0f;
    for (int i = threadIdx.x; i < (d >> 2); i += rms::NT) {
        const f32x4 a = sv[i];
        acc += (a.x + a.y) + (a.z + a.w);
    }
    const float total = rms_block_sum(acc, red);
    if (threadIdx.x == 0) m[row] = total / (float)d;
}

__global__ __launch_bounds__(rms::NT) void rms_scale_kernel(const f32x4 *__restrict__ x,
                                                            const float *__restrict__ m, f32x4 *__restrict__ t,
                                                            int64_t nvec, int dvec, float eps)
{
    for (int64_t i = (int64_t)blockIdx.x * rms::NT + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * rms::NT)
        t[i] = x[i] * (1.0f / sqrtf(m[i / dvec] + eps));
}

__global__ __launch_bounds__(rms::NT) void rms_gain_kernel(const f32x4 *__restrict__ t,
                                                           const f32x4 *__restrict__ g, f32x4 *__restrict__ y,
                                                           int64_t nvec, int dvec)
{
    for (int64_t i = (int64_t)blockIdx.x * rms::NT + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * rms::NT)
        y[i] = t[i] * g[i % dvec];
}

static int rms_grid(int64_t nvec)
{
    int64_t g = ceil_div(nvec, (int64_t)rms::NT * 4);
    return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

template <int NV>
static void launch_fused(const float *x, const float *g, float *y, int64_t rows, int d, float eps, hipStream_t s)
{
    rmsnorm_fused_kernel<NV><<<(unsigned)rows, rms::NT, 0, s>>>(x, g, y, d, eps);
}

}  // namespace fc

using namespace fc;

extern "C" size_t fc_rmsnorm_workspace_bytes(int64_t rows, int d, int mode)
{
    if (rows < 1 || d < 1 || mode != FC_RMSNORM_UNFUSED) return 0;
    const size_t n = (size_t)rows * (size_t)d;
    return ((4 * n + 255) & ~(size_t)255) + 4 * (size_t)rows;
}

extern "C" uint64_t fc_rmsnorm_bytes(int64_t rows, int d, int mode)
{
    if (rows < 1 || d < 1 || (mode != FC_RMSNORM_FUSED && mode != FC_RMSNORM_UNFUSED)) return 0;
    const uint64_t n = (uint64_t)rows * (uint64_t)d;
    return (mode == FC_RMSNORM_FUSED ? 1u : 4u) * 2u * 4u * n;
}

extern "C" int fc_rmsnorm(const float *x, const float *g, float *y, int64_t rows, int d, float eps, int mode,
                          void *workspace, size_t ws_bytes, fc_stream stream)
{
    if (mode != FC_RMSNORM_FUSED && mode != FC_RMSNORM_UNFUSED) return FC_ERR_UNSUPPORTED;
    if (rows < 1 || d < 1) return FC_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return FC_ERR_SHAPE;
    if (d % 4 != 0 || d > rms::NT * 4 * rms::MAXV || rows > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    if (!x || !g || !y) return FC_ERR_NULL;
    if (!aligned16(x) || !aligned16(g) || !aligned16(y)) return FC_ERR_ALIGN;
    const size_t nb = (size_t)rows * (size_t)d * 4;
    if (overlaps(y, nb, x, nb) || overlaps(y, nb, g, (size_t)d * 4)) return FC_ERR_ALIAS;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (mode == FC_RMSNORM_FUSED) {
        const int nv = (d / 4 + rms::NT - 1) / rms::NT;
        if (nv <= 1) launch_fused<1>(x, g, y, rows, d, eps, s);
        else if (nv <= 2) launch_fused<2>(x, g, y, rows, d, eps, s);
        else if (nv <= 4) launch_fused<4>(x, g, y, rows, d, eps, s);
        else if (nv <= 8) launch_fused<8>(x, g, y, rows, d, eps, s);
        else launch_fused<16>(x, g, y, rows, d, eps, s);
        return launch_status();
    }
    const size_t need = fc_rmsnorm_workspace_bytes(rows, d, mode);
    if (!workspace || ws_bytes < need) return FC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FC_ERR_ALIGN;
    if (overlaps(workspace, need, x, nb) || overlaps(workspace, need, y, nb) ||
        overlaps(workspace, need, g, (size_t)d * 4))
        return FC_ERR_ALIAS;
    float *sbuf = static_cast<float *>(workspace);
    float *mbuf = reinterpret_cast<float *>(static_cast<char *>(workspace) + ((4 * (size_t)rows * d + 255) & ~(size_t)255));
    const int64_t nvec = (int64_t)rows * d / 4;
    const int grid = rms_grid(nvec);
    const f32x4 *xv = reinterpret_cast<const f32x4 *>(x);
    f32x4 *sv = reinterpret_cast<f32x4 *>(sbuf);
    rms_square_kernel<<<grid, rms::NT, 0, s>>>(xv, sv, nvec);
    if (launch_status() != FC_OK) return FC_ERR_HIP;
    rms_mean_kernel<<<(unsigned)rows, rms::NT, 0, s>>>(sbuf, mbuf, d);
    if (launch_status() != FC_OK) return FC_ERR_HIP;
    rms_scale_kernel<<<grid, rms::NT, 0, s>>>(xv, mbuf, sv, nvec, d / 4, eps);
    if (launch_status() != FC_OK) return FC_ERR_HIP;
    rms_gain_kernel<<<grid, rms::NT, 0, s>>>(sv, reinterpret_cast<const f32x4 *>(g), reinterpret_cast<f32x4 *>(y),
                                             nvec, d / 4);
    return launch_status();
}
