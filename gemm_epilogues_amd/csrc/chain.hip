// K-stage pointwise chain y = a_s*y + b_s (ReLU after even stages) in three
// forms -- naive (one launch per stage), fused (one launch, stages in VGPRs)
// and fat (fused plus live temporaries that raise register pressure).
// Stage operation and forms: "C-05. Kernel Fusion 代价边界", sections 2-3.
//
// HBM-bound streaming: each lane moves fp32x4 (128-bit global loads/stores),
// UNROLL independent vectors in flight per lane, grid-stride over the tensor.
#include "chain_common.h"

namespace fc {

// Each workgroup streams one contiguous chunk of kChainBlock * kChainVecs
// fp32x4 vectors: all kChainVecs loads of a lane are issued before any
// store, lanes interleave within each 4 KiB run, and at n = 16M the whole
// grid (2048 workgroups, 8 per CU) is resident at once, so there is no tail
// round.
template <int K, bool RELU>
__global__ __launch_bounds__(kChainBlock) void chain_fused_kernel(const float *__restrict__ x,
                                                                  float *__restrict__ y, int64_t n,
                                                                  ChainCoef c)
{
    const int64_t nvec = n >> 2;
    const f32x4 *xv = reinterpret_cast<const f32x4 *>(x);
    f32x4 *yv = reinterpret_cast<f32x4 *>(y);
    const int64_t base = (int64_t)blockIdx.x * kChainBlock * kChainVecs + threadIdx.x;
    f32x4 v[kChainVecs];
#pragma unroll
    for (int u = 0; u < kChainVecs; ++u) {
        const int64_t i = base + u * kChainBlock;
        if (i < nvec) v[u] = __builtin_nontemporal_load(xv + i);
    }
#pragma unroll
    for (int u = 0; u < kChainVecs; ++u) {
        const int64_t i = base + u * kChainBlock;
        if (i < nvec) __builtin_nontemporal_store(chain_vec<K, RELU>(v[u], c), yv + i);
    }
    chain_tail<K, RELU>(x, y, n, c);
}

__global__ __launch_bounds__(kChainBlock) void chain_stage_kernel(const float *__restrict__ x,
                                                                  float *__restrict__ y, int64_t n,
                                                                  float a, float b, int relu)
{
    const int64_t nvec = n >> 2;
    const f32x4 *xv = reinterpret_cast<const f32x4 *>(x);
    f32x4 *yv = reinterpret_cast<f32x4 *>(y);
    const bool r = relu != 0;
    const int64_t base = (int64_t)blockIdx.x * kChainBlock * kChainVecs + threadIdx.x;
    f32x4 v[kChainVecs];
#pragma unroll
    for (int u = 0; u < kChainVecs; ++u) {
        const int64_t i = base + u * kChainBlock;
        if (i < nvec) v[u] = __builtin_nontemporal_load(xv + i);
    }
#pragma unroll
    for (int u = 0; u < kChainVecs; ++u) {
        const int64_t i = base + u * kChainBlock;
        if (i < nvec) {
            f32x4 w = v[u];
            w.x = stage_scalar(w.x, a, b, r);
            w.y = stage_scalar(w.y, a, b, r);
            w.z = stage_scalar(w.z, a, b, r);
            w.w = stage_scalar(w.w, a, b, r);
            __builtin_nontemporal_store(w, yv + i);
        }
    }
    int64_t t = (n & ~int64_t(3)) + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < 4 && t < n) y[t] = stage_scalar(x[t], a, b, r);
}

// ------------------------------------------------------------------ host

static int64_t grid_for(int64_t nvec)
{
    int64_t g = ceil_div(nvec, (int64_t)kChainBlock * kChainVecs);
    return g < 1 ? 1 : g;
}

template <int K, bool RELU>
static void launch_fused(const float *x, float *y, int64_t n, const ChainCoef &c, hipStream_t s)
{
    chain_fused_kernel<K, RELU><<<(unsigned)grid_for(n >> 2), kChainBlock, 0, s>>>(x, y, n, c);
}

template <bool RELU>
static int dispatch_k(int K, int mode, const float *x, float *y, int64_t n, const ChainCoef &c,
                      float *scratch, int temps, hipStream_t s)
{
    if (mode == FC_CHAIN_FAT) return launch_chain_fat(K, RELU, x, y, n, c, scratch, temps, s);
#define FC_K_CASE(KK) \
    case KK: launch_fused<KK, RELU>(x, y, n, c, s); return FC_OK;
    switch (K) {
        FC_K_CASE(1) FC_K_CASE(2) FC_K_CASE(3) FC_K_CASE(4) FC_K_CASE(5) FC_K_CASE(6)
        FC_K_CASE(7) FC_K_CASE(8) FC_K_CASE(9) FC_K_CASE(10) FC_K_CASE(11) FC_K_CASE(12)
        FC_K_CASE(13) FC_K_CASE(14) FC_K_CASE(15) FC_K_CASE(16) FC_K_CASE(17) FC_K_CASE(18)
        FC_K_CASE(19) FC_K_CASE(20) FC_K_CASE(21) FC_K_CASE(22) FC_K_CASE(23) FC_K_CASE(24)
        FC_K_CASE(25) FC_K_CASE(26) FC_K_CASE(27) FC_K_CASE(28) FC_K_CASE(29) FC_K_CASE(30)
        FC_K_CASE(31) FC_K_CASE(32)
    default: return FC_ERR_UNSUPPORTED;
    }
#undef FC_K_CASE
}

}  // namespace fc

using namespace fc;

extern "C" size_t fc_chain_scratch_floats(int64_t n, int K, int mode, int fat_temps)
{
    (void)fat_temps;
    if (n <= 0 || K < 1) return 0;
    if (mode == FC_CHAIN_NAIVE) return K >= 2 ? (size_t)n : 0;
    if (mode == FC_CHAIN_FAT) return (size_t)chain_fat_grid(n) * kChainBlock * 4;
    return 0;
}

extern "C" int fc_chain(const float *x, float *y, int64_t n, const float *a, const float *b, int K,
                        int relu_even, int mode, float *scratch, int fat_temps, fc_stream stream)
{
    if (n < 0) return FC_ERR_SHAPE;
    if ((n >> 2) / ((int64_t)kChainBlock * kChainVecs) >= 0x7fffffff) return FC_ERR_UNSUPPORTED;
    if (K < 1 || K > FC_CHAIN_MAX_STAGES) return FC_ERR_UNSUPPORTED;
    if (mode != FC_CHAIN_NAIVE && mode != FC_CHAIN_FUSED && mode != FC_CHAIN_FAT)
        return FC_ERR_UNSUPPORTED;
    if (!a || !b) return FC_ERR_NULL;
    if (mode == FC_CHAIN_FAT && !chain_fat_supported(K, fat_temps)) return FC_ERR_UNSUPPORTED;
    if (n == 0) return FC_OK;
    if (!x || !y) return FC_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return FC_ERR_ALIGN;
    const size_t nb = (size_t)n * sizeof(float);
    if (x != y && overlaps(x, nb, y, nb)) return FC_ERR_ALIAS;
    const size_t need = fc_chain_scratch_floats(n, K, mode, fat_temps);
    if (need) {
        if (!scratch) return FC_ERR_WORKSPACE;
        if (!aligned16(scratch)) return FC_ERR_ALIGN;
        if (overlaps(scratch, need * sizeof(float), x, nb) ||
            overlaps(scratch, need * sizeof(float), y, nb))
            return FC_ERR_ALIAS;
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (mode == FC_CHAIN_NAIVE) {
        // stage s writes y when (K-1-s) is even, else scratch: the last lands in y
        const unsigned grid = (unsigned)grid_for(n >> 2);
        const float *in = x;
        for (int st = 0; st < K; ++st) {
            float *out = ((K - 1 - st) % 2 == 0) ? y : scratch;
            const int relu = (relu_even && (st % 2) == 0) ? 1 : 0;
            chain_stage_kernel<<<grid, kChainBlock, 0, s>>>(in, out, n, a[st], b[st], relu);
            int rc = launch_status();
            if (rc != FC_OK) return rc;
            in = out;
        }
        return FC_OK;
    }

    ChainCoef c;
    for (int i = 0; i < FC_CHAIN_MAX_STAGES; ++i) {
        c.a[i] = i < K ? a[i] : 0.0f;
        c.b[i] = i < K ? b[i] : 0.0f;
    }
    int rc = relu_even ? dispatch_k<true>(K, mode, x, y, n, c, scratch, fat_temps, s)
                       : dispatch_k<false>(K, mode, x, y, n, c, scratch, fat_temps, s);
    if (rc != FC_OK) return rc;
    return launch_status();
}
