// Shared by the chain translation units (fused/naive and fat probe).
#pragma once

#include "fc_internal.h"

namespace fc {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ChainCoef {
    float a[FC_CHAIN_MAX_STAGES];
    float b[FC_CHAIN_MAX_STAGES];
};

constexpr int kChainBlock = 256;
constexpr int kChainUnroll = 4;     // fat probe: vectors in flight per lane
constexpr int kChainVecs = 8;       // fused / naive: contiguous vectors per lane

template <int K, bool RELU>
__device__ __forceinline__ float chain_scalar(float v, const ChainCoef &c)
{
#pragma unroll
    for (int s = 0; s < K; ++s) {
        v = __builtin_fmaf(c.a[s], v, c.b[s]);
        if (RELU && (s % 2) == 0) v = fmaxf(v, 0.0f);
    }
    return v;
}

template <int K, bool RELU>
__device__ __forceinline__ f32x4 chain_vec(f32x4 v, const ChainCoef &c)
{
    v.x = chain_scalar<K, RELU>(v.x, c);
    v.y = chain_scalar<K, RELU>(v.y, c);
    v.z = chain_scalar<K, RELU>(v.z, c);
    v.w = chain_scalar<K, RELU>(v.w, c);
    return v;
}

// One stage with runtime coefficients (the naive form launches this K times).
__device__ __forceinline__ float stage_scalar(float v, float a, float b, bool relu)
{
    v = __builtin_fmaf(a, v, b);
    return relu ? fmaxf(v, 0.0f) : v;
}

// Scalar tail (n % 4 elements) handled by the first lanes of block 0.
template <int K, bool RELU>
__device__ __forceinline__ void chain_tail(const float *x, float *y, int64_t n, const ChainCoef &c)
{
    int64_t t = (n & ~int64_t(3)) + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < 4 && t < n) y[t] = chain_scalar<K, RELU>(x[t], c);
}

// Fat probe (chain_fat.hip).
int chain_fat_grid(int64_t n);
bool chain_fat_supported(int K, int temps);
int launch_chain_fat(int K, bool relu, const float *x, float *y, int64_t n, const ChainCoef &c,
                     float *sink, int temps, hipStream_t s);

}  // namespace fc
