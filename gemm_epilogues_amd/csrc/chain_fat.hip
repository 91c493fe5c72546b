// Fat probe of the fused chain: the fused kernel plus T live fp32x4
// temporaries per lane, a register-pressure probe ("C-05. Kernel Fusion 代价边界",
// section 3, the fat row of the API table; its occupancy result in section 6.2).
#include "chain_common.h"

namespace fc {

// Fat probe: the fused chain plus T live fp32x4 temporaries per lane.
// Temporaries form a forward recurrence fed by the chain value of the stage
// they are produced at (t_j = 0.5*t_{j-1} + v_{s(j)}, s(j) = floor(j*K/T)),
// and the sink adds them in the reverse order t_0 + (t_1 + (... + t_{T-1})),
// so all T are live at once (no reassociation without fast-math) and none can
// be eliminated.  The chain value itself is untouched: y equals the fused y.
template <int K, bool RELU, int T>
__global__ __launch_bounds__(kChainBlock) void chain_fat_kernel(const float *__restrict__ x,
                                                                float *__restrict__ y, int64_t n,
                                                                ChainCoef c,
                                                                f32x4 *__restrict__ sink)
{
    const int64_t nvec = n >> 2;
    const f32x4 *xv = reinterpret_cast<const f32x4 *>(x);
    f32x4 *yv = reinterpret_cast<f32x4 *>(y);
    const int64_t stride = (int64_t)gridDim.x * kChainBlock;
    const int64_t gtid = (int64_t)blockIdx.x * kChainBlock + threadIdx.x;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = gtid; i < nvec; i += stride) {
        f32x4 v = __builtin_nontemporal_load(xv + i);
        if constexpr (T > 0) {
            f32x4 t[T];
            f32x4 prev = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < K; ++s) {
                v.x = stage_scalar(v.x, c.a[s], c.b[s], RELU && (s % 2) == 0);
                v.y = stage_scalar(v.y, c.a[s], c.b[s], RELU && (s % 2) == 0);
                v.z = stage_scalar(v.z, c.a[s], c.b[s], RELU && (s % 2) == 0);
                v.w = stage_scalar(v.w, c.a[s], c.b[s], RELU && (s % 2) == 0);
#pragma unroll
                for (int jj = 0; jj < T; ++jj) {
                    if ((jj * K) / T == s) {
                        prev.x = __builtin_fmaf(0.5f, prev.x, v.x);
                        prev.y = __builtin_fmaf(0.5f, prev.y, v.y);
                        prev.z = __builtin_fmaf(0.5f, prev.z, v.z);
                        prev.w = __builtin_fmaf(0.5f, prev.w, v.w);
                        t[jj] = prev;
                    }
                }
            }
            f32x4 r = t[T - 1];
#pragma unroll
            for (int jj = T - 2; jj >= 0; --jj) {
                r.x = t[jj].x + r.x;
                r.y = t[jj].y + r.y;
                r.z = t[jj].z + r.z;
                r.w = t[jj].w + r.w;
            }
            acc.x += r.x;
            acc.y += r.y;
            acc.z += r.z;
            acc.w += r.w;
        } else {
            v = chain_vec<K, RELU>(v, c);
        }
        __builtin_nontemporal_store(v, yv + i);
    }
    sink[gtid] = acc;
    chain_tail<K, RELU>(x, y, n, c);
}

// Fat grid: fixed function of n, so the sink layout is reproducible.
constexpr int kFatMaxBlocks = 2048;
int chain_fat_grid(int64_t n)
{
    int64_t want = ceil_div(n >> 2, (int64_t)kChainBlock);
    if (want < 1) want = 1;
    if (want > kFatMaxBlocks) want = kFatMaxBlocks;
    return (int)want;
}

template <int K, bool RELU, int T>
static void launch_fat(const float *x, float *y, int64_t n, const ChainCoef &c, float *sink,
                       hipStream_t s)
{
    chain_fat_kernel<K, RELU, T><<<chain_fat_grid(n), kChainBlock, 0, s>>>(
        x, y, n, c, reinterpret_cast<f32x4 *>(sink));
}

template <int K, bool RELU>
static int dispatch_fat(const float *x, float *y, int64_t n, const ChainCoef &c, float *sink,
                        int temps, hipStream_t s)
{
    switch (temps) {
    case 0: launch_fat<K, RELU, 0>(x, y, n, c, sink, s); break;
    case 16: launch_fat<K, RELU, 16>(x, y, n, c, sink, s); break;
    case 48: launch_fat<K, RELU, 48>(x, y, n, c, sink, s); break;
    case 96:
        if constexpr (K == 4) { launch_fat<K, RELU, 96>(x, y, n, c, sink, s); break; }
        return FC_ERR_UNSUPPORTED;
    case 128:
        if constexpr (K == 4) { launch_fat<K, RELU, 128>(x, y, n, c, sink, s); break; }
        return FC_ERR_UNSUPPORTED;
    default: return FC_ERR_UNSUPPORTED;
    }
    return FC_OK;
}

bool chain_fat_supported(int K, int temps)
{
    const bool k_ok = K == 1 || K == 2 || K == 3 || K == 4 || K == 6 || K == 8;
    const bool t_small = temps == 0 || temps == 16 || temps == 48;
    const bool t_big = (temps == 96 || temps == 128) && K == 4;   // the T sweep runs at K = 4
    return k_ok && (t_small || t_big);
}

template <bool RELU>
static int fat_k(int K, const float *x, float *y, int64_t n, const ChainCoef &c, float *sink,
                 int temps, hipStream_t s)
{
    switch (K) {
    case 1: return dispatch_fat<1, RELU>(x, y, n, c, sink, temps, s);
    case 2: return dispatch_fat<2, RELU>(x, y, n, c, sink, temps, s);
    case 3: return dispatch_fat<3, RELU>(x, y, n, c, sink, temps, s);
    case 4: return dispatch_fat<4, RELU>(x, y, n, c, sink, temps, s);
    case 6: return dispatch_fat<6, RELU>(x, y, n, c, sink, temps, s);
    case 8: return dispatch_fat<8, RELU>(x, y, n, c, sink, temps, s);
    default: return FC_ERR_UNSUPPORTED;
    }
}

int launch_chain_fat(int K, bool relu, const float *x, float *y, int64_t n, const ChainCoef &c,
                     float *sink, int temps, hipStream_t s)
{
    if (!chain_fat_supported(K, temps)) return FC_ERR_UNSUPPORTED;
    return relu ? fat_k<true>(K, x, y, n, c, sink, temps, s)
                : fat_k<false>(K, x, y, n, c, sink, temps, s);
}

}  // namespace fc
