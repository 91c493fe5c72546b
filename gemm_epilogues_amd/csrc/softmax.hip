// Causal scaled-masked softmax over attention scores [BH, S, S] (bf16).
// Definition: query i sees keys j <= i, softmax of scale*s over them, zeros
// above the diagonal ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5;
// the five steps max/subtract/exp/sum/divide in the appendix's attention-tail
// section).
//
//  fused:   one wavefront per row.  The row's kept key tiles 0..floor(i/T) are
//           loaded once with 128-bit loads and held in VGPRs; wave-wide max and
//           sum reductions; the row is written once (zeros for skipped tiles,
//           which are never read).  HBM-bound: (kept-tile reads + full write).
//  unfused: the five steps as five kernels with bf16 intermediates in `out`,
//           fp32 row statistics and a materialised 0/1 mask (the baseline).
#include "fc_internal.h"

namespace fc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 4;          // one wave per row, 4 waves per block
constexpr int kSmBlock = 64 * kRowsPerBlock;
constexpr int kChunk = 512;               // elements per wave-wide 128-bit load
constexpr int kMaxRegChunks = 16;         // register-resident rows up to S = 8192
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void unpack8(u32x4 w, float f[8])
{
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

__device__ __forceinline__ void store8(uint16_t *p, const float f[8])
{
    u32x4 w;
    w.x = pack_bf16x2(f[0], f[1]);
    w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]);
    w.w = pack_bf16x2(f[6], f[7]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ void store8(float *p, const float f[8])
{
    f32x4 a = {f[0], f[1], f[2], f[3]};
    f32x4 b = {f[4], f[5], f[6], f[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(p) + 1);
}

__device__ __forceinline__ void store1(uint16_t *p, float f)
{
    *p = (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}
__device__ __forceinline__ void store1(float *p, float f) { *p = f; }

// ------------------------------------------------------------------ fused

// Register-resident form: S % 8 == 0 and S <= NCH * 512.
template <int NCH, typename OutT, bool COUNT>
__global__ __launch_bounds__(kSmBlock) void softmax_fused_kernel(
    const uint16_t *__restrict__ s, OutT *__restrict__ out, int64_t rows, int S, float k2,
    int tile, int32_t *__restrict__ tiles)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;                       // whole wave leaves; no block barrier below
    const int i = (int)(row % S);
    const int ntiles = i / tile + 1;
    const int L = min(S, ntiles * tile);           // elements this row loads (kept tiles)
    const uint16_t *srow = s + row * (int64_t)S;
    OutT *orow = out + row * (int64_t)S;

    float v[NCH][8];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = c * kChunk + lane * 8;
        if (j0 < L) {
            float f[8];
            unpack8(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(srow + j0)), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float z = (j0 + e <= i) ? f[e] * k2 : -INFINITY;   // log2-domain logit
                v[c][e] = z;
                m = fmaxf(m, z);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = -INFINITY;
        }
    }
    m = wave_max(m);                                // finite: key 0 is always kept
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(v[c][e] - m);  // exp2(-inf) = 0 for masked keys
            v[c][e] = p;
            sum += p;
        }
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = c * kChunk + lane * 8;
        if (j0 < S) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = (j0 < L) ? v[c][e] * inv : 0.0f;
            store8(orow + j0, f);
        }
    }
    if (COUNT && lane == 0) tiles[row] = ntiles;
}

// Generic form (any S): element loads, three sweeps over the kept tiles
// (max, sum, write).  Used when S is not a multiple of 8 or exceeds the
// register-resident limit.
template <typename OutT, bool COUNT>
__global__ __launch_bounds__(kSmBlock) void softmax_fused_generic_kernel(
    const uint16_t *__restrict__ s, OutT *__restrict__ out, int64_t rows, int S, float k2,
    int tile, int32_t *__restrict__ tiles)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % S);
    const int ntiles = i / tile + 1;
    const int L = min(S, ntiles * tile);
    const uint16_t *srow = s + row * (int64_t)S;
    OutT *orow = out + row * (int64_t)S;
    float m = -INFINITY;
    for (int j = lane; j < L; j += 64) {
        const float z = (j <= i) ? bf16_lo(srow[j]) * k2 : -INFINITY;
        m = fmaxf(m, z);
    }
    m = wave_max(m);
    float sum = 0.0f;
    for (int j = lane; j < L; j += 64)
        if (j <= i) sum += fast_exp2(bf16_lo(srow[j]) * k2 - m);
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
    for (int j = lane; j < S; j += 64) {
        const float p = (j <= i) ? fast_exp2(bf16_lo(srow[j]) * k2 - m) * inv : 0.0f;
        store1(orow + j, p);
    }
    if (COUNT && lane == 0) tiles[row] = ntiles;
}

template <typename OutT, bool COUNT>
static int launch_fused(const uint16_t *s, OutT *out, int64_t rows, int S, float scale, int tile,
                        int32_t *tiles, hipStream_t st)
{
    const float k2 = scale * kLog2e;
    const int64_t grid = ceil_div(rows, kRowsPerBlock);
    if (grid > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    const int nch = (int)ceil_div(S, kChunk);
    if (S % 8 != 0 || nch > kMaxRegChunks) {
        softmax_fused_generic_kernel<OutT, COUNT><<<(int)grid, kSmBlock, 0, st>>>(s, out, rows, S, k2,
                                                                                 tile, tiles);
        return launch_status();
    }
#define FC_SM_CASE(NC)                                                                           \
    case NC:                                                                                     \
        softmax_fused_kernel<NC, OutT, COUNT><<<(int)grid, kSmBlock, 0, st>>>(s, out, rows, S, k2, \
                                                                             tile, tiles);       \
        break;
    switch (nch) {
        FC_SM_CASE(1) FC_SM_CASE(2) FC_SM_CASE(3) FC_SM_CASE(4) FC_SM_CASE(5) FC_SM_CASE(6)
        FC_SM_CASE(7) FC_SM_CASE(8) FC_SM_CASE(9) FC_SM_CASE(10) FC_SM_CASE(11) FC_SM_CASE(12)
        FC_SM_CASE(13) FC_SM_CASE(14) FC_SM_CASE(15) FC_SM_CASE(16)
    default: return FC_ERR_UNSUPPORTED;
    }
#undef FC_SM_CASE
    return launch_status();
}

// ------------------------------------------------------------------ unfused

// Row-loop helper: calls f(j, 8 values) over 8-wide chunks when S % 8 == 0,
// else element by element.
#define FC_ROW_VEC(S) (((S) & 7) == 0)

// (1) row max of scale*s over the keys the row keeps (j <= i, from the
// indices).  The whole row is read, as the step's byte count has it; taking
// the max over kept keys only keeps every exp(x) of a kept key <= 1 whatever
// the masked scores hold (a masked score far above the kept ones would
// otherwise underflow every kept exponential).
__global__ __launch_bounds__(kSmBlock) void um_rowmax_kernel(const uint16_t *__restrict__ s,
                                                             float *__restrict__ rmax, int64_t rows,
                                                             int S, float scale)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % S);
    const uint16_t *p = s + row * (int64_t)S;
    float m = -INFINITY;
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            float f[8];
            unpack8(*reinterpret_cast<const u32x4 *>(p + j0), f);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (j0 + e <= i) m = fmaxf(m, f[e] * scale);
        }
    } else {
        for (int j = lane; j < S; j += 64)
            if (j <= i) m = fmaxf(m, bf16_lo(p[j]) * scale);
    }
    m = wave_max(m);
    if (lane == 0) rmax[row] = m;
}

// (2) x = scale*s - max  -> out (bf16)
__global__ __launch_bounds__(kSmBlock) void um_sub_kernel(const uint16_t *__restrict__ s,
                                                          uint16_t *__restrict__ out,
                                                          const float *__restrict__ rmax,
                                                          int64_t rows, int S, float scale)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t *p = s + row * (int64_t)S;
    uint16_t *q = out + row * (int64_t)S;
    const float m = rmax[row];
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            float f[8];
            unpack8(*reinterpret_cast<const u32x4 *>(p + j0), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = f[e] * scale - m;
            store8(q + j0, f);
        }
    } else {
        for (int j = lane; j < S; j += 64) store1(q + j, bf16_lo(p[j]) * scale - m);
    }
}

// (3) e = exp(x) where the mask is 1, else 0 (in place in out).  The mask
// selects rather than multiplies: x of a masked key may be large, and
// exp(x) * 0 would be NaN once exp(x) overflows.
__global__ __launch_bounds__(kSmBlock) void um_expmask_kernel(uint16_t *__restrict__ out,
                                                              const uint16_t *__restrict__ mask,
                                                              int64_t rows, int S)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    uint16_t *q = out + row * (int64_t)S;
    const uint16_t *mk = mask + row * (int64_t)S;
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            float f[8], g[8];
            unpack8(*reinterpret_cast<const u32x4 *>(q + j0), f);
            unpack8(*reinterpret_cast<const u32x4 *>(mk + j0), g);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = g[e] != 0.0f ? fast_exp2(f[e] * kLog2e) : 0.0f;
            store8(q + j0, f);
        }
    } else {
        for (int j = lane; j < S; j += 64)
            store1(q + j, bf16_lo(mk[j]) != 0.0f ? fast_exp2(bf16_lo(q[j]) * kLog2e) : 0.0f);
    }
}

// (4) row sum of e
__global__ __launch_bounds__(kSmBlock) void um_rowsum_kernel(const uint16_t *__restrict__ out,
                                                             float *__restrict__ rsum, int64_t rows,
                                                             int S)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t *q = out + row * (int64_t)S;
    float acc = 0.0f;
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            float f[8];
            unpack8(*reinterpret_cast<const u32x4 *>(q + j0), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += f[e];
        }
    } else {
        for (int j = lane; j < S; j += 64) acc += bf16_lo(q[j]);
    }
    acc = wave_sum(acc);
    if (lane == 0) rsum[row] = acc;
}

// (5) out = e / sum
__global__ __launch_bounds__(kSmBlock) void um_div_kernel(uint16_t *__restrict__ out,
                                                          const float *__restrict__ rsum,
                                                          int64_t rows, int S)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    uint16_t *q = out + row * (int64_t)S;
    const float l = rsum[row];
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            float f[8];
            unpack8(*reinterpret_cast<const u32x4 *>(q + j0), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = f[e] / l;
            store8(q + j0, f);
        }
    } else {
        for (int j = lane; j < S; j += 64) store1(q + j, bf16_lo(q[j]) / l);
    }
}

// Causal mask [BH, S, S]: bf16 1.0 where key j <= query i, else 0.
__global__ __launch_bounds__(kSmBlock) void mask_kernel(uint16_t *__restrict__ mask, int64_t rows,
                                                        int S)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % S);
    uint16_t *q = mask + row * (int64_t)S;
    const uint16_t one = 0x3f80;   // bf16 1.0
    if (FC_ROW_VEC(S)) {
        for (int j0 = lane * 8; j0 < S; j0 += kChunk) {
            u32x4 w;
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (j0 + e <= i) ? one : 0u;
            w.x = h[0] | (h[1] << 16);
            w.y = h[2] | (h[3] << 16);
            w.z = h[4] | (h[5] << 16);
            w.w = h[6] | (h[7] << 16);
            *reinterpret_cast<u32x4 *>(q + j0) = w;
        }
    } else {
        for (int j = lane; j < S; j += 64) q[j] = (j <= i) ? one : (uint16_t)0;
    }
}

static size_t mask_region_bytes(int64_t BH, int S)
{
    size_t b = (size_t)BH * (size_t)S * (size_t)S * 2;
    return (b + 255) & ~(size_t)255;
}

static bool tile_ok(int tile, int S) { return tile == 64 || tile == 128 || tile == 256 || tile == S; }

static int common_checks(const void *scores, const void *out, int64_t BH, int S, size_t out_elem)
{
    if (BH < 1 || S < 1) return FC_ERR_SHAPE;
    if (!scores || !out) return FC_ERR_NULL;
    if (!aligned16(scores) || !aligned16(out)) return FC_ERR_ALIGN;
    const size_t n = (size_t)BH * (size_t)S * (size_t)S;
    if (overlaps(scores, n * 2, out, n * out_elem)) return FC_ERR_ALIAS;
    return FC_OK;
}

}  // namespace fc

using namespace fc;

extern "C" size_t fc_softmax_workspace_bytes(int64_t BH, int S, int mode)
{
    if (BH < 1 || S < 1 || mode != FC_SOFTMAX_UNFUSED) return 0;
    return mask_region_bytes(BH, S) + 8 * (size_t)BH * (size_t)S;
}

extern "C" int fc_causal_mask_materialise(uint16_t *mask, int64_t BH, int S, fc_stream stream)
{
    if (BH < 1 || S < 1) return FC_ERR_SHAPE;
    if (!mask) return FC_ERR_NULL;
    if (!aligned16(mask)) return FC_ERR_ALIGN;
    const int64_t rows = BH * (int64_t)S;
    const int64_t grid = ceil_div(rows, kRowsPerBlock);
    if (grid > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    mask_kernel<<<(int)grid, kSmBlock, 0, reinterpret_cast<hipStream_t>(stream)>>>(mask, rows, S);
    return launch_status();
}

extern "C" int fc_causal_softmax(const uint16_t *scores, uint16_t *out, int64_t BH, int S,
                                 float scale, int tile, int mode, void *workspace, size_t ws_bytes,
                                 fc_stream stream)
{
    int rc = common_checks(scores, out, BH, S, 2);
    if (rc != FC_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t rows = BH * (int64_t)S;
    if (mode == FC_SOFTMAX_FUSED) {
        if (!tile_ok(tile, S)) return FC_ERR_UNSUPPORTED;
        return launch_fused<uint16_t, false>(scores, out, rows, S, scale, tile, nullptr, st);
    }
    if (mode != FC_SOFTMAX_UNFUSED) return FC_ERR_UNSUPPORTED;
    const size_t need = fc_softmax_workspace_bytes(BH, S, mode);
    if (!workspace || ws_bytes < need) return FC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FC_ERR_ALIGN;
    const size_t n = (size_t)rows * (size_t)S;
    if (overlaps(workspace, need, scores, n * 2) || overlaps(workspace, need, out, n * 2))
        return FC_ERR_ALIAS;
    const int64_t grid = ceil_div(rows, kRowsPerBlock);
    if (grid > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    const uint16_t *mask = static_cast<const uint16_t *>(workspace);
    float *rmax = reinterpret_cast<float *>(static_cast<char *>(workspace) + mask_region_bytes(BH, S));
    float *rsum = rmax + rows;
    const int g = (int)grid;
    um_rowmax_kernel<<<g, kSmBlock, 0, st>>>(scores, rmax, rows, S, scale);
    if ((rc = launch_status()) != FC_OK) return rc;
    um_sub_kernel<<<g, kSmBlock, 0, st>>>(scores, out, rmax, rows, S, scale);
    if ((rc = launch_status()) != FC_OK) return rc;
    um_expmask_kernel<<<g, kSmBlock, 0, st>>>(out, mask, rows, S);
    if ((rc = launch_status()) != FC_OK) return rc;
    um_rowsum_kernel<<<g, kSmBlock, 0, st>>>(out, rsum, rows, S);
    if ((rc = launch_status()) != FC_OK) return rc;
    um_div_kernel<<<g, kSmBlock, 0, st>>>(out, rsum, rows, S);
    return launch_status();
}

extern "C" int fc_causal_softmax_f32out(const uint16_t *scores, float *out, int64_t BH, int S,
                                        float scale, int tile, fc_stream stream)
{
    int rc = common_checks(scores, out, BH, S, 4);
    if (rc != FC_OK) return rc;
    if (!tile_ok(tile, S)) return FC_ERR_UNSUPPORTED;
    return launch_fused<float, false>(scores, out, BH * (int64_t)S, S, scale, tile, nullptr,
                                      reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fc_causal_softmax_tiles(const uint16_t *scores, uint16_t *out, int32_t *tiles_per_row,
                                       int64_t BH, int S, float scale, int tile, fc_stream stream)
{
    int rc = common_checks(scores, out, BH, S, 2);
    if (rc != FC_OK) return rc;
    if (!tiles_per_row) return FC_ERR_NULL;
    if (!tile_ok(tile, S)) return FC_ERR_UNSUPPORTED;
    return launch_fused<uint16_t, true>(scores, out, BH * (int64_t)S, S, scale, tile, tiles_per_row,
                                        reinterpret_cast<hipStream_t>(stream));
}
