// fp16 GEMM with a bias + erf-GELU + residual epilogue cut by a split plan
// ("K4 讲解：fusion 的三笔账", section 1: the chain mm -> bias -> gelu -> res and
// its four split plans; every segment is one kernel).
//
// First segment: MFMA GEMM (v_mfma_f32_32x32x16_f16, fp32 accumulate) with the
// segment's epilogue operators applied to the accumulator registers before the
// single fp16 store.  Later segments: pointwise kernels over the fp16 [M,N]
// intermediate (128-bit loads/stores).
//
// GEMM data flow: A [M,K] and B [K,N] are row-major.  Each workgroup owns a
// BM x BN output tile; K advances in BK slabs through a two-stage LDS ring.
// A slabs are copied as-is (k contiguous).  B slabs are loaded as 8x8 fp16
// blocks, transposed in registers and stored n-major, so both MFMA operands
// are read from LDS as 16-byte k-contiguous fragments.  Rows of LDS are padded
// by 16 bytes, which spreads the 16-byte fragment reads across all banks.
#include "fc_internal.h"

namespace fc {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Epilogue operators applied after the GEMM, in chain order.
enum { OP_BIAS = 1, OP_GELU = 2, OP_RES = 3 };

__device__ __forceinline__ float gelu_erf(float z)
{
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// Apply chain operators FIRST..LAST (1 = bias, 2 = gelu, 3 = residual).
template <int FIRST, int LAST>
__device__ __forceinline__ float apply_ops(float v, float bias, float res)
{
    if (FIRST <= OP_BIAS && OP_BIAS <= LAST) v += bias;
    if (FIRST <= OP_GELU && OP_GELU <= LAST) v = gelu_erf(v);
    if (FIRST <= OP_RES && OP_RES <= LAST) v += res;
    return v;
}

// ------------------------------------------------------------------ MFMA GEMM

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;                    // threads
    static constexpr int WTM = BM / WM, WTN = BN / WN;         // wave tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;         // 32x32 MFMA tiles per wave
    static constexpr int LDK = BK + 8;                         // padded LDS row (halfs)
    static constexpr int A_CHUNKS = BM * BK / 8;               // 16-byte chunks of an A slab
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);       // 8x8 blocks of a B slab
    static constexpr int B_PER_T = (B_BLOCKS + NT - 1) / NT;
    static constexpr int LDS_A = BM * LDK, LDS_B = BN * LDK;   // halfs per stage
    static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tiles are 32x32 multiples");
    static_assert(BK % 16 == 0, "BK is a multiple of the MFMA k (16)");
};

template <class C>
struct Prefetch {
    u32x4 a[C::A_PER_T];
    u32x4 b[C::B_PER_T][8];
};

template <class C>
__device__ __forceinline__ void load_slab(Prefetch<C> &pf, const uint16_t *__restrict__ A,
                                          const uint16_t *__restrict__ B, int M, int N, int K,
                                          int m0, int n0, int k0)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int c = t + i * C::NT;
        const int row = c / (C::BK / 8), kc = (c % (C::BK / 8)) * 8;
        const int gm = m0 + row, gk = k0 + kc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c < C::A_CHUNKS && gm < M && gk < K)
            v = *reinterpret_cast<const u32x4 *>(A + (int64_t)gm * K + gk);
        pf.a[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int blk = t + i * C::NT;
        const int kb = blk % (C::BK / 8), nb = blk / (C::BK / 8);
        const int gk = k0 + kb * 8, gn = n0 + nb * 8;
        const bool ok = blk < C::B_BLOCKS && gk < K && gn < N;   // K, N multiples of 8
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = *reinterpret_cast<const u32x4 *>(B + (int64_t)(gk + r) * N + gn);
            pf.b[i][r] = v;
        }
    }
}

// 8x8 fp16 block: rows r (k), 4 dwords each holding column pairs (2q, 2q+1).
// Output column c as 4 dwords holding row pairs (2p, 2p+1).
__device__ __forceinline__ u32x4 transpose_col(const u32x4 rows[8], int c)
{
    const int q = c >> 1;
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t lo = rows[2 * p][q], hi = rows[2 * p + 1][q];
        o[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    return o;
}

template <class C>
__device__ __forceinline__ void store_slab(const Prefetch<C> &pf, uint16_t *As, uint16_t *Bs)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int c = t + i * C::NT;
        if (c < C::A_CHUNKS) {
            const int row = c / (C::BK / 8), kc = (c % (C::BK / 8)) * 8;
            *reinterpret_cast<u32x4 *>(As + row * C::LDK + kc) = pf.a[i];
        }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int blk = t + i * C::NT;
        if (blk < C::B_BLOCKS) {
            const int kb = blk % (C::BK / 8), nb = blk / (C::BK / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<u32x4 *>(Bs + (nb * 8 + c) * C::LDK + kb * 8) =
                    transpose_col(pf.b[i], c);
        }
    }
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs; the remap gives each XCD a contiguous run of logical tile ids, and the
// grouped order (GROUP_M tile rows, column-major inside the group) makes that
// run a compact rectangle, so the A and B panels it reads are shared in the
// XCD's own L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int kXcds = 8, kGroupM = 4;
    const int G = gridDim.x;
    int bid = blockIdx.x;
    if (G % kXcds == 0) bid = (bid % kXcds) * (G / kXcds) + bid / kXcds;
    const int group = kGroupM * tiles_n;
    const int first_m = (bid / group) * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in = bid % group;
    tm = first_m + in % gm;
    tn = in / gm;
}

template <class C, int LAST>
__global__ __launch_bounds__(C::NT) void gemm_epi_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::LDS_A + C::LDS_B)];
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Prefetch<C> pf;
    const int nk = (K + C::BK - 1) / C::BK;
    load_slab<C>(pf, A, B, M, N, K, m0, n0, 0);
    store_slab<C>(pf, lds, lds + C::LDS_A);
    __syncthreads();

    // fragment coordinates inside the stage (halfs)
    const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const uint16_t *As = lds + cur * (C::LDS_A + C::LDS_B);
        const uint16_t *Bs = As + C::LDS_A;
        if (kt + 1 < nk) load_slab<C>(pf, A, B, M, N, K, m0, n0, (kt + 1) * C::BK);
#pragma unroll
        for (int kk = 0; kk < C::BK; kk += 16) {
            f16x8 a[C::TM], b[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                a[i] = *reinterpret_cast<const f16x8 *>(
                    As + (wm * C::WTM + i * 32 + frag_row) * C::LDK + kk + frag_k);
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                b[j] = *reinterpret_cast<const f16x8 *>(
                    Bs + (wn * C::WTN + j * 32 + frag_row) * C::LDK + kk + frag_k);
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            uint16_t *Asn = lds + (cur ^ 1) * (C::LDS_A + C::LDS_B);
            store_slab<C>(pf, Asn, Asn + C::LDS_A);
        }
        __syncthreads();
    }

    // Epilogue on the accumulators.  32x32 MFMA result layout: lane l holds
    // column (l % 32) and rows 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * C::WTN + j * 32 + (lane & 31);
            if (col >= N) continue;
            const float bv = (LAST >= OP_BIAS) ? h2f(bias[col]) : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M) {
                    const int64_t o = (int64_t)row * N + col;
                    const float rv = (LAST >= OP_RES) ? h2f(R[o]) : 0.0f;
                    out[o] = f2h(apply_ops<OP_BIAS, LAST>(acc[i][j][r], bv, rv));
                }
            }
        }
    }
}

// ------------------------------------------------------------------ skinny GEMM (M <= 16)

// Decode shape: one workgroup per 16-column strip of the output; its waves
// split K, each accumulating a 16x16 tile with v_mfma_f32_16x16x32_f16, then
// the partial tiles are summed through LDS and the epilogue is applied before
// the single store.  The whole plan segment stays one launch.
template <int WAVES>
__device__ __forceinline__ void skinny_partial(const uint16_t *__restrict__ A,
                                               const uint16_t *__restrict__ B, int M, int N, int K,
                                               int n0, f32x4 &acc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 16x16x32 operand layout: lane l supplies row/column (l % 16) and
    // k = 8*(l/16) .. 8*(l/16)+7 of a 32-deep k step.
    const int rc = lane & 15, kq = (lane >> 4) * 8;
    const int col = n0 + rc;
    const bool col_ok = col < N;
    const bool row_ok = rc < M;
    const int ksteps = (K + 31) / 32;
    for (int ks = wave; ks < ksteps; ks += WAVES) {
        const int k = ks * 32 + kq;
        f16x8 a, b;
        if (row_ok && k < K) {
            a = *reinterpret_cast<const f16x8 *>(A + (int64_t)rc * K + k);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (_Float16)0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool ok = col_ok && (k + e) < K;
            b[e] = ok ? __builtin_bit_cast(_Float16, B[(int64_t)(k + e) * N + col]) : (_Float16)0.0f;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
}

template <int WAVES, int LAST>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K)
{
    __shared__ float part[WAVES][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    skinny_partial<WAVES>(A, B, M, N, K, n0, acc);
    // 16x16 result layout: lane l holds column (l % 16), rows 4*(l/16) + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += WAVES * 64) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += part[w][e];
        const int row = e >> 4, col = n0 + (e & 15);
        if (row < M && col < N) {
            const int64_t o = (int64_t)row * N + col;
            const float bv = (LAST >= OP_BIAS) ? h2f(bias[col]) : 0.0f;
            const float rv = (LAST >= OP_RES) ? h2f(R[o]) : 0.0f;
            out[o] = f2h(apply_ops<OP_BIAS, LAST>(v, bv, rv));
        }
    }
}

// ------------------------------------------------------------------ pointwise segments

// Operators FIRST..LAST on an fp16 [M,N] intermediate; out may equal in.
template <int FIRST, int LAST>
__global__ __launch_bounds__(256) void epi_pointwise_kernel(const uint16_t *in,
                                                            const uint16_t *__restrict__ bias,
                                                            const uint16_t *__restrict__ R,
                                                            uint16_t *out, int64_t chunks, int N)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += stride) {
        const int64_t e0 = c * 8;
        const int col0 = (int)(e0 % N);                  // N % 8 == 0: a chunk stays in one row
        const u32x4 v = *reinterpret_cast<const u32x4 *>(in + e0);
        u32x4 bw = {0u, 0u, 0u, 0u}, rw = {0u, 0u, 0u, 0u};
        if (FIRST <= OP_BIAS && OP_BIAS <= LAST) bw = *reinterpret_cast<const u32x4 *>(bias + col0);
        if (FIRST <= OP_RES && OP_RES <= LAST) rw = *reinterpret_cast<const u32x4 *>(R + e0);
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = apply_ops<FIRST, LAST>(f16_lo(v[q]), f16_lo(bw[q]), f16_lo(rw[q]));
            const float hi = apply_ops<FIRST, LAST>(f16_hi(v[q]), f16_hi(bw[q]), f16_hi(rw[q]));
            o[q] = pack_f16x2(lo, hi);
        }
        *reinterpret_cast<u32x4 *>(out + e0) = o;
    }
}

// ------------------------------------------------------------------ host

using CfgBig = GemmCfg<256, 256, 64, 2, 2>;     // 4 waves, 128x128 per wave
using CfgMid = GemmCfg<128, 128, 64, 2, 2>;     // 4 waves, 64x64 per wave
constexpr int kSkinnyWaves = 8;

template <class C, int LAST>
static int launch_gemm_cfg(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                           const uint16_t *R, uint16_t *out, int M, int N, int K, hipStream_t s)
{
    const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t grid = (int64_t)tiles_m * tiles_n;
    if (grid > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    gemm_epi_kernel<C, LAST><<<(int)grid, C::NT, 0, s>>>(A, B, bias, R, out, M, N, K, tiles_m, tiles_n);
    return launch_status();
}

template <int LAST>
static int launch_gemm(const uint16_t *A, const uint16_t *B, const uint16_t *bias, const uint16_t *R,
                       uint16_t *out, int M, int N, int K, hipStream_t s)
{
    if (M <= 16) {
        gemm_skinny_kernel<kSkinnyWaves, LAST><<<(N + 15) / 16, kSkinnyWaves * 64, 0, s>>>(
            A, B, bias, R, out, M, N, K);
        return launch_status();
    }
    // large problems: 256x256 tiles; smaller ones: 128x128 (more workgroups)
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= 128) return launch_gemm_cfg<CfgBig, LAST>(A, B, bias, R, out, M, N, K, s);
    return launch_gemm_cfg<CfgMid, LAST>(A, B, bias, R, out, M, N, K, s);
}

static int launch_gemm_segment(int last, const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                               const uint16_t *R, uint16_t *out, int M, int N, int K, hipStream_t s)
{
    switch (last) {
    case 0: return launch_gemm<0>(A, B, bias, R, out, M, N, K, s);
    case 1: return launch_gemm<1>(A, B, bias, R, out, M, N, K, s);
    case 2: return launch_gemm<2>(A, B, bias, R, out, M, N, K, s);
    case 3: return launch_gemm<3>(A, B, bias, R, out, M, N, K, s);
    default: return FC_ERR_PLAN;
    }
}

template <int FIRST, int LAST>
static int launch_pw(const uint16_t *in, const uint16_t *bias, const uint16_t *R, uint16_t *out,
                     int64_t MN, int N, hipStream_t s)
{
    const int64_t chunks = MN / 8;
    int64_t grid = ceil_div(chunks, 256 * 4);
    if (grid < 1) grid = 1;
    if (grid > 65536) grid = 65536;
    epi_pointwise_kernel<FIRST, LAST><<<(int)grid, 256, 0, s>>>(in, bias, R, out, chunks, N);
    return launch_status();
}

static int launch_pointwise(int first, int last, const uint16_t *in, const uint16_t *bias,
                            const uint16_t *R, uint16_t *out, int64_t MN, int N, hipStream_t s)
{
    const int key = first * 4 + last;
    switch (key) {
    case 1 * 4 + 1: return launch_pw<1, 1>(in, bias, R, out, MN, N, s);
    case 1 * 4 + 2: return launch_pw<1, 2>(in, bias, R, out, MN, N, s);
    case 1 * 4 + 3: return launch_pw<1, 3>(in, bias, R, out, MN, N, s);
    case 2 * 4 + 2: return launch_pw<2, 2>(in, bias, R, out, MN, N, s);
    case 2 * 4 + 3: return launch_pw<2, 3>(in, bias, R, out, MN, N, s);
    case 3 * 4 + 3: return launch_pw<3, 3>(in, bias, R, out, MN, N, s);
    default: return FC_ERR_PLAN;
    }
}

static bool plan_valid(const int *plan, int plan_len)
{
    if (!plan || plan_len < 1 || plan_len > 4) return false;
    int sum = 0;
    for (int i = 0; i < plan_len; ++i) {
        if (plan[i] <= 0) return false;
        sum += plan[i];
    }
    return sum == 4;
}

}  // namespace fc

using namespace fc;

extern "C" size_t fc_gemm_workspace_bytes(int M, int N, int K, const int *plan, int plan_len)
{
    (void)K;
    if (!plan_valid(plan, plan_len) || M < 1 || N < 1) return 0;
    return plan_len > 1 ? 2 * (size_t)M * (size_t)N : 0;
}

extern "C" int fc_gemm_epilogue(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                                const uint16_t *R, uint16_t *Y, int M, int N, int K,
                                const int *plan, int plan_len, void *workspace, size_t ws_bytes,
                                fc_stream stream)
{
    if (!plan_valid(plan, plan_len)) return FC_ERR_PLAN;
    if (M < 1 || N < 1 || K < 1) return FC_ERR_SHAPE;
    if (N % 8 != 0 || K % 8 != 0) return FC_ERR_UNSUPPORTED;
    if (!A || !B || !bias || !R || !Y) return FC_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(bias) || !aligned16(R) || !aligned16(Y))
        return FC_ERR_ALIGN;
    const size_t mn = (size_t)M * N * 2;
    if (overlaps(Y, mn, A, (size_t)M * K * 2) || overlaps(Y, mn, B, (size_t)K * N * 2) ||
        overlaps(Y, mn, bias, (size_t)N * 2) || overlaps(Y, mn, R, mn))
        return FC_ERR_ALIAS;
    const size_t need = fc_gemm_workspace_bytes(M, N, K, plan, plan_len);
    uint16_t *ws = static_cast<uint16_t *>(workspace);
    if (need) {
        if (!workspace || ws_bytes < need) return FC_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FC_ERR_ALIGN;
        if (overlaps(ws, need, A, (size_t)M * K * 2) || overlaps(ws, need, B, (size_t)K * N * 2) ||
            overlaps(ws, need, bias, (size_t)N * 2) || overlaps(ws, need, R, mn) ||
            overlaps(ws, need, Y, mn))
            return FC_ERR_ALIAS;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // operators: 0 = mm, 1 = bias, 2 = gelu, 3 = residual
    int first = 0;
    for (int seg = 0; seg < plan_len; ++seg) {
        const int last = first + plan[seg] - 1;
        uint16_t *dst = (seg == plan_len - 1) ? Y : ws;
        int rc;
        if (seg == 0)
            rc = launch_gemm_segment(last, A, B, bias, R, dst, M, N, K, s);
        else
            rc = launch_pointwise(first, last, ws, bias, R, dst, (int64_t)M * N, N, s);
        if (rc != FC_OK) return rc;
        first = last + 1;
    }
    return FC_OK;
}
