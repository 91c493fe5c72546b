// fp16 GEMM with a bias + erf-GELU + residual epilogue cut by a split plan
// ("K4 讲解：fusion 的三笔账", section 1: the chain mm -> bias -> gelu -> res and
// its four split plans; every segment is one kernel).
//
// First segment: MFMA GEMM (v_mfma_f32_32x32x16_f16, fp32 accumulate) with the
// segment's epilogue operators applied to the accumulator registers before the
// single fp16 store.  Later segments: pointwise kernels over the fp16 [M,N]
// intermediate (128-bit loads/stores).
//
// Kernels, by shape: M <= 64 with N % 64 == 0 and K % 256 == 0 runs the
// split-K gemm_decode_kernel; with K % 64 == 0, large problems (more than 512
// tiles of 128x128) run gemm_ring_kernel (loads straight into a 4-stage LDS ring, B
// fragments by the transposing LDS read; see its own comment) and the rest
// gemm_ring128_kernel (the same on 128x128 tiles, K split when the tiles are
// few); other K run register-staged kernels (gemm_big_kernel, gemm_epi_kernel)
// and, for M <= 16 without a decode split, gemm_skinny_kernel.
//
// Register-staged data flow: A [M,K] and B [K,N] are row-major.  Each
// workgroup owns a BM x BN output tile; K advances in BK slabs through a
// two-stage LDS ring.  A slabs are copied as-is (k contiguous).  B slabs are
// loaded as 8x8 fp16 blocks, transposed in registers and stored n-major, so
// both MFMA operands are read from LDS as 16-byte k-contiguous fragments.
// Rows of LDS are padded by 16 bytes, which spreads the 16-byte fragment reads
// across all banks.
#include "fc_internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

// The split-K handoffs of gemm_ring128_kernel and gemm_decode_kernel publish
// fp32 partials and count arrivals without release/acquire fences (those
// write back and invalidate a whole XCD's L2 per workgroup).  They rely on
// the memory model of the gfx9 family as gfx950 implements it; see the
// comment at the first handoff.  Another target needs that argument redone.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "gemm.hip is written for gfx950: its split-K handoff relies on that ISA's memory model"
#endif

namespace fc {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Epilogue operators applied after the GEMM, in chain order.
enum { OP_BIAS = 1, OP_GELU = 2, OP_RES = 3 };

// GELU in erf form, z * Phi(z), Phi the standard normal CDF.  With
// h = erfc(|z| / sqrt 2) / 2, Phi(z) is 1 - h for z >= 0 and h for z < 0, so
//   GELU(z) = max(z, 0) - |z| h,
// one max and one fma after h (relative accuracy of h carries into the
// negative tail, where the result is tiny).  erfc by the Chebyshev fit of
// Press et al., Numerical Recipes, section 6.2 (erfcc): for x >= 0 and
// t = 1/(1 + x/2), erfc(x) = t exp(-x^2 - 1.26551223 + t(1.00002368 + ...)),
// relative error below 1.2e-7.  Here x = |z| / sqrt 2, so t = 1/(1 + |z|/(2 sqrt 2))
// and -x^2 = -z^2 / 2; the exponential is taken in base 2 with log2(e) folded
// into the fit's coefficients and the factor 1/2 of h folded into its
// constant term (minus 1 in the exponent): h = t * 2^(C(t) - z^2 log2(e) / 2),
// C_i = log2(e) c_i (C_0 = log2(e) c_0 - 1).  15 vector instructions and two
// transcendentals per element.
__device__ __forceinline__ float gelu_erf(float z)
{
    const float a = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(a, 0.35355338f, 1.0f));
    float p = 0.24651730f;
    p = __builtin_fmaf(p, t, -1.18611491f);
    p = __builtin_fmaf(p, t, 2.14747453f);
    p = __builtin_fmaf(p, t, -1.63775313f);
    p = __builtin_fmaf(p, t, 0.40232158f);
    p = __builtin_fmaf(p, t, -0.26875687f);
    p = __builtin_fmaf(p, t, 0.13963005f);
    p = __builtin_fmaf(p, t, 0.53970063f);
    p = __builtin_fmaf(p, t, 1.44272923f);
    p = __builtin_fmaf(p, t, -2.82574821f);
    const float h = t * __builtin_amdgcn_exp2f(__builtin_fmaf(z * -0.72134751f, z, p));
    return __builtin_fmaf(-a, h, fmaxf(z, 0.0f));
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

// ------------------------------------------------------------------ large-tile GEMM (8 waves)

// 256x256x64 workgroup tile, 8 waves (two per SIMD) each owning a 128x64
// slice (4x2 MFMA 32x32x16 tiles, 128 fp32 accumulators).  Two waves per SIMD
// let the hardware issue one wave's MFMAs while the other waits on LDS or the
// barrier.  Per k16 step a wave reads 6 fragments and issues 8 MFMAs; the
// fragments for the next step are read while the current MFMAs run
// (double-buffered fragment registers, interleaving pinned with
// sched_group_barrier).  The MFMA operands are swapped (B fragment first), so
// the result tile is C^T in MFMA layout: lane l owns row m = l % 32 and four
// consecutive columns per register quad, giving 8-byte R loads and Y stores.
namespace big {
constexpr int BM = 256, BN = 256, BK = 64, NT = 512, LDK = BK + 8;
constexpr int WN = 4;                        // wave grid 2 (M) x 4 (N)
constexpr int WTM = 128, WTN = 64;
constexpr int TM = WTM / 32, TN = WTN / 32;  // 4 x 2 MFMA tiles per wave
constexpr int STAGE = (BM + BN) * LDK;       // halfs per LDS stage
constexpr int KSTEPS = BK / 16;
}  // namespace big

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct BigPrefetch {
    u32x4 a[4];   // 4 A chunks of 8 halfs
    u32x4 b[4];   // 4 rows (k) x 8 columns (n) of a B block
    bool aok[4];  // chunk inside the matrix (only consulted when CHECKED)
    bool bok;
};

// Global -> registers.  Addresses are clamped into the matrix, so every load
// is valid; chunks outside are zeroed later, at store time, so no wait on the
// loaded data is forced here.  Requires K, N % 8 == 0.
template <bool CHECKED>
__device__ __forceinline__ void big_load(BigPrefetch &pf, const uint16_t *__restrict__ A,
                                         const uint16_t *__restrict__ B, int M, int N, int K,
                                         int m0, int n0, int k0)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * big::NT;
        const int gm = m0 + (c >> 3), gk = k0 + (c & 7) * 8;
        pf.aok[i] = gm < M && gk < K;
        pf.a[i] = *reinterpret_cast<const u32x4 *>(A + (int64_t)min(gm, M - 1) * K + min(gk, K - 8));
    }
    const int blk = t >> 1, h = t & 1;
    const int kb = blk & 7, nb = blk >> 3;
    const int gk = k0 + kb * 8 + h * 4, gn = n0 + nb * 8;
    pf.bok = (k0 + kb * 8) < K && gn < N;
    const int gnc = min(gn, N - 8);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        pf.b[r] = *reinterpret_cast<const u32x4 *>(B + (int64_t)min(gk + r, K - 1) * N + gnc);
}

// Registers -> LDS.  A chunks go k-contiguous; the 4x8 B block is transposed
// into 8 columns of 4 k-values (one 8-byte write each).
template <bool CHECKED>
__device__ __forceinline__ void big_store(const BigPrefetch &pf, uint16_t *As, uint16_t *Bs)
{
    const int t = threadIdx.x;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + i * big::NT;
        *reinterpret_cast<u32x4 *>(As + (c >> 3) * big::LDK + (c & 7) * 8) =
            (!CHECKED || pf.aok[i]) ? pf.a[i] : zero;
    }
    u32x4 b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        b[r] = pf.b[r];
        // opaque redefinition: keeps the transpose below (pure VALU) from being
        // hoisted next to the global load, which would force an early wait
        asm volatile("" : "+v"(b[r]));
        b[r] = (!CHECKED || pf.bok) ? b[r] : zero;
    }
    const int blk = t >> 1, h = t & 1;
    const int kb = blk & 7, nb = blk >> 3;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int q = c >> 1;
        u32x2 o;
        if (c & 1) {
            o.x = (b[0][q] >> 16) | (b[1][q] & 0xffff0000u);
            o.y = (b[2][q] >> 16) | (b[3][q] & 0xffff0000u);
        } else {
            o.x = (b[0][q] & 0xffffu) | (b[1][q] << 16);
            o.y = (b[2][q] & 0xffffu) | (b[3][q] << 16);
        }
        *reinterpret_cast<u32x2 *>(Bs + (nb * 8 + c) * big::LDK + kb * 8 + h * 4) = o;
    }
}

__device__ __forceinline__ void big_frags(const uint16_t *As, const uint16_t *Bs, int kk, int wm,
                                          int wn, f16x8 fa[big::TM], f16x8 fb[big::TN])
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, kq = (lane >> 5) * 8 + kk * 16;
#pragma unroll
    for (int i = 0; i < big::TM; ++i)
        fa[i] = *reinterpret_cast<const f16x8 *>(As + (wm * big::WTM + i * 32 + r) * big::LDK + kq);
#pragma unroll
    for (int j = 0; j < big::TN; ++j)
        fb[j] = *reinterpret_cast<const f16x8 *>(Bs + (wn * big::WTN + j * 32 + r) * big::LDK + kq);
}

template <int LAST, bool CHECKED>
__global__ __launch_bounds__(big::NT, 1) void gemm_big_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * big::STAGE];
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * big::BM, n0 = tn * big::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / big::WN, wn = wave % big::WN;

    f32x16 acc[big::TM][big::TN];
#pragma unroll
    for (int i = 0; i < big::TM; ++i)
#pragma unroll
        for (int j = 0; j < big::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    BigPrefetch pf;
    f16x8 fa[2][big::TM], fb[2][big::TN];
    const int nk = (K + big::BK - 1) / big::BK;
    big_load<CHECKED>(pf, A, B, M, N, K, m0, n0, 0);
    big_store<CHECKED>(pf, lds, lds + big::BM * big::LDK);
    __syncthreads();
    big_frags(lds, lds + big::BM * big::LDK, 0, wm, wn, fa[0], fb[0]);

    // Branch-free body: the last iteration's prefetch reads clamped (valid)
    // addresses and lands in the stage no wave reads any more.
    for (int kt = 0; kt < nk; ++kt) {
        const uint16_t *As = lds + (kt & 1) * big::STAGE;
        const uint16_t *Bs = As + big::BM * big::LDK;
        uint16_t *An = lds + ((kt & 1) ^ 1) * big::STAGE;
        big_load<CHECKED>(pf, A, B, M, N, K, m0, n0, (kt + 1) * big::BK);
        // Each k16 step is its own scheduling region (sched_barrier fences):
        // its 8 independent MFMAs interleave with the fragment reads of the
        // next step (and, in step 0, the next slab's global loads; in step 3,
        // its LDS writes), so no MFMA waits on a fragment read just issued.
#pragma unroll
        for (int kk = 0; kk < big::KSTEPS; ++kk) {
            const int c = kk & 1;
            if (kk + 1 < big::KSTEPS) big_frags(As, Bs, kk + 1, wm, wn, fa[c ^ 1], fb[c ^ 1]);
#pragma unroll
            for (int i = 0; i < big::TM; ++i)
#pragma unroll
                for (int j = 0; j < big::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
            if (kk == 0) {
#pragma unroll
                for (int s = 0; s < 6; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            } else if (kk + 1 < big::KSTEPS) {
#pragma unroll
                for (int s = 0; s < 6; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            } else {
                big_store<CHECKED>(pf, An, An + big::BM * big::LDK);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        big_frags(An, An + big::BM * big::LDK, 0, wm, wn, fa[0], fb[0]);
    }

    // Epilogue.  acc[i][j] holds C^T: lane owns m = (lane % 32) of tile row i
    // and, for register quad g, columns 8g + 4*(lane/32) .. +3 of tile column j.
#pragma unroll
    for (int i = 0; i < big::TM; ++i) {
        const int m = m0 + wm * big::WTM + i * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < big::TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * big::WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= N) continue;                   // N % 8 == 0: n..n+3 all valid
                const int64_t o = (int64_t)m * N + n;
                u32x2 bw = {0u, 0u}, rw = {0u, 0u};
                if (LAST >= OP_BIAS) bw = *reinterpret_cast<const u32x2 *>(bias + n);
                if (LAST >= OP_RES) rw = *reinterpret_cast<const u32x2 *>(R + o);
                u32x2 y;
                y.x = pack_f16x2(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 0], f16_lo(bw.x), f16_lo(rw.x)),
                                 apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 1], f16_hi(bw.x), f16_hi(rw.x)));
                y.y = pack_f16x2(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 2], f16_lo(bw.y), f16_lo(rw.y)),
                                 apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 3], f16_hi(bw.y), f16_hi(rw.y)));
                *reinterpret_cast<u32x2 *>(out + o) = y;
            }
        }
    }
}

// ------------------------------------------------------------------ ring GEMM (direct-to-LDS, 4 stages)

// 256x256 workgroup tile, 8 waves (two per SIMD) each owning 128x64 (4x2
// MFMA 32x32x16 tiles), K in 32-deep slabs through a 4-stage LDS ring.
// Slabs are copied global -> LDS by buffer loads with the LDS destination
// (each lane's 16 bytes land at M0 + 16*lane), issued three slabs ahead, so
// no registers stage the data and HBM latency is covered by three k-steps of
// MFMAs.  The main loop spends no vector instructions on addresses: the
// loads take lane-constant byte offsets computed once (the slab enters as a
// scalar offset for A and as the scalar base of B's buffer descriptor), and
// the fragment reads take lane-constant LDS addresses with the stage in the
// instruction's offset field (the loop is unrolled over the four stages).
// Layouts are XOR-swizzled so every fragment read is bank-conflict free:
//   A stages (4 x 16 KiB from byte 0): [256 rows][32 k] fp16, 64-byte rows,
//            16-byte k-unit u stored at u ^ ((row >> 2) & 3); fragments are
//            ds_read_b128.
//   B stages (4 x 16 KiB from byte 64 KiB): [32 k][256 n] fp16 (B's own
//            row-major layout), 32-byte n-unit v stored at v ^ (2 * (k & 3));
//            fragments are k-contiguous by the transposing read
//            ds_read_b64_tr_b16: within a group of 16 lanes, lane j addresses
//            B[k0 + j/4][n0 + 4(j%4) .. +3] and lane i gets B[k0 .. k0+3][n0 + i].
// A whole k-step of fragments is double-buffered in registers.  Fragment
// reads are inline asm: the compiler cannot prove they miss the in-flight
// direct-to-LDS writes and would drain all loads before each read; ordering is
// instead explicit (vmcnt wait for the slab's own loads, then a barrier), and
// frag_wait*() ties the fragment registers to an lgkmcnt wait before use.
// Epilogue: on an interior tile the fp32 accumulators pass through the freed
// ring (128 rows at a time) into a row-major layout, so bias, GELU and the
// residual run on 8 consecutive columns per lane and R and Y move 16 bytes per
// lane (bit-identical to applying them in the accumulator layout, and 2-5 %
// faster at 4096^3: two 512-byte row pieces per wave instruction instead of
// 8-byte pieces in 32 rows).
// Needs K % 64 == 0 (an even number of slabs), K <= 2^22 and N <= 2^24 (the
// lane offsets are 32-bit); M and N tails read clamped rows/columns whose
// results are never stored.
namespace ring {
constexpr int BM = 256, BN = 256, BK = 32, NT = 512, S = 4, WN = 4;
constexpr int SLAB = BM * BK * 2;            // 16 KiB: one A slab, and one B slab (BN == BM)
constexpr int BREG = S * SLAB;               // the B stages start at 64 KiB
constexpr int ROWB = BN * 2;                 // bytes per B k-row in LDS
constexpr int MAX_K = 1 << 22, MAX_N = 1 << 24;
// buffer descriptor word 3 for raw 32-bit-format dword loads
constexpr int RSRC_WORD3 = 0x00020000;
}  // namespace ring

#define FC_LDS __attribute__((address_space(3)))
#define FC_GLB __attribute__((address_space(1)))

__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr)
{
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
template <int OFF>
__device__ __forceinline__ f16x8 ring_read_b128(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
    f16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x2 ring_read_tr16(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// f(integral_constant<int, I>) for I = 0 .. N-1, so loop indices can be template arguments
template <int I, int N, class F>
__device__ __forceinline__ void ring_static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        ring_static_for<I + 1, N>(f);
    }
}

// One k-step's fragments: A [k16][4 tiles], B [k16][2 tiles][2 halves of 4 k].
struct RingFrags {
    f16x8 a[2][4];
    u32x2 b[2][2][2];
};
// Reads are issued k16-step 0 first; LDS returns in issue order, so
// lgkmcnt(8) covers step 0 and lgkmcnt(0) covers both.
__device__ __forceinline__ void frag_wait0(RingFrags &f)
{
    asm volatile("s_waitcnt lgkmcnt(8)"
                 : "+v"(f.a[0][0]), "+v"(f.a[0][1]), "+v"(f.a[0][2]), "+v"(f.a[0][3]),
                   "+v"(f.b[0][0][0]), "+v"(f.b[0][0][1]), "+v"(f.b[0][1][0]), "+v"(f.b[0][1][1]));
}
__device__ __forceinline__ void frag_wait1(RingFrags &f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[1][0]), "+v"(f.a[1][1]), "+v"(f.a[1][2]), "+v"(f.a[1][3]),
                   "+v"(f.b[1][0][0]), "+v"(f.b[1][0][1]), "+v"(f.b[1][1][0]), "+v"(f.b[1][1][1]));
}
__device__ __forceinline__ f16x8 ring_bfrag(const RingFrags &f, int kk, int j)
{
    const u32x4 w = {f.b[kk][j][0].x, f.b[kk][j][0].y, f.b[kk][j][1].x, f.b[kk][j][1].y};
    return __builtin_bit_cast(f16x8, w);
}

template <int LAST>
__global__ __launch_bounds__(ring::NT, 1) void gemm_ring_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char lds_raw[2 * ring::BREG];
    FC_LDS char *lds = (FC_LDS char *)lds_raw;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * ring::BM, n0 = tn * ring::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / ring::WN, wn = wave % ring::WN;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / ring::BK;                 // even
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // fragment addresses in stage 0 of the A and B regions
    uint32_t fa[2][4], fb[2][2][2];
    {
        const int r = lane & 31, g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int u = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + i * 32 + r;
                fa[kk][i] = lds0 + row * 64 + (u ^ ((row >> 2) & 3)) * 16;
            }
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const int v = (wn * 64 + jt * 32 + 16 * (g & 1)) >> 4;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = kk * 16 + 8 * (g >> 1) + 4 * hh + (j >> 2);
                    fb[kk][jt][hh] = lds0 + ring::BREG + k * ring::ROWB + (v ^ (2 * (k & 3))) * 32 + (j & 3) * 8;
                }
            }
        }
    }
    // This wave's 2 A blocks (16 rows each) and 2 B blocks (2 k-rows each) of
    // every slab, 1 KiB per load instruction: lane byte offsets into the
    // workgroup's A panel (rows from m0, clamped to M-1; the slab adds 2*k0)
    // and into one B slab (k-rows from k0, columns from n0 clamped to N-8).
    uint32_t la[2], lb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int blk = wave * 2 + q;
        const int row = blk * 16 + (lane >> 2);
        const int u = (lane & 3) ^ ((lane >> 4) & 3);      // logical k-unit of this lane's slot
        const int gm = min(m0 + row, M - 1);
        la[q] = (uint32_t)((gm - m0) * K + u * 8) * 2u;
        const int krow = blk * 2 + (lane >> 5);
        const int p = (lane & 31) >> 1, half = lane & 1;  // physical 32-byte unit, 16-byte half
        const int v = p ^ (2 * (krow & 3));
        const int gn = min(n0 + v * 16 + half * 8, N - 8);
        lb[q] = (uint32_t)(krow * N + (gn - n0)) * 2u;
    }
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * K), (short)0, 0x7fffffff, ring::RSRC_WORD3);
    // load X of slab `slab` into stage ST (X = 0..3: A block X/2 when X is
    // even, B block X/2 when odd)
    auto issue1 = [&](int slab, auto stage, auto xc) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value, X = decltype(xc)::value, q = X >> 1;
        const int k0 = slab * ring::BK;
        const int blk = wave_s * 2 + q;
        if constexpr ((X & 1) == 0) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (FC_LDS void *)(lds + ST * ring::SLAB + blk * 1024),
                                                     16, la[q], k0 * 2, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(B + (int64_t)k0 * N + n0), (short)0, 0x7fffffff, ring::RSRC_WORD3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (FC_LDS void *)(lds + ring::BREG + ST * ring::SLAB + blk * 1024), 16, lb[q], 0, 0, 0);
        }
    };
    auto issue = [&](int slab, auto stage) __attribute__((always_inline)) {
        ring_static_for<0, 4>([&](auto xc) __attribute__((always_inline)) { issue1(slab, stage, xc); });
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(min(1, nk - 1), std::integral_constant<int, 1>{});
    issue(min(2, nk - 1), std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_waitcnt(0xF78);           // vmcnt(8): slab 0 of this wave landed
    __builtin_amdgcn_s_barrier();                // ... and of every wave
    RingFrags F[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) F[0].a[kk][i] = ring_read_b128<0>(fa[kk][i]);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) F[0].b[kk][jt][hh] = ring_read_tr16<0>(fb[kk][jt][hh]);
    }
    // k-step tt; H = tt % 4 (the loop base is a multiple of 4), so the stage
    // read now is H, the one read next H+1 and the one loaded now H+3 (mod 4)
    auto step = [&](int tt, auto hc) __attribute__((always_inline)) {
        constexpr int H = decltype(hc)::value, cb = H & 1, nb = cb ^ 1;
        constexpr int SNEXT = ((H + 1) & 3) * ring::SLAB, SLOAD = (H + 3) & 3;
        frag_wait0(F[cb]);
        __builtin_amdgcn_sched_barrier(0);
        // The first k16-step's 8 MFMAs, one of the wave's 4 loads of slab tt+3
        // after every second: issued in one burst after the MFMAs, the loads of
        // all waves queue together and stall the MFMA issue (1,127 vs 1,066
        // cycles per k-step; 0.9 % less time, the clock falls with the denser
        // MFMA issue).  Slab tt+3 goes to the stage read for step tt-1:
        // every wave read its fragments for step tt-1 during step tt-2 and
        // waited for all of them before the barrier of step tt-1; past the end
        // a clamped re-read lands in a stage that is never read.
        const int lslab = min(tt + ring::S - 1, nk - 1);
        ring_static_for<0, 8>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value, i = q >> 1, j = q & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring_bfrag(F[cb], 0, j), F[cb].a[0][i], acc[i][j],
                                                               0, 0, 0);
            if constexpr ((q & 1) != 0)
                issue1(lslab, std::integral_constant<int, SLOAD>{}, std::integral_constant<int, (q >> 1)>{});
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_waitcnt(0xF78);       // vmcnt(8): slab tt+1 of this wave landed
        frag_wait1(F[cb]);                       // every fragment read of stage tt done
        __builtin_amdgcn_s_barrier();            // ... in every wave, and slab tt+1 landed
        __builtin_amdgcn_sched_barrier(0);
        ring_static_for<0, 8>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value, i = q >> 1, j = q & 1;
            constexpr int kk = q >> 2, rr = q & 3;   // next step's k16-step-0 frags first
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring_bfrag(F[cb], 1, j), F[cb].a[1][i], acc[i][j],
                                                               0, 0, 0);
            F[nb].a[kk][rr] = ring_read_b128<SNEXT>(fa[kk][rr]);
            F[nb].b[kk][rr >> 1][rr & 1] = ring_read_tr16<SNEXT>(fb[kk][rr >> 1][rr & 1]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int t = 0;
    for (; t + 4 <= nk; t += 4) {
        step(t + 0, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
        step(t + 2, std::integral_constant<int, 2>{});
        step(t + 3, std::integral_constant<int, 3>{});
    }
    if (t < nk) {                                // nk % 4 == 2
        step(t + 0, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0xF70);           // drain the clamped prefetches
    frag_wait0(F[0]);
    frag_wait1(F[0]);

    if (m0 + ring::BM <= M && n0 + ring::BN <= N) {
        // Interior tile: the accumulators go through LDS, half a tile (128 rows
        // x 256 columns of fp32, 128 KiB, the ring's space) at a time, so that
        // every lane then owns 8 consecutive columns of a row: its bias values
        // once, and R loads and Y stores of 16 bytes, a wave covering two
        // 512-byte row pieces per instruction (in the accumulator layout a
        // wave's 8-byte accesses touch 32 rows each).  LDS: row r at r * 1 KiB,
        // 16-byte unit u at u ^ ((u >> 4) & 1) ^ (r & 63): 16 lanes writing one
        // unit of 16 rows, or reading units 2c (or 2c + 1) of one row, cover all
        // 16 bank groups (no conflicts).  Same arithmetic per element as the
        // accumulator-layout path.  R and Y are touched once: streaming
        // (nontemporal) loads and stores (4096 x 4096 x 512: 3.4 % faster,
        // 4096^3 1.1-1.6 %).
        __syncthreads();                         // every wave is done with the ring
        FC_LDS float *sh = (FC_LDS float *)lds;
        const int rl = lane >> 5, cu = lane & 31;
        const int col = 8 * cu;                  // the lane's 8 columns of the tile
        float bv[8];
        {
            u32x4 bw = {0u, 0u, 0u, 0u};
            if (LAST >= OP_BIAS) bw = *reinterpret_cast<const u32x4 *>(bias + n0 + col);
            bv[0] = f16_lo(bw.x); bv[1] = f16_hi(bw.x); bv[2] = f16_lo(bw.y); bv[3] = f16_hi(bw.y);
            bv[4] = f16_lo(bw.z); bv[5] = f16_hi(bw.z); bv[6] = f16_lo(bw.w); bv[7] = f16_hi(bw.w);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // rows of the half tile this lane finishes: q * 16 + 2 * wave + rl
            const int64_t rbase = (int64_t)(m0 + 128 * p + 2 * wave + rl) * N + n0 + col;
            u32x4 rw[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                rw[q] = u32x4{0u, 0u, 0u, 0u};
                if (LAST >= OP_RES) rw[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(R + rbase + (int64_t)q * 16 * N));
            }
            if (wm == p) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int r = 32 * i + (lane & 31);
                            const int u = 16 * wn + 8 * j + 2 * g + rl;
                            const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                             acc[i][j][4 * g + 3]};
                            *(FC_LDS f32x4 *)(sh + r * 256 + ((u ^ ((u >> 4) & 1) ^ (r & 63)) << 2)) = v;
                        }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = q * 16 + 2 * wave + rl;
                const int u0 = 2 * cu, u1 = 2 * cu + 1;
                const f32x4 x0 = *(const FC_LDS f32x4 *)(sh + r * 256 + ((u0 ^ ((u0 >> 4) & 1) ^ (r & 63)) << 2));
                const f32x4 x1 = *(const FC_LDS f32x4 *)(sh + r * 256 + ((u1 ^ ((u1 >> 4) & 1) ^ (r & 63)) << 2));
                u32x4 y;
                y.x = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x0.x, bv[0], f16_lo(rw[q].x)),
                                     apply_ops<OP_BIAS, LAST>(x0.y, bv[1], f16_hi(rw[q].x)));
                y.y = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x0.z, bv[2], f16_lo(rw[q].y)),
                                     apply_ops<OP_BIAS, LAST>(x0.w, bv[3], f16_hi(rw[q].y)));
                y.z = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x1.x, bv[4], f16_lo(rw[q].z)),
                                     apply_ops<OP_BIAS, LAST>(x1.y, bv[5], f16_hi(rw[q].z)));
                y.w = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x1.z, bv[6], f16_lo(rw[q].w)),
                                     apply_ops<OP_BIAS, LAST>(x1.w, bv[7], f16_hi(rw[q].w)));
                __builtin_nontemporal_store(y, reinterpret_cast<u32x4 *>(out + rbase + (int64_t)q * 16 * N));
            }
            if (p == 0) __syncthreads();         // the next half overwrites what was just read
        }
        return;
    }
    // Tiles with an M or N tail: straight from the accumulators (C^T layout:
    // lane owns row m = lane % 32 of tile row i and columns 8g + 4*(lane/32)
    // .. +3 of tile column j), every store checked.
    float bf[2][4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * 64 + j * 32 + 8 * g + 4 * (lane >> 5);
            u32x2 bw = {0u, 0u};
            if (LAST >= OP_BIAS && n < N) bw = *reinterpret_cast<const u32x2 *>(bias + n);
            bf[j][g][0] = f16_lo(bw.x);
            bf[j][g][1] = f16_hi(bw.x);
            bf[j][g][2] = f16_lo(bw.y);
            bf[j][g][3] = f16_hi(bw.y);
        }
    auto out4 = [&](int i, int j, int g, u32x2 rw) __attribute__((always_inline)) {
        u32x2 y;
        y.x = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 0], bf[j][g][0], f16_lo(rw.x)),
                             apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 1], bf[j][g][1], f16_hi(rw.x)));
        y.y = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 2], bf[j][g][2], f16_lo(rw.y)),
                             apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 3], bf[j][g][3], f16_hi(rw.y)));
        return y;
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 64 + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= N) continue;
                const int64_t o = (int64_t)m * N + n;
                u32x2 rw = {0u, 0u};
                if (LAST >= OP_RES) rw = *reinterpret_cast<const u32x2 *>(R + o);
                *reinterpret_cast<u32x2 *>(out + o) = out4(i, j, g, rw);
            }
        }
    }
}

// ------------------------------------------------------------------ ring GEMM, 128x128 tiles

// gemm_ring_kernel's dataflow on a quarter of its tile, for problems with too
// few 256x256 tiles to fill the chip: 4 waves (2 x 2, each 64 x 64 as 2 x 2
// MFMA tiles), a 4-stage LDS ring of 8 KiB A and 8 KiB B slabs (64 KiB, two
// workgroups per CU), each wave loading 2 A and 2 B blocks of 1 KiB per slab,
// fragment addresses computed once (the stage in the offset field).  When
// even these tiles are too few, K is split over blockIdx.y: each split
// publishes its fp32 partial tile (64 KiB, in register order, so every access
// is coalesced and the summing workgroup finds each value in the register it
// left) with device-scope stores and takes a ticket; the workgroup that draws
// the last ticket sums the P partials in split order and applies the
// epilogue.  The partial of a 128x128 tile is a quarter of a 256x256 one, so
// that last workgroup reads little.
namespace r128 {
constexpr int BM = 128, BN = 128, BK = 32, NT = 256, S = 4, WN = 2;
constexpr int SLAB = BM * BK * 2;            // 8 KiB: one A slab, and one B slab
constexpr int BREG = S * SLAB;               // the B stages start at 32 KiB
constexpr int ROWB = BN * 2;                 // bytes per B k-row in LDS
}

// One k-step's fragments: A [k16][2 tiles], B [k16][2 tiles][2 halves of 4 k].
struct Ring128Frags {
    f16x8 a[2][2];
    u32x2 b[2][2][2];
};
// Reads are issued k16-step 0 first (6 of them), then step 1.
__device__ __forceinline__ void r128_wait0(Ring128Frags &f)
{
    asm volatile("s_waitcnt lgkmcnt(6)"
                 : "+v"(f.a[0][0]), "+v"(f.a[0][1]), "+v"(f.b[0][0][0]), "+v"(f.b[0][0][1]), "+v"(f.b[0][1][0]),
                   "+v"(f.b[0][1][1]));
}
__device__ __forceinline__ void r128_wait1(Ring128Frags &f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[1][0]), "+v"(f.a[1][1]), "+v"(f.b[1][0][0]), "+v"(f.b[1][0][1]), "+v"(f.b[1][1][0]),
                   "+v"(f.b[1][1][1]));
}
__device__ __forceinline__ f16x8 r128_bfrag(const Ring128Frags &f, int kk, int j)
{
    const u32x4 w = {f.b[kk][j][0].x, f.b[kk][j][0].y, f.b[kk][j][1].x, f.b[kk][j][1].y};
    return __builtin_bit_cast(f16x8, w);
}

template <int LAST>
__global__ __launch_bounds__(r128::NT, 2) void gemm_ring128_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n, int P, uint32_t *__restrict__ counters,
    float *__restrict__ partials)
{
    __shared__ __attribute__((aligned(1024))) char lds_raw[2 * r128::BREG];
    __shared__ int is_last;
    FC_LDS char *lds = (FC_LDS char *)lds_raw;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * r128::BM, n0 = tn * r128::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / r128::WN, wn = wave % r128::WN;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // split blockIdx.y of P takes k-rows kofs .. kofs + K/P - 1
    const int split = blockIdx.y, kofs = split * (K / P);
    const int nk = K / P / r128::BK;             // even
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // fragment addresses in stage 0 (A: [128 rows][32 k], 16-byte k-units
    // swizzled by row; B: [32 k][128 n], 32-byte n-units swizzled by k)
    uint32_t fa[2][2], fb[2][2][2];
    {
        const int r = lane & 31, g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int u = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + r;
                fa[kk][i] = lds0 + row * 64 + (u ^ ((row >> 2) & 3)) * 16;
            }
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const int v = (wn * 64 + jt * 32 + 16 * (g & 1)) >> 4;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = kk * 16 + 8 * (g >> 1) + 4 * hh + (j >> 2);
                    fb[kk][jt][hh] = lds0 + r128::BREG + k * r128::ROWB + (v ^ (2 * (k & 3))) * 32 + (j & 3) * 8;
                }
            }
        }
    }
    // This wave's 2 A blocks (16 rows each) and 2 B blocks (4 k-rows each) of
    // every slab: lane byte offsets into the workgroup's A panel (rows from
    // m0, clamped to M-1; the slab adds 2*k0) and into one B slab (k-rows from
    // k0, columns from n0 clamped to N-8).
    uint32_t la[2], lb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int blk = wave * 2 + q;
        const int row = blk * 16 + (lane >> 2);
        const int u = (lane & 3) ^ ((lane >> 4) & 3);      // logical k-unit of this lane's slot
        const int gm = min(m0 + row, M - 1);
        la[q] = (uint32_t)((gm - m0) * K + u * 8) * 2u;
        const int krow = blk * 4 + (lane >> 4);
        const int p = (lane & 15) >> 1, half = lane & 1;  // physical 32-byte unit, 16-byte half
        const int v = p ^ (2 * (krow & 3));
        const int gn = min(n0 + v * 16 + half * 8, N - 8);
        lb[q] = (uint32_t)(krow * N + (gn - n0)) * 2u;
    }
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * K), (short)0, 0x7fffffff, ring::RSRC_WORD3);
    auto issue = [&](int slab, auto stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        const int k0 = kofs + slab * r128::BK;
        const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(B + (int64_t)k0 * N + n0), (short)0, 0x7fffffff, ring::RSRC_WORD3);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int blk = wave_s * 2 + q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (FC_LDS void *)(lds + ST * r128::SLAB + blk * 1024),
                                                     16, la[q], k0 * 2, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (FC_LDS void *)(lds + r128::BREG + ST * r128::SLAB + blk * 1024), 16, lb[q], 0, 0, 0);
        }
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(min(1, nk - 1), std::integral_constant<int, 1>{});
    issue(min(2, nk - 1), std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_waitcnt(0xF78);           // vmcnt(8): slab 0 of this wave landed
    __builtin_amdgcn_s_barrier();                // ... and of every wave
    Ring128Frags F[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) F[0].a[kk][i] = ring_read_b128<0>(fa[kk][i]);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) F[0].b[kk][jt][hh] = ring_read_tr16<0>(fb[kk][jt][hh]);
    }
    // k-step tt; H = tt % 4, so the stage read now is H, the one read next
    // H+1 and the one loaded now H+3 (mod 4)
    auto step = [&](int tt, auto hc) __attribute__((always_inline)) {
        constexpr int H = decltype(hc)::value, cb = H & 1, nb = cb ^ 1;
        constexpr int SNEXT = ((H + 1) & 3) * r128::SLAB, SLOAD = (H + 3) & 3;
        r128_wait0(F[cb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r128_bfrag(F[cb], 0, j), F[cb].a[0][i],
                                                                   acc[i][j], 0, 0, 0);
        // slab tt+3 goes to the stage read for step tt-1, which every wave
        // finished reading before the barrier of step tt-1; past the end a
        // clamped re-read lands in a stage that is never read.  (Spreading the
        // four loads between these MFMAs, as the 256x256 kernel does, was 2.7 %
        // slower here: this kernel's LDS port is the busier one.)
        issue(min(tt + r128::S - 1, nk - 1), std::integral_constant<int, SLOAD>{});
        __builtin_amdgcn_s_waitcnt(0xF78);       // vmcnt(8): slab tt+1 of this wave landed
        r128_wait1(F[cb]);                       // every fragment read of stage tt done
        __builtin_amdgcn_s_barrier();            // ... in every wave, and slab tt+1 landed
        __builtin_amdgcn_sched_barrier(0);
        // the second k16-step's 4 MFMAs, each followed by 3 of the next
        // step's 12 fragment reads (its k16-step 0 first)
        ring_static_for<0, 4>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value, i = q >> 1, j = q & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r128_bfrag(F[cb], 1, j), F[cb].a[1][i], acc[i][j],
                                                               0, 0, 0);
            ring_static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int rr = 3 * q + decltype(rc)::value, kk = rr / 6, x = rr % 6;
                if constexpr (x < 2)
                    F[nb].a[kk][x] = ring_read_b128<SNEXT>(fa[kk][x]);
                else
                    F[nb].b[kk][(x - 2) >> 1][(x - 2) & 1] =
                        ring_read_tr16<SNEXT>(fb[kk][(x - 2) >> 1][(x - 2) & 1]);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int t = 0;
    for (; t + 4 <= nk; t += 4) {
        step(t + 0, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
        step(t + 2, std::integral_constant<int, 2>{});
        step(t + 3, std::integral_constant<int, 3>{});
    }
    if (t < nk) {                                // nk % 4 == 2
        step(t + 0, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0xF70);           // drain the clamped prefetches
    r128_wait0(F[0]);
    r128_wait1(F[0]);
    r128_wait0(F[1]);
    r128_wait1(F[1]);

    if (P > 1) {
        const int tile = tm * tiles_n + tn;
        uint64_t *mine = reinterpret_cast<uint64_t *>(partials) + ((int64_t)tile * P + split) * 16 * 256 * 2 +
                         2 * threadIdx.x;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const f32x16 &a = acc[v >> 3][(v >> 2) & 1];
            const int q = v & 3;
            __hip_atomic_store(mine + v * 512, __builtin_bit_cast(uint64_t, make_float2(a[4 * q], a[4 * q + 1])),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + v * 512 + 1,
                               __builtin_bit_cast(uint64_t, make_float2(a[4 * q + 2], a[4 * q + 3])),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // Handoff without fences.  What it relies on (gfx9 family, gfx950):
        //  1. an agent-scope atomic store is a global store with the device
        //     scope bit set: it writes through this XCD's L2 to the device
        //     coherence point, and its completion is acknowledged from there;
        //  2. on gfx9 the vector memory counter also counts stores (there is no
        //     separate store counter), so s_waitcnt vmcnt(0) returns only once
        //     every partial store of this thread is complete at that point;
        //  3. the barrier after the wait orders every thread's completed stores
        //     before thread 0's ticket, an agent-scope atomic performed at the
        //     same coherence point;
        //  4. the last workgroup reads partials with agent-scope atomic loads,
        //     which bypass its own XCD's L2 and read the coherence point, so
        //     they cannot hit a stale line.
        // A compiler that moved a store past the wait, or a target without (1)
        // or (2), would break this silently; the guard at the top of the file
        // keeps other targets out.
        __builtin_amdgcn_s_waitcnt(0xF70);       // vmcnt(0): the partial is at the coherence point
        __syncthreads();
        if (threadIdx.x == 0)
            is_last = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)(P - 1);
        __syncthreads();
        if (!is_last) return;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        const uint64_t *base = reinterpret_cast<const uint64_t *>(partials) + (int64_t)tile * P * 16 * 256 * 2 +
                               2 * threadIdx.x;
        for (int p = 0; p < P; ++p) {
            const uint64_t *src = base + (int64_t)p * 16 * 256 * 2;
#pragma unroll
            for (int v0 = 0; v0 < 16; v0 += 8) {
                uint64_t w[8][2];
#pragma unroll
                for (int dv = 0; dv < 8; ++dv) {
                    w[dv][0] = __hip_atomic_load(src + (v0 + dv) * 512, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    w[dv][1] =
                        __hip_atomic_load(src + (v0 + dv) * 512 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int dv = 0; dv < 8; ++dv) {
                    const int v = v0 + dv, q = v & 3;
                    f32x16 &a = acc[v >> 3][(v >> 2) & 1];
                    const float2 lo = __builtin_bit_cast(float2, w[dv][0]), hi = __builtin_bit_cast(float2, w[dv][1]);
                    a[4 * q] += lo.x;
                    a[4 * q + 1] += lo.y;
                    a[4 * q + 2] += hi.x;
                    a[4 * q + 3] += hi.y;
                }
            }
        }
        if (threadIdx.x == 0) __hip_atomic_store(counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    if (m0 + r128::BM <= M && n0 + r128::BN <= N) {
        // Interior tile: as the 256x256 kernel, the accumulators pass through
        // the freed ring (the whole 128x128 fp32 tile, 64 KiB, one pass) into a
        // row-major layout; a lane then finishes 8 consecutive columns of a
        // row with 16-byte R loads and Y stores (streaming, as in
        // gemm_ring_kernel).  Row r at r * 512 bytes, 16-byte unit u at
        // u ^ ((u >> 4) & 1) ^ (r & 31) (no bank conflicts).
        __syncthreads();                         // every wave is done with the ring
        FC_LDS float *sh = (FC_LDS float *)lds;
        const int rq = threadIdx.x >> 4, cu = threadIdx.x & 15;   // 16 rows x 16 lanes per pass of q
        const int col = 8 * cu;
        float bv[8];
        {
            u32x4 bw = {0u, 0u, 0u, 0u};
            if (LAST >= OP_BIAS) bw = *reinterpret_cast<const u32x4 *>(bias + n0 + col);
            bv[0] = f16_lo(bw.x); bv[1] = f16_hi(bw.x); bv[2] = f16_lo(bw.y); bv[3] = f16_hi(bw.y);
            bv[4] = f16_lo(bw.z); bv[5] = f16_hi(bw.z); bv[6] = f16_lo(bw.w); bv[7] = f16_hi(bw.w);
        }
        const int64_t rbase = (int64_t)(m0 + rq) * N + n0 + col;
        u32x4 rw[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            rw[q] = u32x4{0u, 0u, 0u, 0u};
            if (LAST >= OP_RES) rw[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(R + rbase + (int64_t)q * 16 * N));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r = wm * 64 + 32 * i + (lane & 31);
                    const int u = 16 * wn + 8 * j + 2 * g + (lane >> 5);
                    const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    *(FC_LDS f32x4 *)(sh + r * 128 + ((u ^ ((u >> 4) & 1) ^ (r & 31)) << 2)) = v;
                }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = q * 16 + rq;
            const int u0 = 2 * cu, u1 = 2 * cu + 1;
            const f32x4 x0 = *(const FC_LDS f32x4 *)(sh + r * 128 + ((u0 ^ ((u0 >> 4) & 1) ^ (r & 31)) << 2));
            const f32x4 x1 = *(const FC_LDS f32x4 *)(sh + r * 128 + ((u1 ^ ((u1 >> 4) & 1) ^ (r & 31)) << 2));
            u32x4 y;
            y.x = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x0.x, bv[0], f16_lo(rw[q].x)),
                                 apply_ops<OP_BIAS, LAST>(x0.y, bv[1], f16_hi(rw[q].x)));
            y.y = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x0.z, bv[2], f16_lo(rw[q].y)),
                                 apply_ops<OP_BIAS, LAST>(x0.w, bv[3], f16_hi(rw[q].y)));
            y.z = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x1.x, bv[4], f16_lo(rw[q].z)),
                                 apply_ops<OP_BIAS, LAST>(x1.y, bv[5], f16_hi(rw[q].z)));
            y.w = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(x1.z, bv[6], f16_lo(rw[q].w)),
                                 apply_ops<OP_BIAS, LAST>(x1.w, bv[7], f16_hi(rw[q].w)));
            __builtin_nontemporal_store(y, reinterpret_cast<u32x4 *>(out + rbase + (int64_t)q * 16 * N));
        }
        return;
    }
    // Tiles with an M or N tail: straight from the accumulators (C^T layout:
    // lane owns row m = lane % 32 of tile row i and columns 8g + 4*(lane/32)
    // .. +3 of tile column j), every store checked.
    float bf[2][4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * 64 + j * 32 + 8 * g + 4 * (lane >> 5);
            u32x2 bw = {0u, 0u};
            if (LAST >= OP_BIAS && n < N) bw = *reinterpret_cast<const u32x2 *>(bias + n);
            bf[j][g][0] = f16_lo(bw.x);
            bf[j][g][1] = f16_hi(bw.x);
            bf[j][g][2] = f16_lo(bw.y);
            bf[j][g][3] = f16_hi(bw.y);
        }
    auto out4 = [&](int i, int j, int g, u32x2 rw) __attribute__((always_inline)) {
        u32x2 y;
        y.x = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 0], bf[j][g][0], f16_lo(rw.x)),
                             apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 1], bf[j][g][1], f16_hi(rw.x)));
        y.y = pack_f16x2_rne(apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 2], bf[j][g][2], f16_lo(rw.y)),
                             apply_ops<OP_BIAS, LAST>(acc[i][j][4 * g + 3], bf[j][g][3], f16_hi(rw.y)));
        return y;
    };
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + i * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 64 + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= N) continue;
                const int64_t o = (int64_t)m * N + n;
                u32x2 rw = {0u, 0u};
                if (LAST >= OP_RES) rw = *reinterpret_cast<const u32x2 *>(R + o);
                *reinterpret_cast<u32x2 *>(out + o) = out4(i, j, g, rw);
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

// ------------------------------------------------------------------ decode GEMM (M <= 64, split K)

// At M <= 64 the GEMM is a stream over B (K x N fp16), so the layout is
// chosen for the stream: every workgroup owns a 64-column strip of B (one
// full 128-byte line per k-row) and a 1/P share of K, and requests its whole
// slab (at most 1024 k-rows, 128 KiB) at once with direct-to-LDS loads; its 8
// waves each take a contiguous eighth of the slab and read only what they
// loaded, so no barrier sits between the loads and the MFMAs.  B slab layout
// per wave: k-row k at 128 k bytes, 16-byte unit u at u ^ dec_swz(k), which
// spreads the transposing reads (ds_read_b64_tr_b16, four k-rows per
// 16-lane group) over all banks.  A fragments (MB blocks of 16 rows x the
// wave's k-range) go straight to registers.  Per 32-deep k-step and 16-column
// tile, one B fragment read feeds one v_mfma_f32_16x16x32_f16 per row block,
// so B leaves LDS once whatever M is.
//
// The eight wave partials are summed through LDS in wave order, one 16-row
// block at a time.  With P = 1 the workgroup applies the epilogue and stores
// Y.  With P > 1 it publishes its MB x 16 x 64 fp32 partial to the workspace
// and takes a ticket from the strip's arrival counter; the workgroup that
// draws the last ticket sums the P partials in split order (so the result
// does not depend on arrival order), applies the epilogue, stores Y and puts
// the counter back to zero.  No workgroup ever waits for another, so the
// launch needs no co-residency.
//
// Visibility across XCDs without a full L2 write-back: partials are written
// with device-scope stores (they write through to the device coherence point
// and count as complete only once there), every thread waits for its stores
// before the workgroup barrier that precedes the ticket, and the last
// workgroup reads the partials with device-scope loads, which are served from
// the coherence point rather than a possibly stale line of its own XCD's L2.
namespace dec {
constexpr int WAVES = 8, NT = WAVES * 64, W = 64, ROW = W * 2, KSTEP = 32;
constexpr int TILE = 16 * W;                                     // outputs per strip and 16-row block
constexpr int MAXMB = 4;                                         // 16-row blocks: M <= 64
constexpr int MAXP = 64;
// k-steps a wave may hold (its A fragments stay in registers): 4 up to 32
// rows, 2 at 64 rows, keeping the kernel within 128 VGPRs (4 waves per SIMD)
__host__ __device__ constexpr int max_steps(int mb) { return mb <= 2 ? 4 : 2; }
constexpr int MAX_LDS = WAVES * KSTEP * 4 * ROW;                 // 128 KiB
}

__device__ __forceinline__ int dec_swz(int k) { return 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1); }

// Epilogue of one output pair (row, col), (row, col+1): bw and rw are the
// fp16 pairs of bias and R, loaded at kernel start.
template <int LAST>
__device__ __forceinline__ void dec_store_pair(uint16_t *__restrict__ out, int N, int row, int col, uint32_t bw,
                                               uint32_t rw, float v0, float v1)
{
    *reinterpret_cast<uint32_t *>(out + (int64_t)row * N + col) =
        pack_f16x2(apply_ops<OP_BIAS, LAST>(v0, f16_lo(bw), f16_lo(rw)),
                   apply_ops<OP_BIAS, LAST>(v1, f16_hi(bw), f16_hi(rw)));
}

template <int LAST, int MB>
__global__ __launch_bounds__(dec::NT, 1) void gemm_decode_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
    int M, int N, int K, int P, uint32_t *__restrict__ counters, float *__restrict__ partials)
{
    constexpr int MS = dec::max_steps(MB);
    extern __shared__ __attribute__((aligned(1024))) char dec_lds[];
    __shared__ int is_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a run of
    // consecutive (strip, split) pairs so the splits of one strip, and the A
    // slices they share, stay in one L2.
    const int G = gridDim.x;
    int b = blockIdx.x;
    if (G % 8 == 0) b = (b % 8) * (G / 8) + b / 8;
    const int strip = b / P, split = b - strip * P;
    const int n0 = strip * dec::W;
    const int kw = K / (P * dec::WAVES);                          // k-rows per wave, multiple of 32
    const int kbase = split * (K / P) + wave * kw;
    const int nsteps = kw / dec::KSTEP;
    FC_LDS char *slab = (FC_LDS char *)dec_lds + wave * kw * dec::ROW;
    const uint32_t slab0 = (uint32_t)(uintptr_t)slab;
    const int g = lane >> 4, i = lane & 15;

    // the output pairs this thread stores if its workgroup finishes the strip
    // (row 16 rb + e / 64 of each row block rb): bias and R are fetched now,
    // off the critical tail
    const int e = 2 * threadIdx.x, erow = e / dec::W, col = n0 + e % dec::W;
    uint32_t bw = 0u, rw[MB];
    if (LAST >= OP_BIAS) bw = *reinterpret_cast<const uint32_t *>(bias + col);
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        rw[rb] = 0u;
        const int row = 16 * rb + erow;
        if (LAST >= OP_RES && row < M) rw[rb] = *reinterpret_cast<const uint32_t *>(R + (int64_t)row * N + col);
    }

    // A fragments (16x16x32 A operand: row 16 rb + i, k = 8g .. 8g+7 of each
    // k-step); rows past M repeat row M-1 and are never stored.
    f16x8 afr[MB][MS];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        const uint16_t *arow = A + (int64_t)min(16 * rb + i, M - 1) * K + kbase + 8 * g;
#pragma unroll
        for (int t = 0; t < MS; ++t)
            afr[rb][t] = *reinterpret_cast<const f16x8 *>(arow + min(t, nsteps - 1) * dec::KSTEP);
    }
    // B slab: each instruction moves 8 k-rows (1 KiB); lane l lands at byte
    // 16 l, i.e. row l / 8, unit l % 8, so it fetches the unit that the
    // swizzle places there.
    {
        const int r = lane >> 3;
        for (int blk = 0; blk < kw / 8; ++blk) {
            const int k = blk * 8 + r;
            const int u = (lane & 7) ^ dec_swz(k);
            __builtin_amdgcn_global_load_lds(
                (const FC_GLB void *)(B + (int64_t)(kbase + k) * N + n0 + u * 8),
                (FC_LDS void *)(slab + blk * 1024), 16, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);                            // vmcnt(0): slab and A landed

    f32x4 acc[MB][4];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rb][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < MS; ++t) {
        if (t < nsteps) {
            // all 8 fragment reads of the k-step first, one wait: lane i of
            // group g addresses k-row 32t + 8g + 4hh + i/4, columns 16j +
            // 4(i%4) .. +3; the transposing read hands lane i column 16j + i
            // at four consecutive k
            u32x2 bh[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = dec::KSTEP * t + 8 * g + 4 * hh + (i >> 2);
                    bh[j][hh] = lds_read_tr16(slab0 + k * dec::ROW +
                                              16 * ((2 * j + ((i & 3) >> 1)) ^ dec_swz(k)) + (i & 1) * 8);
                }
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(bh[0][0]), "+v"(bh[0][1]), "+v"(bh[1][0]), "+v"(bh[1][1]), "+v"(bh[2][0]),
                           "+v"(bh[2][1]), "+v"(bh[3][0]), "+v"(bh[3][1]));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 bq = {bh[j][0].x, bh[j][0].y, bh[j][1].x, bh[j][1].y};
#pragma unroll
                for (int rb = 0; rb < MB; ++rb)
                    acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[rb][t], __builtin_bit_cast(f16x8, bq),
                                                                        acc[rb][j], 0, 0, 0);
            }
        }
    }
    // 16x16 result layout: lane holds column 16j + i, rows 4g + r.  Each
    // thread owns the output pair e, e+1 of every 16x64 row block.
    float *part = (float *)dec_lds;
    float v0[MB], v1[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        __syncthreads();                                          // slab (or previous block) consumed
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[wave * dec::TILE + (4 * g + r) * dec::W + 16 * j + i] = acc[rb][j][r];
        __syncthreads();
        v0[rb] = 0.0f;
        v1[rb] = 0.0f;
#pragma unroll
        for (int w = 0; w < dec::WAVES; ++w) {
            const float2 pv = *reinterpret_cast<const float2 *>(part + w * dec::TILE + e);
            v0[rb] += pv.x;
            v1[rb] += pv.y;
        }
    }
    if (P == 1) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
            if (16 * rb + erow < M) dec_store_pair<LAST>(out, N, 16 * rb + erow, col, bw, rw[rb], v0[rb], v1[rb]);
        return;
    }
    // partials: [strip][split][row block][16 x 64]
    const int64_t pbase = ((int64_t)strip * P + split) * MB * dec::TILE + e;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
        __hip_atomic_store(reinterpret_cast<uint64_t *>(partials + pbase + rb * dec::TILE),
                           __builtin_bit_cast(uint64_t, make_float2(v0[rb], v1[rb])), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // the same fence-free handoff as gemm_ring128_kernel's (the four rules
    // listed there): device-scope stores, vmcnt(0), barrier, ticket, and
    // device-scope loads by the last workgroup
    __builtin_amdgcn_s_waitcnt(0xF70);                            // vmcnt(0): the partial is at the coherence point
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = __hip_atomic_fetch_add(counters + strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(P - 1);
    __syncthreads();
    if (!is_last) return;
    // the P partials of each row block, eight loads in flight at a time,
    // summed in split order
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        float s0 = 0.0f, s1 = 0.0f;
        const uint64_t *src =
            reinterpret_cast<const uint64_t *>(partials + (int64_t)strip * P * MB * dec::TILE + rb * dec::TILE + e);
        for (int p0 = 0; p0 < P; p0 += 8) {
            uint64_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (p0 + q < P)
                    w[q] = __hip_atomic_load(src + (int64_t)(p0 + q) * (MB * dec::TILE / 2), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (p0 + q < P) {
                    const float2 pv = __builtin_bit_cast(float2, w[q]);
                    s0 += pv.x;
                    s1 += pv.y;
                }
        }
        if (16 * rb + erow < M) dec_store_pair<LAST>(out, N, 16 * rb + erow, col, bw, rw[rb], s0, s1);
    }
    if (threadIdx.x == 0) __hip_atomic_store(counters + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-row blocks of the decode kernel for M rows (1, 2 or 4), 0 past 64 rows
// (from 65 rows the 128x128 ring kernel is faster: 30-34 vs 34-38 us for
// 65..128 x 4096 x 4096 with eight blocks of 16 rows).
static int decode_blocks(int M)
{
    return M <= 16 ? 1 : M <= 32 ? 2 : M <= 16 * dec::MAXMB ? 4 : 0;
}

// Split of K for the decode kernel: the smallest power of two P with at least
// 512 workgroups (strips x P: two per CU, which streams B faster than one
// workgroup per CU with twice the loads in flight per wave), each wave
// holding 1 .. max_steps k-steps; else the largest P that fits.  0 when the
// shape does not fit (then another kernel runs).
static int decode_splits(int M, int N, int K)
{
    const int mb = decode_blocks(M);
    if (mb == 0 || N % dec::W != 0 || K % (dec::WAVES * dec::KSTEP) != 0) return 0;
    const int strips = N / dec::W;
    int best = 0;
    for (int P = 1; P <= dec::MAXP; P *= 2) {
        if (K % (P * dec::WAVES * dec::KSTEP) != 0) break;
        if (K > P * dec::WAVES * dec::KSTEP * dec::max_steps(mb)) continue;
        best = P;
        if ((int64_t)strips * P >= 512) break;
    }
    return best;
}

// Split of K for the 128x128 ring kernel: 1 when there are at least 128
// tiles; else the smallest power of two P up to 16 that brings the grid to
// 128 workgroups, with every split at least 256 k-rows (8 slabs) deep, else
// the largest such P (1 when none).  Measured on 129..1024 x 4096 x 4096 and
// 1024^3, 2048^3: splitting further (to 256 or 512 workgroups) costs more in
// partial traffic and summing than the extra workgroups gain.
static int ring128_splits(int M, int N, int K)
{
    const int64_t tiles = (int64_t)((M + r128::BM - 1) / r128::BM) * ((N + r128::BN - 1) / r128::BN);
    int best = 1;
    if (tiles >= 128) return best;
    for (int P = 2; P <= 16; P *= 2) {
        if (K % (64 * P) != 0 || K / P < 256) break;
        best = P;
        if (tiles * P >= 128) break;
    }
    return best;
}

// Which kernel runs the GEMM segment of (M, N, K), and its split of K.
enum GemmRoute { ROUTE_DECODE, ROUTE_SKINNY, ROUTE_RING, ROUTE_RING128, ROUTE_BIG, ROUTE_MID };

static GemmRoute gemm_route(int M, int N, int K, int &P)
{
    P = decode_splits(M, N, K);
    if (P > 0) return ROUTE_DECODE;
    P = 1;
    if (M <= 16) return ROUTE_SKINNY;
    const bool ring_ok = K % 64 == 0 && K <= ring::MAX_K && N <= ring::MAX_N;
    // The 128x128 ring kernel while its tiles fit in one round of two
    // workgroups on each of the 256 CUs; past that the 256x256 one, whose
    // round holds four times the work (measured: 2048 x 4096 x 4096, 512
    // small tiles: 101 vs 109 us; 2088 x 4072, 544 small tiles and a second
    // round of 32: 123 vs 98 us; 3072 rows: 135 vs 119 us)
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    const int64_t small_tiles = (int64_t)((M + r128::BM - 1) / r128::BM) * ((N + r128::BN - 1) / r128::BN);
    if (ring_ok && small_tiles > 512) return ROUTE_RING;
    if (ring_ok) {
        P = ring128_splits(M, N, K);
        return ROUTE_RING128;
    }
    return big_tiles >= 128 ? ROUTE_BIG : ROUTE_MID;
}

// Split-K scratch inside the caller's workspace, for the decode kernel or the
// split 128x128 ring kernel: arrival counters (one per strip or tile, 256-byte
// rounded), then the fp32 partials; both 0 when the shape takes no split.
static void split_scratch(int M, int N, int K, size_t &counter_bytes, size_t &partial_bytes)
{
    counter_bytes = partial_bytes = 0;
    int P;
    const GemmRoute route = gemm_route(M, N, K, P);
    if (P <= 1) return;
    if (route == ROUTE_DECODE) {
        const size_t strips = (size_t)(N / dec::W);
        counter_bytes = (strips * 4 + 255) & ~(size_t)255;
        partial_bytes = strips * (size_t)P * decode_blocks(M) * dec::TILE * 4;
    } else if (route == ROUTE_RING128) {
        const size_t tiles = (size_t)((M + r128::BM - 1) / r128::BM) * ((N + r128::BN - 1) / r128::BN);
        counter_bytes = (tiles * 4 + 255) & ~(size_t)255;
        partial_bytes = tiles * (size_t)P * r128::BM * r128::BN * 4;
    }
}

static size_t split_scratch_bytes(int M, int N, int K)
{
    size_t c, p;
    split_scratch(M, N, K, c, p);
    return c + p;
}

// ------------------------------------------------------------------ pointwise segments

// Operators FIRST..LAST on an fp16 [M,N] intermediate; out may equal in.
constexpr int kPwBlock = 256;

template <int FIRST, int LAST>
__global__ __launch_bounds__(kPwBlock) void epi_pointwise_kernel(const uint16_t *in,
                                                            const uint16_t *__restrict__ bias,
                                                            const uint16_t *__restrict__ R,
                                                            uint16_t *out, int64_t chunks, int N)
{
    const int64_t stride = (int64_t)gridDim.x * kPwBlock;
    for (int64_t c = (int64_t)blockIdx.x * kPwBlock + threadIdx.x; c < chunks; c += stride) {
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

// Split-K scratch (decode or 128x128 ring kernel) inside the caller's workspace.
struct DecodeScratch {
    uint32_t *counters;
    float *partials;
};

template <int LAST, int MB>
static int launch_decode(const uint16_t *A, const uint16_t *B, const uint16_t *bias, const uint16_t *R,
                         uint16_t *out, int M, int N, int K, int P, int grid, int lds, DecodeScratch ds,
                         hipStream_t s)
{
    // dynamic LDS above 64 KiB has to be allowed per kernel
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)gemm_decode_kernel<LAST, MB>, hipFuncAttributeMaxDynamicSharedMemorySize, dec::MAX_LDS);
    if (attr != hipSuccess) return FC_ERR_HIP;
    gemm_decode_kernel<LAST, MB><<<grid, dec::NT, lds, s>>>(A, B, bias, R, out, M, N, K, P, ds.counters,
                                                             ds.partials);
    return launch_status();
}

template <int LAST>
static int launch_gemm(const uint16_t *A, const uint16_t *B, const uint16_t *bias, const uint16_t *R,
                       uint16_t *out, int M, int N, int K, DecodeScratch ds, hipStream_t s)
{
    int P;
    const GemmRoute route = gemm_route(M, N, K, P);
    if (route == ROUTE_DECODE) {
        const int grid = (N / dec::W) * P;
        const int lds = (K / P) * dec::ROW;
        switch (decode_blocks(M)) {
        case 1: return launch_decode<LAST, 1>(A, B, bias, R, out, M, N, K, P, grid, lds, ds, s);
        case 2: return launch_decode<LAST, 2>(A, B, bias, R, out, M, N, K, P, grid, lds, ds, s);
        default: return launch_decode<LAST, 4>(A, B, bias, R, out, M, N, K, P, grid, lds, ds, s);
        }
    }
    if (route == ROUTE_SKINNY) {
        gemm_skinny_kernel<kSkinnyWaves, LAST><<<(N + 15) / 16, kSkinnyWaves * 64, 0, s>>>(
            A, B, bias, R, out, M, N, K);
        return launch_status();
    }
    if (route == ROUTE_RING) {
        const int tiles_m = (M + ring::BM - 1) / ring::BM, tiles_n = (N + ring::BN - 1) / ring::BN;
        gemm_ring_kernel<LAST><<<tiles_m * tiles_n, ring::NT, 0, s>>>(A, B, bias, R, out, M, N, K, tiles_m,
                                                                     tiles_n);
        return launch_status();
    }
    if (route == ROUTE_RING128) {
        const int tiles_m = (M + r128::BM - 1) / r128::BM, tiles_n = (N + r128::BN - 1) / r128::BN;
        gemm_ring128_kernel<LAST><<<dim3(tiles_m * tiles_n, P), r128::NT, 0, s>>>(
            A, B, bias, R, out, M, N, K, tiles_m, tiles_n, P, ds.counters, ds.partials);
        return launch_status();
    }
    if (route == ROUTE_BIG) {
        const int tiles_m = (M + big::BM - 1) / big::BM, tiles_n = (N + big::BN - 1) / big::BN;
        const bool interior = M % big::BM == 0 && N % big::BN == 0 && K % big::BK == 0;
        if (interior)
            gemm_big_kernel<LAST, false><<<tiles_m * tiles_n, big::NT, 0, s>>>(A, B, bias, R, out, M, N, K,
                                                                              tiles_m, tiles_n);
        else
            gemm_big_kernel<LAST, true><<<tiles_m * tiles_n, big::NT, 0, s>>>(A, B, bias, R, out, M, N, K,
                                                                             tiles_m, tiles_n);
        return launch_status();
    }
    return launch_gemm_cfg<CfgMid, LAST>(A, B, bias, R, out, M, N, K, s);
}

static int launch_gemm_segment(int last, const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                               const uint16_t *R, uint16_t *out, int M, int N, int K, DecodeScratch ds,
                               hipStream_t s)
{
    switch (last) {
    case 0: return launch_gemm<0>(A, B, bias, R, out, M, N, K, ds, s);
    case 1: return launch_gemm<1>(A, B, bias, R, out, M, N, K, ds, s);
    case 2: return launch_gemm<2>(A, B, bias, R, out, M, N, K, ds, s);
    case 3: return launch_gemm<3>(A, B, bias, R, out, M, N, K, ds, s);
    default: return FC_ERR_PLAN;
    }
}

template <int FIRST, int LAST>
static int launch_pw(const uint16_t *in, const uint16_t *bias, const uint16_t *R, uint16_t *out,
                     int64_t MN, int N, hipStream_t s)
{
    // one 16-byte chunk per thread and a grid that covers the tensor once
    // (faster than a grid-stride loop over fewer workgroups: at the decode
    // shape the old grid of 8 workgroups made the cut plans 11-15 % slower;
    // 64-thread workgroups measured no better); the loop in the kernel covers
    // what a capped grid leaves
    const int64_t chunks = MN / 8;
    int64_t grid = ceil_div(chunks, (int64_t)kPwBlock);
    if (grid < 1) grid = 1;
    if (grid > 0x7fffffff) grid = 0x7fffffff;
    epi_pointwise_kernel<FIRST, LAST><<<(int)grid, kPwBlock, 0, s>>>(in, bias, R, out, chunks, N);
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

// Workspace layout: [split-K counters + partials, when the shape takes the
// split decode or 128x128 ring kernel][fp16 intermediate, 2MN bytes rounded up
// to 256, when the plan has a cut].  The counters sit at offset 0 for every plan of a
// shape, so one workspace serves all plans of that shape.
static size_t inter_bytes(int M, int N, int plan_len)
{
    return plan_len > 1 ? ((2 * (size_t)M * (size_t)N + 255) & ~(size_t)255) : 0;
}

extern "C" size_t fc_gemm_workspace_bytes(int M, int N, int K, const int *plan, int plan_len)
{
    if (!plan_valid(plan, plan_len) || M < 1 || N < 1 || K < 1) return 0;
    return inter_bytes(M, N, plan_len) + split_scratch_bytes(M, N, K);
}

// Argument checks of both GEMM entry points; no HIP call.
static int gemm_validate(const uint16_t *A, const uint16_t *B, const uint16_t *bias, const uint16_t *R,
                         const uint16_t *Y, int M, int N, int K, const int *plan, int plan_len)
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
    return FC_OK;
}

// Enqueues the plan's kernels: the GEMM segment (split-K scratch in ds), then
// the pointwise segments through the fp16 intermediate `inter`.
static int gemm_enqueue(const uint16_t *A, const uint16_t *B, const uint16_t *bias, const uint16_t *R,
                        uint16_t *Y, int M, int N, int K, const int *plan, int plan_len, DecodeScratch ds,
                        uint16_t *inter, hipStream_t s)
{
    // operators: 0 = mm, 1 = bias, 2 = gelu, 3 = residual
    int first = 0;
    for (int seg = 0; seg < plan_len; ++seg) {
        const int last = first + plan[seg] - 1;
        uint16_t *dst = (seg == plan_len - 1) ? Y : inter;
        int rc;
        if (seg == 0)
            rc = launch_gemm_segment(last, A, B, bias, R, dst, M, N, K, ds, s);
        else
            rc = launch_pointwise(first, last, inter, bias, R, dst, (int64_t)M * N, N, s);
        if (rc != FC_OK) return rc;
        first = last + 1;
    }
    return FC_OK;
}

extern "C" int fc_gemm_epilogue(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                                const uint16_t *R, uint16_t *Y, int M, int N, int K,
                                const int *plan, int plan_len, void *workspace, size_t ws_bytes,
                                fc_stream stream)
{
    const int v = gemm_validate(A, B, bias, R, Y, M, N, K, plan, plan_len);
    if (v != FC_OK) return v;
    const size_t mn = (size_t)M * N * 2;
    const size_t need = fc_gemm_workspace_bytes(M, N, K, plan, plan_len);
    size_t counter_bytes, partial_bytes;
    split_scratch(M, N, K, counter_bytes, partial_bytes);
    const size_t dsb = counter_bytes + partial_bytes;
    uint16_t *ws = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + dsb);
    DecodeScratch ds = {nullptr, nullptr};
    if (need) {
        if (!workspace || ws_bytes < need) return FC_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FC_ERR_ALIGN;
        if (overlaps(workspace, need, A, (size_t)M * K * 2) || overlaps(workspace, need, B, (size_t)K * N * 2) ||
            overlaps(workspace, need, bias, (size_t)N * 2) || overlaps(workspace, need, R, mn) ||
            overlaps(workspace, need, Y, mn))
            return FC_ERR_ALIAS;
        if (dsb) {
            char *base = static_cast<char *>(workspace);
            ds.counters = reinterpret_cast<uint32_t *>(base);
            ds.partials = reinterpret_cast<float *>(base + counter_bytes);
        }
    }
    return gemm_enqueue(A, B, bias, R, Y, M, N, K, plan, plan_len, ds, ws, reinterpret_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ no-allocation variant

// The workspace of fc_gemm_epilogue_noalloc: one array per device, held until
// the process ends.  Host code never uses its name as an address (on the host
// the name is a stand-in, not the device allocation): the device address is
// looked up once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FC_GEMM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];   // device address of `scratch` on device d, once looked up
}  // namespace

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).  A stream of another
// device would run the kernels against this device's array: refused.
static int scratch_on_current_device(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FC_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FC_ERR_UNSUPPORTED;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return FC_ERR_HIP;
        }
        if (sdev != dev) return FC_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return FC_ERR_HIP;
        }
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return FC_OK;
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

extern "C" int fc_gemm_epilogue_noalloc(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                                        const uint16_t *R, uint16_t *Y, int M, int N, int K,
                                        const int *plan, int plan_len, fc_stream stream)
{
    const int v = gemm_validate(A, B, bias, R, Y, M, N, K, plan, plan_len);
    if (v != FC_OK) return v;
    const size_t need = fc_gemm_workspace_bytes(M, N, K, plan, plan_len);
    if (need > FC_GEMM_NOALLOC_SCRATCH_BYTES) return FC_ERR_SCRATCH;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *base = nullptr;
    if (need) {
        void *p = nullptr;
        const int rc = scratch_on_current_device(s, &p);
        if (rc != FC_OK) return rc;
        base = static_cast<char *>(p);
    }
    size_t counter_bytes, partial_bytes;
    split_scratch(M, N, K, counter_bytes, partial_bytes);
    DecodeScratch ds = {nullptr, nullptr};
    if (counter_bytes) {
        // the previous call on this device may have left anything here (another
        // shape's partials or intermediate): the arrival counters start at zero
        ds.counters = reinterpret_cast<uint32_t *>(base);
        ds.partials = reinterpret_cast<float *>(base + counter_bytes);
        const int64_t words = (int64_t)(counter_bytes / 4);
        zero_words_kernel<<<(int)std::min<int64_t>(64, ceil_div(words, (int64_t)256)), 256, 0, s>>>(ds.counters,
                                                                                                  words);
        const int rc = launch_status();
        if (rc != FC_OK) return rc;
    }
    uint16_t *inter = need ? reinterpret_cast<uint16_t *>(base + counter_bytes + partial_bytes) : nullptr;
    return gemm_enqueue(A, B, bias, R, Y, M, N, K, plan, plan_len, ds, inter, s);
}
