// Causal attention in one kernel that never writes the scores: per query tile,
// key/value tiles stream through LDS and an online softmax keeps the running
// row max and sum ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5: causal
// mask and block skipping; its further-reading list: the attention kernel
// that removes the S x S score tensor by normalising as it goes).
//
// Layout: Q, K, V, O bf16 [BH, S, 128] row-major.  A workgroup owns 128
// queries of one head (4 waves x 32); 64-key tiles of K and V are loaded
// into a double-buffered LDS ring (2 x (16 + 16) KiB) one tile ahead, by
// buffer loads that write LDS directly (the tile's row offset rides in the
// scalar offset, so the per-lane addresses are computed once); only a ragged
// last tile goes through clamped per-lane global loads.  Per tile each wave
// computes
//   S^T = K Q^T           (v_mfma_f32_32x32x16_bf16, K from LDS as the A
//                          operand, Q fragments held in registers)
// so a lane owns one query and 32 of the tile's 64 keys (the other 32 are in
// lane +-32): the row max and sum need one cross-half swap
// (v_permlane32_swap), the running rescale of the output stays in the lane.
//   O^T += V^T P^T        (P packed to bf16 straight from the S registers as
//                          the B operand; V^T fragments come from LDS with the
//                          transposing read ds_read_b64_tr_b16 in the same key
//                          order as the P registers)
// The softmax runs in the log2 domain: the running max is taken over the raw
// scores and the scale (times log2 e) enters once per score, fused into the
// exponent's argument (v_fma + v_exp_f32); a positive scale is required.  The
// reference subtracted in the exponents trails the running max by at most 8
// (a factor 2^8; it is moved only past that), so the output rescale is rare.
// Key tiles entirely above a wave's queries are skipped; tiles that cross its
// diagonal are masked per element.  Query tiles with the most keys are
// dispatched first.
//
// LDS swizzles (16-byte units u of a 256-byte key row r):
//   K: u ^ (r & 15)      -- the b128 fragment reads of 16 consecutive keys hit
//                           16 different units
//   V: u ^ 4 (r & 3)     -- the transposing reads of 4 consecutive keys x two
//                           32-byte column pairs hit 8 different 32-byte slots
#include "fc_internal.h"

#include <type_traits>

#define FC_LDS __attribute__((address_space(3)))
#define FC_GLB __attribute__((address_space(1)))

namespace fc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace att {
constexpr int D = 128, BQ = 128, BKV = 64, WAVES = 4, NT = WAVES * 64;
constexpr int ROWB = D * 2;                   // bytes per key row
constexpr int TILE = BKV * ROWB;              // 16 KiB
constexpr int STAGE = 2 * TILE;               // K tile, then V tile
constexpr int LDS_BYTES = 2 * STAGE;          // two stages
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LAZY = 8.0f;                  // base-2 exponent slack of the running reference
constexpr int MAX_S = 1 << 22;                // byte offsets inside one head stay 32-bit
// buffer descriptor word 3 for raw 32-bit-format dword loads
constexpr int RSRC_WORD3 = 0x00020000;
}

// LDS fragment reads with the constant part of the address (stage, key
// block) in the instruction's 16-bit offset field, so the loop spends no
// VALU on addresses: the per-lane part is computed once per kernel.
template <int OFF>
__device__ __forceinline__ u32x4 att_read_b128(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x2 att_read_tr16(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// v_max3 without the operand canonicalisation the compiler adds to fmaxf
__device__ __forceinline__ float att_max3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// f(integral_constant<int, I>) for I = 0 .. N-1, so loop indices can be template arguments
template <int I, int N, class F>
__device__ __forceinline__ void att_static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        att_static_for<I + 1, N>(f);
    }
}

// This wave's quarter of key/value tile kt (rows clamped to S-1; such rows
// only meet masked queries or queries past S) into stage st.
__device__ __forceinline__ void att_issue(const uint16_t *__restrict__ Kh, const uint16_t *__restrict__ Vh,
                                          int S, int kt, FC_LDS char *st)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int blk = wave * 4 + q;                       // 1 KiB = 4 key rows
        const int r = blk * 4 + (lane >> 4);
        const int64_t key = min(kt * att::BKV + r, S - 1);
        __builtin_amdgcn_global_load_lds((const FC_GLB void *)(Kh + key * att::D + (p ^ (r & 15)) * 8),
                                         (FC_LDS void *)(st + blk * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const FC_GLB void *)(Vh + key * att::D + (p ^ (4 * (r & 3))) * 8),
                                         (FC_LDS void *)(st + att::TILE + blk * 1024), 16, 0, 0);
    }
}

__device__ __forceinline__ float att_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max and sum over the two 32-lane halves: both halves end with the same value
__device__ __forceinline__ float att_half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float att_half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t att_pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

__global__ __launch_bounds__(att::NT, 2) void attention_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, int64_t BH, int S, float scale_log2)
{
    __shared__ __attribute__((aligned(1024))) char lds_raw[att::LDS_BYTES];
    FC_LDS char *lds = (FC_LDS char *)lds_raw;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane >> 5, l32 = lane & 31;

    // heaviest query tiles first: the first BH workgroups take the last tile of every head
    const int nqt = (S + att::BQ - 1) / att::BQ;
    const int64_t bh = blockIdx.x % BH;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);
    const int q0 = qt * att::BQ;
    const uint16_t *Qh = Q + bh * (int64_t)S * att::D;
    const uint16_t *Kh = K + bh * (int64_t)S * att::D;
    const uint16_t *Vh = V + bh * (int64_t)S * att::D;

    const int wq0 = q0 + wave * 32;                         // this wave's first query
    const int query = wq0 + l32;                            // this lane's query
    const int kt_last = min(q0 + att::BQ - 1, S - 1) / att::BKV;
    const int wave_kt_last = min(wq0 + 31, S - 1) / att::BKV;

    // Q fragments (B operand of S^T = K Q^T): query l32, d = 16 ks + 8 hl .. +7
    u32x4 qf[8];
    {
        const uint16_t *qrow = Qh + (int64_t)min(query, S - 1) * att::D + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const u32x4 *>(qrow + 16 * ks);
    }

    // per-lane LDS addresses in stage 0 (stage 1 adds STAGE in the offset field)
    uint32_t ka[2][8];                                      // K: [key m-tile][k-step]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int r = 32 * t + l32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) ka[t][ks] = lds0 + r * att::ROWB + (((2 * ks + hl) ^ (r & 15)) * 16);
    }
    // V^T fragments: lane (group g = lane / 16, j = lane % 16) addresses key
    // k0 + j/4, d = 32 mt + 16 (g & 1) + 4 (j % 4); k0 = 32 t + 16 h + 8 e2 + 4 hl.
    // The key block (t, h) enters through the offset field; the d-tile mt
    // meets the swizzle in an XOR, so it gets its own address.
    uint32_t va[4][2];                                      // [mt][e2], for t = h = 0
    {
        const int g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int key = 8 * e2 + 4 * hl + (j >> 2);    // key & 3 == j >> 2 for every t, h
            const int unit = (16 * (g & 1) + 4 * (j & 3)) / 8;
            const uint32_t vb = att::TILE + key * att::ROWB + ((unit ^ (4 * (key & 3))) * 16) + (j & 1) * 8;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) va[mt][e2] = lds0 + (vb ^ (uint32_t)(mt * 64));
        }
    }

    f32x16 oacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // Tiles wholly below S load through buffer descriptors of this head's K and
    // V: per-lane byte offsets of this wave's rows inside a tile (computed once),
    // the tile as a scalar offset and the LDS block as a scalar M0, so the load
    // issue costs no vector instructions.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    uint32_t boff_k[4], boff_v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int blk = wave * 4 + q, r = blk * 4 + (lane >> 4), pu = lane & 15;
        boff_k[q] = (uint32_t)(r * att::D + (pu ^ (r & 15)) * 8) * 2u;
        boff_v[q] = (uint32_t)(r * att::D + (pu ^ (4 * (r & 3))) * 8) * 2u;
    }
    const int head_bytes = S * att::ROWB;
    const __amdgpu_buffer_rsrc_t rsrc_k =
        __builtin_amdgcn_make_buffer_rsrc((void *)Kh, (short)0, head_bytes, att::RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rsrc_v =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vh, (short)0, head_bytes, att::RSRC_WORD3);
    att_issue(Kh, Vh, S, 0, lds);

    // One key tile kt, read from stage ST (= kt & 1, a compile-time constant).
    auto tile = [&](int kt, auto stage) {
        constexpr int ST = decltype(stage)::value;
        constexpr int SOFF = ST * att::STAGE;
        __builtin_amdgcn_s_waitcnt(0xF70);                  // vmcnt(0): this wave's share of tile kt landed
        __builtin_amdgcn_s_barrier();                       // every wave's share landed; stage kt-1 is free
        __builtin_amdgcn_sched_barrier(0);
        if (kt < kt_last) {
            const int kn = kt + 1;
            FC_LDS char *stn = lds + (ST ^ 1) * att::STAGE;
            if ((kn + 1) * att::BKV <= S) {
                const int toff = kn * att::BKV * att::ROWB;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int blk = wave_s * 4 + q;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (FC_LDS void *)(stn + blk * 1024), 16,
                                                             boff_k[q], toff, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (FC_LDS void *)(stn + att::TILE + blk * 1024),
                                                             16, boff_v[q], toff, 0, 0);
                }
            } else {
                att_issue(Kh, Vh, S, kn, stn);                  // ragged last tile: rows clamped to S-1
            }
        }
        if (kt > wave_kt_last) return;                      // every key of this tile is above the diagonal

        // ---- S^T = K Q^T over d (8 k-steps), K fragments one step ahead
        f32x16 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[t][r] = 0.0f;
        u32x4 kf[2][2];
        kf[0][0] = att_read_b128<SOFF>(ka[0][0]);
        kf[0][1] = att_read_b128<SOFF>(ka[1][0]);
        att_static_for<0, 8>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value, cb = ks & 1;
            if constexpr (ks < 7) {
                kf[cb ^ 1][0] = att_read_b128<SOFF>(ka[0][ks + 1]);
                kf[cb ^ 1][1] = att_read_b128<SOFF>(ka[1][ks + 1]);
                asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(kf[cb][0]), "+v"(kf[cb][1]));
            } else {
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[cb][0]), "+v"(kf[cb][1]));
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
                sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[cb][t]),
                                                                  __builtin_bit_cast(bf16x8, qf[ks]), sacc[t],
                                                                  0, 0, 0);
        });
        __builtin_amdgcn_sched_barrier(0);

        // V^T fragments of key block kk (16 keys) into vr; the first block's
        // reads go out now, under the softmax
        auto read_v = [&](auto kkc, u32x2 (&vr)[4][2]) __attribute__((always_inline)) {
            constexpr int kk = decltype(kkc)::value;
            constexpr int VOFF = SOFF + (32 * (kk >> 1) + 16 * (kk & 1)) * att::ROWB;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                vr[mt][0] = att_read_tr16<VOFF>(va[mt][0]);
                vr[mt][1] = att_read_tr16<VOFF>(va[mt][1]);
            }
        };
        u32x2 vbuf[2][4][2];
        read_v(std::integral_constant<int, 0>{}, vbuf[0]);

        // ---- online softmax: lane holds query `query`, keys kt*64 + 32 t + 8 (r/4) + 4 hl + r%4.
        // Raw scores are masked and maximised (a positive scale keeps the
        // order); the scale enters once, fused into each exponent's argument.
        if (kt * att::BKV + att::BKV - 1 > wq0) {          // tile crosses this wave's diagonal
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * att::BKV + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (key > query) sacc[t][r] = -INFINITY;
                }
        }
        // max of the lane's 32 scores and the running max: a v_max3 tree of depth 4
        float a[11];
#pragma unroll
        for (int u = 0; u < 10; ++u) {
            const int i0 = 3 * u, i1 = i0 + 1, i2 = i0 + 2;
            a[u] = att_max3(sacc[i0 >> 4][i0 & 15], sacc[i1 >> 4][i1 & 15], sacc[i2 >> 4][i2 & 15]);
        }
        a[10] = att_max3(sacc[1][14], sacc[1][15], m_run);
        const float mloc = att_max3(att_max3(a[0], a[1], a[2]), att_max3(a[3], a[4], a[5]),
                                    att_max3(a[6], a[7], att_max3(a[8], a[9], a[10])));
        // The reference m_run trails the row max lazily: it moves only when the
        // max passes it by more than LAZY in the base-2 exponent, so that
        // probabilities stay <= 2^LAZY (exact in fp32, no loss in bf16's
        // relative rounding) and the output rescale below is rarely needed.
        const float m_max = att_half_max(mloc);             // >= m_run, which entered the max
        const float m_new = ((m_max - m_run) * scale_log2 > att::LAZY) ? m_max : m_run;  // finite after tile 0
        const float mc = m_new * scale_log2;
        const float alpha = att_exp2((m_run - m_new) * scale_log2);
        // P^T fragments (B operand): k-step (t, h) holds rows r = 8h .. 8h+7.
        // The row sum adds the bf16-rounded probabilities that multiply V
        // (v_dot2 against (1, 1)), so the weights applied to V sum to one.
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
        u32x4 pf[2][2];
        float lloc = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w =
                        att_pack_bf16(att_exp2(__builtin_fmaf(sacc[t][8 * h + 2 * q], scale_log2, -mc)),
                                      att_exp2(__builtin_fmaf(sacc[t][8 * h + 2 * q + 1], scale_log2, -mc)));
                    pf[t][h][q] = w;
                    lloc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, lloc, false);
                }
        l_run = l_run * alpha + att_half_sum(lloc);
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {  // no lane's reference moved: nothing to rescale
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) oacc[mt] *= alpha;
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T += V^T P^T over the tile's keys (4 k-steps x 4 d-tiles); the
        // V^T fragments of k-step kk+1 are read while those of kk feed the MFMAs
        att_static_for<0, 4>([&](auto kkc) {
            constexpr int kk = decltype(kkc)::value, t = kk >> 1, h = kk & 1, cb = kk & 1;
            if constexpr (kk < 3) {
                read_v(std::integral_constant<int, kk + 1>{}, vbuf[cb ^ 1]);
                asm volatile("s_waitcnt lgkmcnt(8)"
                             : "+v"(vbuf[cb][0][0]), "+v"(vbuf[cb][0][1]), "+v"(vbuf[cb][1][0]), "+v"(vbuf[cb][1][1]),
                               "+v"(vbuf[cb][2][0]), "+v"(vbuf[cb][2][1]), "+v"(vbuf[cb][3][0]), "+v"(vbuf[cb][3][1]));
            } else {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(vbuf[cb][0][0]), "+v"(vbuf[cb][0][1]), "+v"(vbuf[cb][1][0]), "+v"(vbuf[cb][1][1]),
                               "+v"(vbuf[cb][2][0]), "+v"(vbuf[cb][2][1]), "+v"(vbuf[cb][3][0]), "+v"(vbuf[cb][3][1]));
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const u32x4 av = {vbuf[cb][mt][0].x, vbuf[cb][mt][0].y, vbuf[cb][mt][1].x, vbuf[cb][mt][1].y};
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                   __builtin_bit_cast(bf16x8, pf[t][h]), oacc[mt],
                                                                   0, 0, 0);
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt <= kt_last; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 <= kt_last) tile(kt + 1, std::integral_constant<int, 1>{});
    }

    // ---- O = O^T / l, lane: query `query`, d = 32 mt + 8 gq + 4 hl + (0..3)
    if (query < S) {
        const float inv = 1.0f / l_run;
        uint16_t *orow = O + (bh * (int64_t)S + query) * att::D;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w.x = att_pack_bf16(oacc[mt][4 * gq + 0] * inv, oacc[mt][4 * gq + 1] * inv);
                w.y = att_pack_bf16(oacc[mt][4 * gq + 2] * inv, oacc[mt][4 * gq + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + 32 * mt + 8 * gq + 4 * hl) = w;
            }
    }
}

}  // namespace fc

using namespace fc;

extern "C" uint64_t fc_attention_flops(int64_t BH, int S, int D)
{
    if (BH < 1 || S < 1 || D < 1) return 0;
    return 2ull * (uint64_t)D * (uint64_t)S * (uint64_t)(S + 1) * (uint64_t)BH;
}

extern "C" uint64_t fc_attention_bytes(int64_t BH, int S, int D)
{
    if (BH < 1 || S < 1 || D < 1) return 0;
    return 8ull * (uint64_t)BH * (uint64_t)S * (uint64_t)D;
}

extern "C" int fc_causal_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O,
                                   int64_t BH, int S, int D, float scale, fc_stream stream)
{
    if (BH < 1 || S < 1 || D < 1) return FC_ERR_SHAPE;
    if (D != att::D) return FC_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || scale > 3.0e38f) return FC_ERR_SHAPE;   // also rejects NaN
    if (!Q || !K || !V || !O) return FC_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return FC_ERR_ALIGN;
    const size_t bytes = (size_t)BH * (size_t)S * (size_t)D * 2;
    if (overlaps(O, bytes, Q, bytes) || overlaps(O, bytes, K, bytes) || overlaps(O, bytes, V, bytes))
        return FC_ERR_ALIAS;
    const int64_t nqt = (S + att::BQ - 1) / att::BQ;
    if (BH * nqt > 0x7fffffff || S > att::MAX_S) return FC_ERR_UNSUPPORTED;
    attention_fwd_kernel<<<(unsigned)(BH * nqt), att::NT, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        Q, K, V, O, BH, S, scale * att::LOG2E);
    return launch_status();
}
