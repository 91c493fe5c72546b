// Reference rates for the hot-path kernels: plain streams over HBM and a
// plain MFMA loop.  These probes carry none of the method's arithmetic; they
// tell what a straightforward kernel gets out of the device for the same mix
// of traffic (or the same matrix instruction on random operands), so a
// kernel's roofline fraction can be read beside a rate that is reachable.
//
// Streams: every workgroup owns one 32 KiB chunk of the destination (256
// lanes x 8 x 16 bytes, block-contiguous, nontemporal).  A workgroup that also
// owns a source chunk loads all 8 of its vectors before it stores any, as the
// hot-path streaming kernels do; the source chunks are spread evenly over the
// destination, so reads and writes stay mixed across the whole launch.  Sizes
// are whole chunks, so no lane is predicated.
//
// MFMA: each wave keeps 8 independent 32x32x16 fp16 accumulations whose
// operands start from a hash of the lane id and flip one mantissa bit per
// iteration, so the multipliers see changing random data (constant operands
// draw less power and run at a higher clock than real data).
#include "fc_internal.h"
#include "../../include/fc_envelope.h"

namespace fce {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256, kVecs = 8;
constexpr size_t kChunk = (size_t)kBlock * kVecs * 16;    // 32 KiB
constexpr int kMfmaAcc = 8, kMfmaBlocks = 1024, kMfmaThreads = 256;

// MODE 0: copy (every workgroup owns a source chunk), 1: pure write,
// 2: read_chunks < write_chunks, owners spread evenly.
template <int MODE>
__global__ __launch_bounds__(kBlock) void mix_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst,
                                                     int64_t read_chunks, int64_t write_chunks)
{
    const int64_t w = blockIdx.x;
    int64_t r0 = w, r1 = w + 1;
    if (MODE == 1) r1 = r0;
    if (MODE == 2) {
        r0 = w * read_chunks / write_chunks;
        r1 = (w + 1) * read_chunks / write_chunks;
    }
    f32x4 *out = dst + w * (kBlock * kVecs) + threadIdx.x;
    if (r1 > r0) {
        const f32x4 *in = src + r0 * (kBlock * kVecs) + threadIdx.x;
        f32x4 v[kVecs];
#pragma unroll
        for (int u = 0; u < kVecs; ++u) v[u] = __builtin_nontemporal_load(in + u * kBlock);
#pragma unroll
        for (int u = 0; u < kVecs; ++u) __builtin_nontemporal_store(v[u], out + u * kBlock);
    } else {
        const f32x4 c = {1.0f, 2.0f, 3.0f, (float)threadIdx.x};
#pragma unroll
        for (int u = 0; u < kVecs; ++u) __builtin_nontemporal_store(c, out + u * kBlock);
    }
}

// Flat streams: one 16-byte vector per lane, one 4 KiB workgroup per 256
// vectors, a grid that covers the buffer once (the fastest plain write and
// copy shape measured on this device: each workgroup's footprint is small).
__global__ __launch_bounds__(kBlock) void flat_write_kernel(f32x4 *__restrict__ dst)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    dst[i] = f32x4{1.0f, 2.0f, 3.0f, (float)threadIdx.x};
}

__global__ __launch_bounds__(kBlock) void flat_copy_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kBlock) void read_kernel(const f32x4 *__restrict__ src, float *__restrict__ sink)
{
    const f32x4 *in = src + (int64_t)blockIdx.x * (kBlock * kVecs) + threadIdx.x;
    f32x4 v[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; ++u) v[u] = __builtin_nontemporal_load(in + u * kBlock);
    f32x4 s = v[0];
#pragma unroll
    for (int u = 1; u < kVecs; ++u) s += v[u];
    // a store no input makes: keeps the loads without writing per lane
    if (s.x == 1.5f && s.y == -2.5f && s.z == 3.5f && s.w == -4.5f) sink[0] = s.x;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(float *__restrict__ sink, int iters)
{
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t x = (uint32_t)((blockIdx.x * kMfmaThreads + threadIdx.x) * 8 + e) * 2654435761u;
        x ^= x >> 15;
        x *= 0x2c1b3c6du;
        x ^= x >> 12;
        a[e] = (_Float16)((float)(x & 0xffffu) * (1.0f / 65536.0f) - 0.5f);
        b[e] = (_Float16)((float)(x >> 16) * (1.0f / 65536.0f) - 0.5f);
    }
    f32x16 acc[kMfmaAcc];
#pragma unroll
    for (int i = 0; i < kMfmaAcc; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kMfmaAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
        a = __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, a) ^ 0x00010001u);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMfmaAcc; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

__global__ void empty_kernel(float *__restrict__ sink)
{
    // stores only for a block index no launch reaches: the kernel does no work
    if (blockIdx.x == 0x7fffffff) sink[threadIdx.x] = 0.0f;
}

}  // namespace fce

using namespace fce;

extern "C" int fce_empty_n(int blocks, int n, float *sink, fc_stream stream)
{
    if (!sink) return FC_ERR_NULL;
    if (blocks < 1 || n < 1) return FC_ERR_SHAPE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int k = 0; k < n; ++k) empty_kernel<<<blocks, 64, 0, s>>>(sink);
    return fc::launch_status();
}

extern "C" int fce_empty(int blocks, float *sink, fc_stream stream) { return fce_empty_n(blocks, 1, sink, stream); }

extern "C" size_t fce_chunk_bytes(void) { return kChunk; }

extern "C" int fce_mix_n(const void *src, size_t read_bytes, void *dst, size_t write_bytes, int n,
                         fc_stream stream)
{
    if (!dst || (read_bytes && !src)) return FC_ERR_NULL;
    if (n < 1) return FC_ERR_SHAPE;
    if (write_bytes == 0 || write_bytes % kChunk || read_bytes % kChunk || read_bytes > write_bytes)
        return FC_ERR_SHAPE;
    if (!fc::aligned16(src) || !fc::aligned16(dst)) return FC_ERR_ALIGN;
    if (read_bytes && fc::overlaps(src, read_bytes, dst, write_bytes)) return FC_ERR_ALIAS;
    const int64_t wc = (int64_t)(write_bytes / kChunk), rc = (int64_t)(read_bytes / kChunk);
    if (wc > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const f32x4 *in = static_cast<const f32x4 *>(src);
    f32x4 *out = static_cast<f32x4 *>(dst);
    for (int k = 0; k < n; ++k) {
        if (rc == wc)
            mix_kernel<0><<<(unsigned)wc, kBlock, 0, s>>>(in, out, rc, wc);
        else if (rc == 0)
            mix_kernel<1><<<(unsigned)wc, kBlock, 0, s>>>(in, out, rc, wc);
        else
            mix_kernel<2><<<(unsigned)wc, kBlock, 0, s>>>(in, out, rc, wc);
    }
    return fc::launch_status();
}

extern "C" int fce_mix(const void *src, size_t read_bytes, void *dst, size_t write_bytes, fc_stream stream)
{
    return fce_mix_n(src, read_bytes, dst, write_bytes, 1, stream);
}

// Flat granule: 256 lanes x 16 bytes.
static constexpr size_t kFlat = (size_t)kBlock * 16;

extern "C" int fce_flat(const void *src, void *dst, size_t bytes, fc_stream stream)
{
    if (!dst) return FC_ERR_NULL;
    if (bytes == 0 || bytes % kFlat) return FC_ERR_SHAPE;
    if (!fc::aligned16(src) || !fc::aligned16(dst)) return FC_ERR_ALIGN;
    if (src && fc::overlaps(src, bytes, dst, bytes)) return FC_ERR_ALIAS;
    const int64_t blocks = (int64_t)(bytes / kFlat);
    if (blocks > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (src)
        flat_copy_kernel<<<(unsigned)blocks, kBlock, 0, s>>>(static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst));
    else
        flat_write_kernel<<<(unsigned)blocks, kBlock, 0, s>>>(static_cast<f32x4 *>(dst));
    return fc::launch_status();
}

extern "C" int fce_read(const void *src, size_t read_bytes, float *sink, fc_stream stream)
{
    if (!src || !sink) return FC_ERR_NULL;
    if (read_bytes == 0 || read_bytes % kChunk) return FC_ERR_SHAPE;
    if (!fc::aligned16(src)) return FC_ERR_ALIGN;
    const int64_t rc = (int64_t)(read_bytes / kChunk);
    if (rc > 0x7fffffff) return FC_ERR_UNSUPPORTED;
    read_kernel<<<(unsigned)rc, kBlock, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const f32x4 *>(src), sink);
    return fc::launch_status();
}

extern "C" size_t fce_mfma_sink_floats(void) { return (size_t)kMfmaBlocks * kMfmaThreads; }

extern "C" double fce_mfma_flops(int iters)
{
    return iters < 1 ? 0.0
                     : (double)kMfmaBlocks * (kMfmaThreads / 64) * (double)iters * kMfmaAcc * (2.0 * 32 * 32 * 16);
}

extern "C" int fce_mfma(float *sink, int iters, fc_stream stream)
{
    if (!sink) return FC_ERR_NULL;
    if (iters < 1) return FC_ERR_SHAPE;
    mfma_kernel<<<kMfmaBlocks, kMfmaThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(sink, iters);
    return fc::launch_status();
}
