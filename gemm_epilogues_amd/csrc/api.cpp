// Host-only entry points: byte/launch accounting, status strings, version.
// Pure integer functions; they never touch the device.
#include <stdint.h>
#include <stddef.h>

#include "../../include/fc.h"

namespace {

bool plan_ok(const int *plan, int plan_len)
{
    if (!plan || plan_len < 1 || plan_len > 4) return false;
    int sum = 0;
    for (int i = 0; i < plan_len; ++i) {
        if (plan[i] <= 0) return false;
        sum += plan[i];
    }
    return sum == 4;
}

}  // namespace

// Split plan of the GEMM epilogue chain ("K4 讲解：fusion 的三笔账", section 1):
// A, B, bias and R are read once, Y written once, and each cut writes one
// [M,N] intermediate and reads it back.
extern "C" uint64_t fc_plan_bytes(int64_t M, int64_t N, int64_t K, const int *plan, int plan_len,
                                  int elem_bytes)
{
    if (!plan_ok(plan, plan_len) || M < 1 || N < 1 || K < 1 || elem_bytes < 1) return 0;
    const uint64_t mn = (uint64_t)M * (uint64_t)N;
    const uint64_t cuts = (uint64_t)(plan_len - 1);
    const uint64_t elems = (uint64_t)M * K + (uint64_t)K * N + (uint64_t)N + 2 * mn + 2 * cuts * mn;
    return elems * (uint64_t)elem_bytes;
}

extern "C" int fc_plan_launches(const int *plan, int plan_len)
{
    return plan_ok(plan, plan_len) ? plan_len : 0;
}

// fp32 chain ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.2): one pass
// reads and writes n floats; naive makes K passes, fused one.
extern "C" uint64_t fc_chain_bytes(int64_t n, int K, int mode)
{
    if (n < 0 || K < 1) return 0;
    const uint64_t pass = 8 * (uint64_t)n;
    if (mode == FC_CHAIN_NAIVE) return (uint64_t)K * pass;
    if (mode == FC_CHAIN_FUSED || mode == FC_CHAIN_FAT) return pass;
    return 0;
}

// Causal softmax: fused reads each row's kept key tiles (section 3.5 block
// skipping) and writes the whole output; unfused touches the score-sized
// tensor 8 times, reads the mask once and moves fp32 row statistics.
extern "C" uint64_t fc_softmax_bytes(int64_t BH, int S, int tile, int mode)
{
    if (BH < 1 || S < 1) return 0;
    const uint64_t s = (uint64_t)S;
    const uint64_t score = (uint64_t)BH * s * s;
    if (mode == FC_SOFTMAX_UNFUSED) return 2 * score * 9 + 16 * (uint64_t)BH * s;
    if (mode != FC_SOFTMAX_FUSED) return 0;
    if (!(tile == 64 || tile == 128 || tile == 256 || tile == S)) return 0;
    const uint64_t t = (uint64_t)tile;
    const uint64_t full = s / t;               // complete key tiles; rows of tile b read (b+1)*t
    const uint64_t rest = s % t;               // rows of the partial last tile read all S keys
    const uint64_t per_head = t * t * full * (full + 1) / 2 + rest * s;
    return 2 * ((uint64_t)BH * per_head + score);
}

extern "C" const char *fc_status_string(int status)
{
    switch (status) {
    case FC_OK: return "ok";
    case FC_ERR_NULL: return "null pointer";
    case FC_ERR_SHAPE: return "invalid shape";
    case FC_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FC_ERR_PLAN: return "split plan is not a composition of 4";
    case FC_ERR_UNSUPPORTED: return "unsupported argument";
    case FC_ERR_WORKSPACE: return "workspace missing or too small";
    case FC_ERR_HIP: return "HIP launch failed";
    case FC_ERR_ALIAS: return "buffers overlap";
    default: return "unknown status";
    }
}

extern "C" const char *fc_version(void) { return "fc 0.1.0 gfx950"; }
