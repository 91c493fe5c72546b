// Host-only entry points: byte/launch accounting, status strings, version.
// Pure integer functions; they never touch the device.
#include <stdint.h>
#include <stddef.h>

#include "../../include/fc.h"
#include "kernel_info.h"

#include <string.h>

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

// ------------------------------------------------------------------ cost model

// The split-plan time model of "K4 讲解：fusion 的三笔账", section 2: a plan's
// segments each cost max(memory time, compute time) plus one launch, where a
// segment's bytes are its stages' external reads, the intermediate it reads
// from the previous segment (none for the first) and the one tensor it
// writes; the memory time is stretched by a factor that depends on the live
// registers of the fused segment (the sum over its stages).  The pages use a
// single threshold (255 registers, factor 3 beyond it); the model here takes
// a table of register levels so a device's occupancy steps can be entered.

namespace {

bool composition_ok(const int *plan, int plan_len, int n)
{
    if (!plan || plan_len < 1 || plan_len > n) return false;
    int sum = 0;
    for (int i = 0; i < plan_len; ++i) {
        if (plan[i] <= 0) return false;
        sum += plan[i];
    }
    return sum == n;
}

bool model_ok(const fc_cost_model *m)
{
    if (!m || !(m->hbm_bytes_per_s > 0) || !(m->flops_per_s > 0) || !(m->launch_s >= 0)) return false;
    if (m->n_levels < 0 || m->n_levels > FC_COST_MAX_LEVELS || !(m->spill_factor > 0)) return false;
    for (int i = 0; i < m->n_levels; ++i) {
        if (!(m->mem_factor[i] > 0)) return false;
        if (i > 0 && m->reg_level[i] <= m->reg_level[i - 1]) return false;
    }
    return true;
}

double mem_factor(const fc_cost_model *m, double regs)
{
    for (int i = 0; i < m->n_levels; ++i)
        if (regs <= m->reg_level[i]) return m->mem_factor[i];
    return m->spill_factor;
}

}  // namespace

extern "C" double fc_segments_time(const fc_stage *stages, int n_stages, const int *plan, int plan_len,
                                   int elem_bytes, const fc_cost_model *m)
{
    if (!stages || n_stages < 1 || n_stages > FC_COST_MAX_STAGES || elem_bytes < 1 || !model_ok(m)) return -1.0;
    if (!composition_ok(plan, plan_len, n_stages)) return -1.0;
    double t = 0.0;
    int s = 0;
    for (int seg = 0; seg < plan_len; ++seg) {
        double elems = 0.0, flops = 0.0, regs = 0.0;
        if (s > 0) elems += stages[s - 1].writes;          // the intermediate written by the previous segment
        for (int k = s; k < s + plan[seg]; ++k) {
            elems += stages[k].ext_reads;
            flops += stages[k].flops;
            regs += stages[k].live_regs;
        }
        elems += stages[s + plan[seg] - 1].writes;          // the segment's one output
        const double tm = elems * elem_bytes / m->hbm_bytes_per_s * mem_factor(m, regs);
        const double tc = flops / m->flops_per_s;
        t += (tm > tc ? tm : tc) + m->launch_s;
        s += plan[seg];
    }
    return t;
}

extern "C" int fc_best_split(const fc_stage *stages, int n_stages, int elem_bytes, const fc_cost_model *m,
                             int *plan_out, int *plan_len_out, double *t_out)
{
    if (!stages || n_stages < 1 || n_stages > FC_COST_MAX_STAGES || elem_bytes < 1 || !model_ok(m))
        return FC_ERR_SHAPE;
    if (!plan_out || !plan_len_out) return FC_ERR_NULL;
    // bit k of the mask set = a cut after stage k; all 2^(n-1) compositions
    double best = -1.0;
    int best_plan[FC_COST_MAX_STAGES], best_len = 0;
    for (unsigned mask = 0; mask < (1u << (n_stages - 1)); ++mask) {
        int plan[FC_COST_MAX_STAGES], len = 0, run = 1;
        for (int k = 0; k < n_stages - 1; ++k) {
            if (mask & (1u << k)) {
                plan[len++] = run;
                run = 1;
            } else {
                ++run;
            }
        }
        plan[len++] = run;
        const double t = fc_segments_time(stages, n_stages, plan, len, elem_bytes, m);
        if (best < 0.0 || t < best) {                       // first minimum in mask order wins ties
            best = t;
            best_len = len;
            for (int i = 0; i < len; ++i) best_plan[i] = plan[i];
        }
    }
    for (int i = 0; i < best_len; ++i) plan_out[i] = best_plan[i];
    *plan_len_out = best_len;
    if (t_out) *t_out = best;
    return FC_OK;
}

// The K4 chain mm -> bias -> gelu -> res as stages (section 1 table): writes
// and external reads in elements, flops, and the pages' live-register figures
// (128 for the GEMM tile, 8 for bias, 16 for GELU, 8 for the residual, which
// give the table's per-plan peaks 128 / 128 / 136 / 160).
extern "C" int fc_gemm_epilogue_stages(int64_t M, int64_t N, int64_t K, fc_stage *out)
{
    if (!out) return FC_ERR_NULL;
    if (M < 1 || N < 1 || K < 1) return FC_ERR_SHAPE;
    const double mn = (double)M * (double)N;
    out[0] = fc_stage{mn, (double)M * K + (double)K * N, 2.0 * mn * (double)K, 128};
    out[1] = fc_stage{mn, (double)N, mn, 8};
    out[2] = fc_stage{mn, 0.0, 8.0 * mn, 16};
    out[3] = fc_stage{mn, mn, mn, 8};
    return FC_OK;
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
    case FC_ERR_SCRATCH: return "needs more scratch than the library's fixed no-allocation array";
    default: return "unknown status";
    }
}

extern "C" const char *fc_version(void) { return "fc 0.1.0 gfx950"; }

// Register and LDS use per kernel, the quantities behind the occupancy side of
// fusion ("C-05. Kernel Fusion 代价边界", section 2: every live value a fused
// kernel keeps costs registers per thread, and more registers per thread
// means fewer resident waves).  Served from the table build.py writes from
// the compiler's resource report of this build.
extern "C" int fc_kernel_info(const char *name, int *vgprs, int *agprs, int *sgprs, int *lds_bytes,
                              int *scratch_bytes, int *waves_per_simd)
{
    if (!name) return FC_ERR_NULL;
    for (int i = 0; i < fc::kKernelInfoCount; ++i) {
        const fc::KernelInfoRow &r = fc::kKernelInfo[i];
        if (strcmp(r.name, name) != 0) continue;
        if (vgprs) *vgprs = r.vgprs;
        if (agprs) *agprs = r.agprs;
        if (sgprs) *sgprs = r.sgprs;
        if (lds_bytes) *lds_bytes = r.lds_bytes;
        if (scratch_bytes) *scratch_bytes = r.scratch_bytes;
        if (waves_per_simd) *waves_per_simd = r.waves_per_simd;
        return FC_OK;
    }
    return FC_ERR_UNSUPPORTED;
}

extern "C" const char *fc_kernel_name(int i)
{
    return (i >= 0 && i < fc::kKernelInfoCount) ? fc::kKernelInfo[i].name : nullptr;
}
