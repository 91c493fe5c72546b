/*
 * fc.h -- C ABI of the fused-chain library for AMD Instinct MI355X (gfx950).
 *
 * Vertical fusion of three operator chains: intermediates stay in VGPRs or
 * LDS instead of making HBM round trips.
 *
 * Conventions for every entry point:
 *  - Plain C types only; no exceptions cross the boundary.
 *  - The caller owns all memory.  Device pointers must point to device memory
 *    of the current HIP device; "host" pointers to ordinary host memory.
 *  - The library never allocates, frees or synchronises.  Compute entry points
 *    validate their arguments synchronously, before any HIP call, then enqueue
 *    kernels on `stream` (NULL = the null stream) and return.
 *  - Layouts are row-major and contiguous.
 *  - Return value: FC_OK or one of the negative FC_ERR_* codes.  On any
 *    validation error nothing is enqueued.  FC_ERR_HIP means a launch failed
 *    (hipGetLastError after the launch); the stream state is then undefined.
 *  - The library keeps no state; every entry point is re-entrant.
 */
#ifndef FC_H
#define FC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *fc_stream;   /* the same type as hipStream_t */

enum {
    FC_OK = 0,
    FC_ERR_NULL = -1,         /* a required pointer is NULL                      */
    FC_ERR_SHAPE = -2,        /* a size is negative or zero where not allowed     */
    FC_ERR_ALIGN = -3,        /* a pointer is not 16-byte aligned                 */
    FC_ERR_PLAN = -4,         /* split plan is not a composition of 4             */
    FC_ERR_UNSUPPORTED = -5,  /* valid but unsupported (K stages, tile, temps...) */
    FC_ERR_WORKSPACE = -6,    /* workspace missing or smaller than required       */
    FC_ERR_HIP = -7,          /* a HIP launch failed                              */
    FC_ERR_ALIAS = -8,        /* buffers overlap where they must not              */
    FC_ERR_SCRATCH = -9       /* a no-allocation call needs more scratch than the
                                 library's fixed array holds                      */
};

enum { FC_CHAIN_NAIVE = 0, FC_CHAIN_FUSED = 1, FC_CHAIN_FAT = 2 };
enum { FC_SOFTMAX_FUSED = 0, FC_SOFTMAX_UNFUSED = 1 };
enum { FC_RMSNORM_FUSED = 0, FC_RMSNORM_UNFUSED = 1 };

#define FC_CHAIN_MAX_STAGES 32

/* ------------------------------------------------------------------ chain */

/*
 * fc_chain -- K-stage pointwise chain ("C-05. Kernel Fusion 代价边界", section 3,
 * the API / experiment-form table and the stage operation under it):
 *     for s = 0 .. K-1:  y = a[s] * y + b[s];  if (relu_even && s % 2 == 0) y = max(y, 0)
 * Every stage is one fused multiply-add (a single rounding) in fp32, so the
 * three modes produce bit-identical y.
 *
 *  x        device, fp32 [n], 16-byte aligned.  May equal y (in place); any
 *           other overlap with y is undefined.
 *  y        device, fp32 [n], 16-byte aligned.
 *  n        number of elements, n >= 0 (n == 0 enqueues nothing).
 *  a, b     HOST arrays of K fp32 coefficients, copied into the launch.
 *  K        1 .. FC_CHAIN_MAX_STAGES.
 *  mode     FC_CHAIN_NAIVE: K launches, stage s reads the previous stage's
 *                 buffer and writes the other (ping-pong between y and
 *                 scratch, the last stage lands in y);
 *           FC_CHAIN_FUSED: one launch, all K stages in registers;
 *           FC_CHAIN_FAT:   FUSED plus `fat_temps` live fp32x4 temporaries per
 *                 lane, reduced into a sink so they cannot be eliminated (a
 *                 register-pressure probe, not a production form).
 *  scratch  device, fp32; NAIVE with K >= 2: n floats, 16-byte aligned, must
 *           not overlap x or y.  FAT: the sink, fc_chain_scratch_floats()
 *           floats.  FUSED: ignored (may be NULL).
 *  fat_temps  FAT only: one of 0, 16, 48, 96, 128; FAT supports K in {1,2,3,4,6,8}.
 */
int fc_chain(const float *x, float *y, int64_t n, const float *a, const float *b, int K,
             int relu_even, int mode, float *scratch, int fat_temps, fc_stream stream);

/* Floats of scratch fc_chain needs for (n, K, mode, fat_temps); 0 if none.
 * NAIVE with K >= 2: n (the second ping-pong buffer of "C-05", section 3, API
 * table, naive row).  FAT: 4 * L, one fp32x4 sink entry per lane of the
 * launch, L = 256 * min(2048, max(1, ceil(floor(n/4) / 256))); lane l visits
 * the fp32x4 vectors q = l, l + L, l + 2L, ... of x (the n mod 4 trailing
 * elements are computed without temporaries and do not enter the sink) and
 * writes sink[4l .. 4l+3] = per component, the sum over its vectors of
 * t_0 + (t_1 + (... + t_{T-1})), where t_j = fmaf(0.5, t_{j-1}, y_{s(j)}),
 * t_{-1} = 0, y_s the element's chain value after stage s and its ReLU and
 * s(j) = floor(j*K/T) (the fat row of the same table gives no formula; this
 * one keeps all T temporaries live).  FUSED: 0. */
size_t fc_chain_scratch_floats(int64_t n, int K, int mode, int fat_temps);

/* -------------------------------------------------------- GEMM + epilogue */

/*
 * fc_gemm_epilogue -- Y = GELU(A.B + bias) + R, the four-operator chain
 * mm -> bias -> gelu -> res of "K4 讲解：fusion 的三笔账", section 1, cut into
 * kernels by a split plan.  GELU is the erf form 0.5*z*(1 + erf(z/sqrt(2))).
 *
 *  A     device fp16 [M,K];  B device fp16 [K,N];  bias device fp16 [N];
 *  R     device fp16 [M,N];  Y device fp16 [M,N] (must not overlap A, B,
 *        bias or R).  All 16-byte aligned.
 *  M >= 1; N >= 8 and K >= 8, both multiples of 8.
 *  plan  HOST array of plan_len positive segment lengths summing to 4, e.g.
 *        {1,1,1,1}, {1,3}, {2,2}, {4}; all 8 compositions are accepted.  Each
 *        segment is one kernel: the first is the MFMA GEMM with the
 *        segment's operators applied on the accumulator registers; later
 *        segments are pointwise kernels.  At every cut the running value is
 *        rounded to fp16 and written to the workspace, and the next kernel
 *        reads it back.  Arithmetic is fp32 between cuts; Y is rounded to fp16
 *        (round to nearest even).
 *  workspace  device, >= fc_gemm_workspace_bytes() bytes, 16-byte aligned
 *        (NULL allowed when that is 0), not overlapping any operand.  Layout:
 *        first, for shapes that take a split-K kernel (see
 *        fc_gemm_workspace_bytes), arrival counters and fp32 partial sums (D
 *        bytes, where D = fc_gemm_workspace_bytes(M, N, K, {4}, 1)); then, when
 *        the plan
 *        has a cut, the fp16 intermediate (round_up(2*M*N, 256) bytes at byte
 *        offset D): after a plan whose first segment is the bare GEMM it holds
 *        C = A.B until the next segment overwrites it in place.  The counters
 *        must be zero when a call starts: hand in a zero-filled workspace the
 *        first time; every call that completes leaves them zero again, so one
 *        workspace serves any number of calls of one (M, N, K), under any
 *        plan, without clearing.  Clear it again after using it for anything
 *        else (another shape, other data).  Calls that overlap in time
 *        (different streams) must not share a workspace.
 *
 *  Returns FC_OK, or FC_ERR_PLAN / FC_ERR_SHAPE / FC_ERR_UNSUPPORTED (N or
 *  K not a multiple of 8) / FC_ERR_NULL / FC_ERR_ALIGN / FC_ERR_ALIAS /
 *  FC_ERR_WORKSPACE (missing or too small) before anything is launched, or
 *  FC_ERR_HIP if a launch fails.  The caller owns every buffer; the call is
 *  asynchronous on `stream`.
 */
int fc_gemm_epilogue(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                     const uint16_t *R, uint16_t *Y, int M, int N, int K,
                     const int *plan, int plan_len, void *workspace, size_t ws_bytes,
                     fc_stream stream);

/* Bytes of workspace for (M, N, K, plan) ("K4 讲解", section 1: every cut of
 * a plan writes one [M,N] fp16 intermediate that the next kernel reads back;
 * the split-K scratch is this library's own): D + round_up(2*M*N, 256) when the
 * plan has a cut, else D, the split-K scratch of the GEMM kernel the shape
 * takes (0 when it takes no split):
 *  - M <= 64, N % 64 == 0, K % 256 == 0: the decode kernel, MB = 1, 2 or 4
 *    blocks of 16 rows (M <= 16, <= 32, <= 64) and K split into P parts, P
 *    the smallest power of two up to 64 with 256*P dividing K,
 *    K <= 256*S*P (S = 4 k-steps per wave for MB <= 2, 2 for MB = 4) and
 *    (N/64)*P >= 512, else the largest one meeting the first two conditions;
 *    D = round_up(4*N/64, 256) + 64*N*P*MB when P > 1;
 *  - otherwise, K % 64 == 0 and T = ceil(M/128)*ceil(N/128) <= 512: the
 *    128x128 ring kernel over those T tiles, K split P ways when
 *    T < 128 (P the smallest power of two up to 16 with T*P >= 128, 64*P
 *    dividing K and K/P >= 256, else the largest one meeting the last two);
 *    D = round_up(4*T, 256) + 65536*T*P when P > 1.
 * 0 for an invalid plan or shape (fc_gemm_epilogue then returns an error). */
size_t fc_gemm_workspace_bytes(int M, int N, int K, const int *plan, int plan_len);

/*
 * fc_gemm_epilogue_noalloc -- fc_gemm_epilogue without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * allocates nothing and calls no allocating routine: the split-K scratch and
 * the fp16 intermediate of a cut plan live in a fixed array of
 * FC_GEMM_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device,
 * held until the process ends.  Same kernels, same results as
 * fc_gemm_epilogue (bit for bit) and the same arguments without workspace and
 * ws_bytes.
 *
 *  Limit: calls whose fc_gemm_workspace_bytes(M, N, K, plan) exceeds
 *  FC_GEMM_NOALLOC_SCRATCH_BYTES return FC_ERR_SCRATCH before anything is
 *  launched (e.g. any plan with a cut needs 2*M*N bytes for its intermediate,
 *  so M*N <= 32M elements less the split scratch).
 *  Every call on a device shares that device's array: the call clears the
 *  arrival counters it needs (a small fill kernel on `stream`, no memset) and
 *  overwrites the rest, so back-to-back calls of any shapes need nothing from
 *  the caller, but calls that overlap in time on one device (different
 *  streams or host threads without ordering) race and give undefined results.
 *  The array used is the current device's: `stream` must belong to the
 *  current device (FC_ERR_UNSUPPORTED otherwise, before any launch).  The
 *  first call on a device looks the array's address up with that device
 *  current (FC_ERR_HIP if that fails).  Other errors as fc_gemm_epilogue.
 */
#define FC_GEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fc_gemm_epilogue_noalloc(const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                             const uint16_t *R, uint16_t *Y, int M, int N, int K,
                             const int *plan, int plan_len, fc_stream stream);

/* ---------------------------------------------------- causal softmax */

/*
 * fc_causal_softmax -- causal scaled-masked softmax over attention scores
 * ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5, causal mask and
 * block skipping; appendix attention-tail section, the five steps).  For
 * every row (bh, i) with z_j = scale * scores[bh, i, j]:
 *     out[bh, i, j] = exp(z_j - max_{k<=i} z_k) / sum_{k<=i} exp(z_k - max) for j <= i,
 *     out[bh, i, j] = 0 exactly for j > i.
 *
 *  scores  device bf16 [BH, S, S];  out device bf16 [BH, S, S] (round to
 *          nearest even; must not overlap scores).  16-byte aligned.
 *  BH >= 1, S >= 1.
 *  tile    FUSED: key-tile edge for block skipping, 64, 128, 256, or S (no
 *          skipping).  Row i loads only key tiles 0 .. floor(i/tile); the rest
 *          of the row is written as zeros without being read.  UNFUSED: ignored.
 *  mode    FC_SOFTMAX_FUSED: one kernel, one pass over the kept tiles.
 *          FC_SOFTMAX_UNFUSED: the five-step baseline -- row max of scale*s over
 *          the kept keys (the whole row is read); x = scale*s - max; e = exp(x)
 *          where the mask is 1, else 0; row sum; e/sum -- each step its own
 *          kernel, bf16 intermediates in `out`, fp32 row statistics, and a
 *          materialised bf16 0/1 mask.  Masked scores never reach the result,
 *          whatever they hold (inf and NaN included).
 *  workspace  UNFUSED: device, >= fc_softmax_workspace_bytes() bytes, laid out
 *          as [mask bf16 BH*S*S, padded to a multiple of 256 bytes]
 *          [row max fp32 BH*S][row sum fp32 BH*S]; the
 *          mask part must have been filled by fc_causal_mask_materialise()
 *          for the same (BH, S).  FUSED: ignored (may be NULL).
 */
int fc_causal_softmax(const uint16_t *scores, uint16_t *out, int64_t BH, int S, float scale,
                      int tile, int mode, void *workspace, size_t ws_bytes, fc_stream stream);

/* The fused kernel with fp32 output (same arithmetic; only the store type
 * differs).  out: device fp32 [BH, S, S], 16-byte aligned. */
int fc_causal_softmax_f32out(const uint16_t *scores, float *out, int64_t BH, int S, float scale,
                             int tile, fc_stream stream);

/* The fused kernel, also writing for every row the number of key tiles it
 * loaded (device int32 [BH*S]).  For checking block skipping. */
int fc_causal_softmax_tiles(const uint16_t *scores, uint16_t *out, int32_t *tiles_per_row,
                            int64_t BH, int S, float scale, int tile, fc_stream stream);

/* The unfused baseline's materialised mask ("AIGC 基本功", appendix byte
 * ledger, attention-tail entry: five score-sized steps plus one materialised
 * mask of the score tensor's size): writes bf16 1.0 where key j <= query i
 * and 0.0 where j > i into mask [BH, S, S] (device, 16-byte aligned; the
 * first part of the UNFUSED workspace).  BH >= 1, S >= 1; FC_ERR_NULL /
 * FC_ERR_SHAPE / FC_ERR_ALIGN before any launch, FC_ERR_HIP if it fails. */
int fc_causal_mask_materialise(uint16_t *mask, int64_t BH, int S, fc_stream stream);

/* Workspace of fc_causal_softmax: UNFUSED round_up(2*BH*S*S, 256) + 8*BH*S
 * bytes (the materialised mask of the appendix ledger's attention-tail entry,
 * then the fp32 row max and row sum the five steps pass between kernels);
 * FUSED 0.  0 for invalid arguments. */
size_t fc_softmax_workspace_bytes(int64_t BH, int S, int mode);

/* ------------------------------------------------------------ causal attention */

/*
 * fc_causal_attention -- O = softmax(scale * Q K^T under the causal mask) V in
 * one kernel that never writes the scores: key/value tiles stream through the
 * chip while an online softmax keeps each query row's running max and sum
 * ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5: query i sees keys
 * j <= i, and key tiles wholly above the diagonal are skipped; its further-
 * reading list names this online-softmax kernel as the way to remove the
 * S x S score tensor).
 *
 *  Q, K, V  device bf16 [BH, S, D] row-major (head-major rows), 16-byte aligned.
 *  O        device bf16 [BH, S, D], must not overlap Q, K or V.
 *  D        128 (FC_ERR_UNSUPPORTED otherwise); 1 <= S <= 2^22 (any length:
 *           the last tiles are ragged; longer S returns FC_ERR_UNSUPPORTED);
 *           BH >= 1; scale finite and > 0 (the pages' 1/sqrt(128);
 *           FC_ERR_SHAPE otherwise).
 *  Arithmetic: fp32 accumulation of the products; the softmax in fp32 (base-2
 *  exponent of scale*log2(e) times the score minus a running reference that
 *  trails the row max by at most 8 in the exponent, so probabilities are <= 2^8);
 *  the probabilities are rounded to bf16
 *  before their product with V and the row sum adds those rounded values, so
 *  the weights applied to V sum to one; O is rounded to bf16 (round to
 *  nearest even).
 *
 *  Returns FC_OK, or FC_ERR_SHAPE / FC_ERR_UNSUPPORTED / FC_ERR_NULL /
 *  FC_ERR_ALIGN / FC_ERR_ALIAS before anything is launched, or FC_ERR_HIP if
 *  the launch fails.  No workspace; asynchronous on `stream`.
 */
int fc_causal_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O,
                        int64_t BH, int S, int D, float scale, fc_stream stream);

/* Algorithmic work of fc_causal_attention: flops of the two products over the
 * kept (j <= i) pairs, 2*D*S*(S+1)*BH; DRAM bytes with Q, K, V read once and O
 * written once, 8*BH*S*D.  0 for invalid arguments. */
uint64_t fc_attention_flops(int64_t BH, int S, int D);
uint64_t fc_attention_bytes(int64_t BH, int S, int D);

/* ------------------------------------------------------------ RMSNorm */

/*
 * fc_rmsnorm -- y[i][j] = x[i][j] / sqrt(mean_j x[i][j]^2 + eps) * g[j], fp32
 * ("AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.2 byte ledger and the
 * appendix ledger's RMSNorm entry: square, mean, multiply by the reciprocal
 * root, multiply by the gain; four passes unfused, one fused).
 *
 *  x, y   device fp32 [rows, d] row-major; g device fp32 [d]; all 16-byte
 *         aligned; y must not overlap x or g.
 *  rows >= 1; d a multiple of 4 with 4 <= d <= 16384 (FC_ERR_UNSUPPORTED
 *  otherwise); eps finite and >= 0.
 *  mode   FC_RMSNORM_FUSED: one kernel, one workgroup per row, the row held in
 *         registers; x read once, y written once.  No workspace.
 *         FC_RMSNORM_UNFUSED: the four passes as four kernels through the
 *         workspace (squares, then row means, then x times the reciprocal
 *         root written over the squares, then the gain).
 *  workspace  device, >= fc_rmsnorm_workspace_bytes() bytes, 16-byte aligned,
 *         not overlapping x, g or y (NULL allowed for FUSED).
 *  Every sum, root and product is fp32; the 1/sqrt is correctly rounded.
 *  Returns FC_OK or an error code before anything is launched (FC_ERR_HIP if
 *  a launch fails).
 */
int fc_rmsnorm(const float *x, const float *g, float *y, int64_t rows, int d, float eps, int mode,
               void *workspace, size_t ws_bytes, fc_stream stream);

/* UNFUSED: round_up(4*rows*d, 256) + 4*rows bytes; FUSED: 0. */
size_t fc_rmsnorm_workspace_bytes(int64_t rows, int d, int mode);

/* The appendix ledger's bytes: every pass reads and writes the n = rows*d
 * fp32 tensor once, so FUSED 8n and UNFUSED 4 * 8n (the gain vector and the
 * per-row statistics are not counted).  0 for invalid arguments. */
uint64_t fc_rmsnorm_bytes(int64_t rows, int d, int mode);

/* ------------------------------------------------------------ accounting */

/*
 * Algorithmic DRAM bytes and launches, pure host integer functions (no device).
 *
 * fc_plan_bytes: bytes of a split plan of the GEMM epilogue chain ("K4 讲解",
 *   section 1): every external operand (A, B, bias, R) is read once, Y written
 *   once, and every cut writes one [M,N] intermediate and reads it back:
 *     elem_bytes * (M*K + K*N + N + 2*M*N + 2*cuts*M*N);  0 for an invalid plan.
 * fc_plan_launches: number of segments; 0 for an invalid plan.
 * fc_chain_bytes: fp32 chain, NAIVE 8*K*n, FUSED and FAT 8*n (the fat sink is
 *   probe overhead and not counted) ("AIGC 基本功", section 3.2).
 * fc_softmax_bytes: FUSED reads each row's kept tiles and writes the whole
 *   output: 2*(BH*sum_i min(S, (floor(i/tile)+1)*tile) + BH*S*S);
 *   UNFUSED 2*BH*S*S*(8 + 1 mask) + 16*BH*S (fp32 row statistics written and
 *   read once each).  0 for invalid arguments.
 */
uint64_t fc_plan_bytes(int64_t M, int64_t N, int64_t K, const int *plan, int plan_len,
                       int elem_bytes);
int fc_plan_launches(const int *plan, int plan_len);
uint64_t fc_chain_bytes(int64_t n, int K, int mode);
uint64_t fc_softmax_bytes(int64_t BH, int S, int tile, int mode);

/* ------------------------------------------------------------ cost model */

/*
 * The split-plan time model of "K4 讲解：fusion 的三笔账", section 2 (its time
 * estimate and best-plan search), host only.  A chain is a list of stages; a
 * plan cuts it into segments, one kernel each.  A segment's time is
 *   max(bytes / hbm_bytes_per_s * factor(live registers), flops / flops_per_s)
 *   + launch_s
 * where bytes = elem_bytes * (its stages' external reads + the intermediate
 * written by the previous segment + its own one output), and the live
 * registers are the sum over its stages.  factor(r) = mem_factor[i] for the
 * first level with r <= reg_level[i], else spill_factor; the pages' model is
 * one level {255: 1.0} and spill_factor 3.
 */
#define FC_COST_MAX_LEVELS 8
#define FC_COST_MAX_STAGES 16
typedef struct {
    double writes;      /* elements the stage writes */
    double ext_reads;   /* elements it reads from outside the chain (weights, bias, residual) */
    double flops;
    int live_regs;      /* registers the stage keeps live when fused */
} fc_stage;
typedef struct {
    double hbm_bytes_per_s;
    double flops_per_s;
    double launch_s;                        /* per-kernel cost */
    int n_levels;                           /* 0 .. FC_COST_MAX_LEVELS, reg_level strictly increasing */
    int reg_level[FC_COST_MAX_LEVELS];
    double mem_factor[FC_COST_MAX_LEVELS];
    double spill_factor;                    /* factor beyond the last level */
} fc_cost_model;

/* Estimated seconds of a plan (a composition of n_stages, 1 <= n_stages <=
 * FC_COST_MAX_STAGES); -1 for invalid arguments. */
double fc_segments_time(const fc_stage *stages, int n_stages, const int *plan, int plan_len,
                        int elem_bytes, const fc_cost_model *model);

/* The plan with the least estimate over all 2^(n_stages-1) compositions
 * (the first one in cut-mask order on ties): plan_out (host, >= n_stages
 * ints), *plan_len_out, and *t_out (may be NULL).  FC_OK or an error code. */
int fc_best_split(const fc_stage *stages, int n_stages, int elem_bytes, const fc_cost_model *model,
                  int *plan_out, int *plan_len_out, double *t_out);

/* The four stages of the GEMM epilogue chain for (M, N, K) into out[4]. */
int fc_gemm_epilogue_stages(int64_t M, int64_t N, int64_t K, fc_stage *out);

/* ------------------------------------------------------ kernel resources */

/*
 * fc_kernel_info -- registers and LDS of one kernel of this library as built,
 * the quantities that set occupancy ("C-05. Kernel Fusion 代价边界", section 2:
 * a fused kernel pays for every value it keeps live in registers per thread,
 * and fewer resident waves follow).  Values come from the compiler's resource
 * report of this build, compiled into the library: vector registers (VGPRs),
 * accumulation registers (AGPRs), scalar registers, static LDS bytes per
 * workgroup, scratch bytes per lane (non-zero means spills) and the waves per
 * SIMD the register and LDS use allow.
 *
 *  name     the kernel's demangled name without its parameter list, e.g.
 *           "fc::attention_fwd_kernel" or "fc::chain_fat_kernel<4, true, 48>";
 *           fc_kernel_name() lists every name.
 *  outputs  host ints; any of them may be NULL.
 * Host only: never touches the device.  Returns FC_OK, FC_ERR_NULL (name is
 * NULL) or FC_ERR_UNSUPPORTED (no kernel of that name).
 */
int fc_kernel_info(const char *name, int *vgprs, int *agprs, int *sgprs, int *lds_bytes,
                   int *scratch_bytes, int *waves_per_simd);

/* Name of kernel i (0-based, sorted by name) for fc_kernel_info, or NULL when
 * i is out of range.  The string is static. */
const char *fc_kernel_name(int i);

/* Static text for a status code. */
const char *fc_status_string(int status);

/* Library version string. */
const char *fc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FC_H */
