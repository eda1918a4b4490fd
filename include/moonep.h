/*
 * moonep.h -- C ABI of the MI355X (gfx950) MoonEP hot path.
 *
 * The path (one MoE layer, all R expert-parallel ranks held as "virtual ranks"
 * in one GPU's memory):
 *
 *   moe_plan_run         router histogram + Theorem-1 planner + route map
 *   moe_plan_run_policy  the same with a choice of the donor's experts
 *   moe_prefetch_weight  copy redundant experts into prefetch rows [E, E+B)
 *   moe_dispatch         fused permute into expert-grouped [S*K, H] buffers
 *   moe_grouped_gemm     grouped GEMM over the [E+B, H, H'] weight view
 *   moe_grouped_gemm_noalloc  the same with no workspace argument
 *   moe_combine          gate-weighted unpermute back to tokens
 *   moe_grouped_gemm_wgrad  fp32 weight gradients of the grouped GEMM
 *   moe_reduce_grad      fold prefetch-slot gradients into home rows
 *
 * and its data backward:
 *
 *   moe_combine_backward    gradients of combine: permuted dy and gate grads
 *   moe_grouped_gemm_dgrad  dxperm = dy @ W^T over the same rows
 *   moe_dispatch_backward   sum each token's K permuted gradient rows
 *
 * and the deduplicated dispatch:
 *
 *   moe_route_encode     route map with repeats on a rank as -(row)-1
 *   moe_dispatch_dedup   payload once per (token, rank), then local copies
 *
 * and the two-projection SwiGLU expert:
 *
 *   moe_grouped_gemm_swiglu  first projection [E+B, H, 2H'] fused with
 *                            act = silu(gate) * up
 *   moe_swiglu_backward      gradients of the activation
 *
 * Prefetch pool ("Moonshot AI 开源 MoonEP", 核心思想: the prefetch slots come
 * from one rank-global pool shared by all layers, so the extra memory is B
 * expert weights per projection in total, not per layer).  w_pref and
 * grad_pref may be one buffer per projection shared by every layer; a slot
 * is only read when the current plan puts an expert in it, and reduce_grad
 * consumes what the weight gradient wrote, so stale contents never matter.
 * The caller keeps three orders (one stream keeps them all): a layer's
 * moe_prefetch_weight after the previous user's last moe_grouped_gemm /
 * moe_grouped_gemm_dgrad of the slots; in the backward, each layer's own
 * moe_prefetch_weight again before its moe_grouped_gemm_dgrad (the pool
 * holds another layer's experts); a layer's moe_grouped_gemm_wgrad after
 * the previous layer's moe_reduce_grad.
 *
 * Every projection of an expert is its own [E+B, H_in, H_out] weight view;
 * the GEMM, prefetch, wgrad, dgrad, combine and reduce_grad entry points take
 * the projection's widths as cfg->H (input) and cfg->Hp (output), so a down
 * projection [E+B, H', H] passes a moe_cfg with H = H' and Hp = H.  The plan
 * does not depend on H or Hp and serves every projection of the layer.
 *
 * Sources: "Kimi K3 模型结构（8）：训练并行，MoonEP 与四类等待" (blog.javazero.top),
 * "Moonshot AI 开源 MoonEP" (feinterview), "MoonEP : l'équilibrage parfait"
 * (mkdocs.reaper.mx), "大规模 LLM 训练系统研究账本" (llm-atlas); each entry
 * point cites the passage that defines it.
 *
 * Conventions for every entry point:
 *  - every pointer argument is a DEVICE pointer unless stated otherwise, and
 *    the caller allocates and owns it; the library allocates nothing and
 *    keeps no state between calls (except the fixed work-list array of
 *    moe_grouped_gemm_noalloc, described there);
 *  - every call is asynchronous on `stream` and never synchronises the host;
 *  - the return value is MOE_OK or a negative MOE_E* code, detected on the
 *    host before anything is launched (bad configuration, null pointer, a
 *    size beyond the documented limits) or reported by the HIP launch;
 *  - conditions only the device can see (expert ids outside [0, E)) set bits
 *    in plan->status instead.  Such a plan is empty: every route is -1,
 *    cu_seqlens is all zero and no prefetch slot holds an expert.  Every
 *    later step of that plan then follows its own definition with no routes
 *    and no segments: what a route, a segment or a slot addresses is not
 *    written (xperm, y, dy, dxperm, act, h13, w_pref, grad_pref, and
 *    reduce_grad changes nothing); sums over a token's routes are empty
 *    and written as zero (combine's out, dispatch_backward's dx, dgates);
 *    the weight gradient writes zero to every home row (each home segment
 *    is empty);
 *  - every bf16 and fp32 tensor argument (and every `workspace`) starts on a
 *    16-byte boundary (the kernels move 16-byte vectors); a misaligned base
 *    is MOE_EINVAL.  torch and hipMalloc allocations are 256-byte aligned;
 *  - bf16 tensors are raw IEEE bfloat16 bit patterns (moe_bf16); rounding to
 *    bf16 is round-to-nearest-even; all arrays are dense row-major.
 *
 * Notation: R ranks, S tokens per rank, E experts (E % R == 0, n = E/R home
 * experts per rank, rank r owns experts [r*n, (r+1)*n)), K distinct experts
 * per token, H hidden size, Hp = H' expert intermediate size, B prefetch slots
 * per rank.  Slot i = t*K + k is the k-th route of global token t = r*S + s.
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16;

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1, /* bad configuration, null pointer or rank range        */
  MOE_EHIP = -2,   /* a HIP launch or runtime call failed                   */
  MOE_ELIMIT = -3  /* a size beyond the limits below                        */
};

enum { MOE_MODE_TRAIN = 0, MOE_MODE_INFER = 1 };

/* Device-side status bits (plan->status[2]). */
enum {
  MOE_STATUS_BAD_ID = 1,     /* some topk id outside [0, E): plan not built */
  MOE_STATUS_UNBALANCED = 2, /* loads do not add up to R*S*K               */
  MOE_STATUS_CAPACITY = 4,   /* train mode needed more than B slots         */
  MOE_STATUS_INTERNAL = 8    /* a planner invariant failed                  */
};

/* Limits checked on the host (MOE_ELIMIT beyond them).  Besides these:
 * R*S*K < 2^31 slots, R*S < 2^24 tokens (dispatch runs one 256-thread
 * workgroup per token, and one launch holds fewer than 2^32 threads), one
 * weight matrix H*Hp*2 bytes < 4 GiB and one rank's permuted rows
 * S*K*max(H, Hp)*2 bytes < 4 GiB. */
#define MOE_MAX_E 2048
#define MOE_MAX_R 1024
#define MOE_MAX_K 64

/*
 * Layer configuration.  mode = MOE_MODE_TRAIN requires B == E/R: the planner
 * may copy up to E/R experts from one home rank, and training keeps every
 * expert the GEMM touches local ("Moonshot AI 开源 MoonEP", 核心思想, B policy).
 * mode = MOE_MODE_INFER allows 0 <= B <= E/R; redundant experts beyond B are
 * computed from their home row e of the weight view (overflow).
 * Requirements: R >= 1, S >= 0, E % R == 0, 1 <= K <= E, H % 8 == 0,
 * Hp % 8 == 0, R*S*K < 2^31.
 */
typedef struct {
  int32_t R, S, E, K, H, Hp, B, mode;
} moe_cfg;

/*
 * Plan: a bundle of caller-allocated device arrays (sizes from
 * moe_plan_sizes, in this field order).  Filled by moe_plan_run and read by
 * every later step of the same layer.
 */
typedef struct {
  int32_t *counts;      /* [E]            T_e, routes per expert              */
  int32_t *load0;       /* [R]            initial load of each rank           */
  int32_t *route;       /* [R*S*K]        destination row r*S*K + offset of
                                          slot i; -1 if the plan failed      */
  int32_t *cu_seqlens;  /* [R][E+B+1]     per-rank prefix over weight rows    */
  int32_t *slot_expert; /* [R][B]         expert held by prefetch slot, or -1 */
  int32_t *n_redundant; /* [R]            distinct remote experts received    */
  int32_t *src_rank;    /* [R]            the single donor rank, or -1        */
  int32_t *moves;       /* [E+R-1][4]     (e, dst, lo, hi) in fill order      */
  int32_t *status;      /* [4]            n_fills, n_moves, status bits, 0    */
  void *workspace;      /* opaque scratch of moe_plan_sizes()[9] bytes        */
} moe_plan;

#define MOE_PLAN_NARRAYS 10

/*
 * Host only.  Writes the byte size of each moe_plan array, in field order
 * (counts ... status, workspace), into sizes_out[0..9].  Returns MOE_EINVAL
 * or MOE_ELIMIT for a configuration the library cannot run.
 */
int moe_plan_sizes(const moe_cfg *cfg, size_t sizes_out[MOE_PLAN_NARRAYS]);

/*
 * Histogram, planner and route map ("Kimi K3 模型结构（8）", 定理 1 and
 * 在线规划、零拷贝、静态 shape; "MoonEP : l'équilibrage parfait", Le théorème).
 *
 * topk_ids [R*S][K] int32: expert ids of each token, K distinct per token.
 * Computes T_e, each rank's home load, and runs the constructive proof of
 * Theorem 1 deterministically: while a rank holds fewer than S*K slots, the
 * lowest-id such rank u is filled to exactly S*K from the rank with the
 * largest load (ties: lowest id), which gives its home experts in ascending
 * id and, inside an expert, its earliest remaining slots in (token, k)
 * order.  At most R-1 fills; every rank ends with S*K slots, receives from
 * one rank only and needs at most E/R redundant experts.  Then lays out each
 * rank's S*K buffer by weight row (ascending j in [0, E+B); ascending
 * (token, k) inside) and writes cu_seqlens, slot_expert and route.
 * Deterministic: the same ids give bit-identical outputs.
 */
int moe_plan_run(const moe_cfg *cfg, const int32_t *topk_ids,
                 const moe_plan *plan, hipStream_t stream);

/* Donor policies of moe_plan_run_policy. */
enum {
  MOE_PLAN_ASCENDING = 0,     /* as moe_plan_run                              */
  MOE_PLAN_LARGEST_FIRST = 1  /* the donor's largest remaining experts first  */
};

/*
 * moe_plan_run with a choice of which home experts a donor gives ("MoonEP :
 * l'équilibrage parfait", La planification en ligne: the online planner is a
 * near-optimal heuristic, checked against an offline integer program; Le
 * théorème: any single donor keeps the E/R bound).  MOE_PLAN_ASCENDING is
 * moe_plan_run.  MOE_PLAN_LARGEST_FIRST: within a fill, the donor gives the
 * expert with the most slots still at home in full (ties: lowest id), then
 * the next, and the last one chosen gives only the part still needed; each
 * expert still gives its earliest remaining slots, and a fill's moves are
 * listed in ascending expert id.  Receiver and donor choice, layout and
 * outputs are as for moe_plan_run.  Any other policy: MOE_EINVAL.
 */
int moe_plan_run_policy(const moe_cfg *cfg, const int32_t *topk_ids,
                        const moe_plan *plan, int32_t policy, hipStream_t stream);

/*
 * prefetch_weight ("Moonshot AI 开源 MoonEP", 核心思想: rows [E, E+B) are local
 * prefetch slots filled by buffer.prefetch_weight).  For every rank r and
 * slot b with slot_expert[r][b] = e >= 0, copies w_home[e] ([H][Hp] bf16)
 * to w_pref[r][b].  Slots holding no expert (or an id outside [0, E)) are not
 * written.
 * w_home [E][H][Hp], w_pref [R][B][H][Hp]; they must not overlap.
 */
int moe_prefetch_weight(const moe_cfg *cfg, const moe_plan *plan,
                        const moe_bf16 *w_home, moe_bf16 *w_pref,
                        hipStream_t stream);

/*
 * Fused permute ("Kimi K3 模型结构（8）", 在线规划、零拷贝、静态 shape: rows go
 * straight to expert-grouped places in a fixed S*K buffer per rank).
 * xperm[route[t*K + k]] = x[t] for every token t and k; x [R*S][H] bf16,
 * xperm [R][S*K][H] bf16.  Bit copy.  Slots with route -1 are skipped.
 */
int moe_dispatch(const moe_cfg *cfg, const moe_plan *plan, const moe_bf16 *x,
                 moe_bf16 *xperm, hipStream_t stream);

/*
 * Host only.  Bytes of scratch that moe_grouped_gemm, moe_grouped_gemm_dgrad,
 * moe_grouped_gemm_wgrad and moe_grouped_gemm_swiglu need in their
 * `workspace` argument.  The size depends on R, S, K, E and B only, so one
 * workspace serves every projection of a layer.
 */
int moe_gemm_workspace_size(const moe_cfg *cfg, size_t *bytes_out);

/*
 * Grouped GEMM over one [E+B, H, Hp] weight view addressed by row index
 * ("Moonshot AI 开源 MoonEP", 核心思想: VM grouped GEMM, cu_seqlens[E+B]
 * selects the active rows; rows [0, E) are every rank's home experts, rows
 * [E, E+B) the rank's prefetch slots).  For ranks r in [rank_begin,
 * rank_end) and rows j with cu_seqlens[r][j] < cu_seqlens[r][j+1]:
 *   y[r][cu[j]:cu[j+1]] = bf16( xperm[r][cu[j]:cu[j+1]] @ W(r, j) )
 * with W(r, j) = w_home[j] for j < E and w_pref[r][j-E] otherwise; products
 * accumulate in fp32 and round once to bf16.  xperm [R][S*K][H],
 * y [R][S*K][Hp], w_home [E][H][Hp], w_pref [R][B][H][Hp] (may be NULL when
 * B == 0), cu_seqlens [R][E+B+1] (as written by moe_plan_run).  Rows of y
 * outside the listed ranks are not written.  `workspace` holds
 * moe_gemm_workspace_size() bytes; concurrent calls need distinct ones.
 */
int moe_grouped_gemm(const moe_cfg *cfg, const moe_bf16 *xperm,
                     const moe_bf16 *w_home, const moe_bf16 *w_pref,
                     const int32_t *cu_seqlens, moe_bf16 *y,
                     int32_t rank_begin, int32_t rank_end, void *workspace,
                     hipStream_t stream);

/*
 * Allocation-free moe_grouped_gemm, for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same operation, arguments and results as moe_grouped_gemm
 * without the `workspace` argument: the work list lives in a fixed device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library (one copy per
 * device, looked up on the first call on that device and held until the
 * process ends).  The work lists of the listed ranks (one per tile height
 * class) must fit it:
 *   256 + 24 * (rank_end - rank_begin) * (ceil(S*K / 256) + 3 * (E + B))
 * bytes at most, else MOE_ELIMIT (checked on the host before any launch).
 * No call allocates or frees anything.  Every call on one device shares
 * that array, so calls that overlap on one device (on streams with no order
 * between them) race; calls on one stream are ordered and safe.  Nothing in
 * the array needs clearing between calls.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_grouped_gemm_noalloc(const moe_cfg *cfg, const moe_bf16 *xperm,
                             const moe_bf16 *w_home, const moe_bf16 *w_pref,
                             const int32_t *cu_seqlens, moe_bf16 *y,
                             int32_t rank_begin, int32_t rank_end,
                             hipStream_t stream);

/*
 * Gate-weighted combine ("Kimi K3 模型结构（8）", 在线规划、零拷贝、静态 shape:
 * each expert output is multiplied by its own fp32 router weight).
 *   out[t] = bf16( sum_{k ascending} gates[t][k] * y[route[t*K + k]] )
 * accumulated in fp32.  y [R][S*K][Hp] bf16, gates [R*S][K] fp32,
 * out [R*S][Hp] bf16.  Routes of -1 contribute nothing.
 */
int moe_combine(const moe_cfg *cfg, const moe_plan *plan, const moe_bf16 *y,
                const float *gates, moe_bf16 *out, hipStream_t stream);

/*
 * Weight gradients of the grouped GEMM, fp32 ("Moonshot AI 开源 MoonEP",
 * 核心思想: training mirrors the weight layout in fp32; rows [E, E+B) are
 * backed by a separate reduce buffer).  Train mode only.  For every rank r:
 *   grad_home[j]   = xperm_seg(r, j)^T @ dy_seg(r, j)  for r's home rows j
 *                    (overwritten; zero when the segment is empty)
 *   grad_pref[r][b] = the same for row E+b, for every slot b holding an
 *                    expert; other slots are not written.
 * xperm [R][S*K][H] bf16, dy [R][S*K][Hp] bf16, grad_home [E][H][Hp],
 * grad_pref [R][B][H][Hp].  `workspace` as for moe_grouped_gemm.
 * Hp must stay at or below 1398101 (a 384-row tile of one gradient then
 * spans less than 2 GiB, the reach of the stores' 32-bit offsets), else
 * MOE_ELIMIT.
 */
int moe_grouped_gemm_wgrad(const moe_cfg *cfg, const moe_plan *plan,
                           const moe_bf16 *xperm, const moe_bf16 *dy,
                           float *grad_home, float *grad_pref,
                           void *workspace, hipStream_t stream);

/*
 * reduce_grad ("Moonshot AI 开源 MoonEP", 核心思想: each rank reads its own
 * experts' slots from every rank, accumulates them into its parameter
 * gradient and zeroes the consumed slots).  For every expert e:
 *   grad_home[e] += sum over ranks r ascending of grad_pref[r][b],
 *                   slot_expert[r][b] == e
 * in fp32, then every slot with slot_expert >= 0 is set to zero; other slots
 * are untouched.
 */
int moe_reduce_grad(const moe_cfg *cfg, const moe_plan *plan, float *grad_home,
                    float *grad_pref, hipStream_t stream);

/*
 * Gradients of combine ("大规模 LLM 训练系统研究账本" §9.5: the MoE backward
 * works on the permuted layout; the gradient of the gate-weighted sum in
 * "Kimi K3 模型结构（8）", 在线规划、零拷贝、静态 shape).  For every token t
 * and k with q = route[t*K + k] >= 0:
 *   dy[q]          = bf16( gates[t][k] * dout[t] )   (exact product, rounded once)
 *   dgates[t][k]   = sum_h dout[t][h] * y[q][h]      (fp32)
 * dgates[t][k] = 0 for routes of -1.  dout [R*S][Hp] bf16, y [R][S*K][Hp]
 * bf16 (the forward GEMM output), gates [R*S][K] fp32, dy [R][S*K][Hp] bf16,
 * dgates [R*S][K] fp32.  Rows of dy no route names are not written.
 */
int moe_combine_backward(const moe_cfg *cfg, const moe_plan *plan,
                         const moe_bf16 *dout, const moe_bf16 *y,
                         const float *gates, moe_bf16 *dy, float *dgates,
                         hipStream_t stream);

/*
 * Data gradient of the grouped GEMM ("大规模 LLM 训练系统研究账本" §9.5: the
 * group GEMM backward runs over the rows that dispatch laid out).  For ranks
 * r in [rank_begin, rank_end) and rows j with cu_seqlens[r][j] <
 * cu_seqlens[r][j+1]:
 *   dxperm[r][cu[j]:cu[j+1]] = bf16( dy[r][cu[j]:cu[j+1]] @ W(r, j)^T )
 * with W(r, j) as for moe_grouped_gemm; fp32 accumulation, one rounding.
 * dy [R][S*K][Hp], dxperm [R][S*K][H].  Rows outside the listed ranks are
 * not written.  `workspace` as for moe_grouped_gemm.
 */
int moe_grouped_gemm_dgrad(const moe_cfg *cfg, const moe_bf16 *dy,
                           const moe_bf16 *w_home, const moe_bf16 *w_pref,
                           const int32_t *cu_seqlens, moe_bf16 *dxperm,
                           int32_t rank_begin, int32_t rank_end,
                           void *workspace, hipStream_t stream);

/*
 * Gradient of dispatch ("大规模 LLM 训练系统研究账本" §9.5, as for
 * moe_combine_backward): every token's input gradient is the sum of the
 * gradients of its K permuted copies,
 *   dx[t] = bf16( sum_{k ascending} dxperm[route[t*K + k]] )
 * accumulated in fp32.  dxperm [R][S*K][H] bf16, dx [R*S][H] bf16.  Routes
 * of -1 contribute nothing.
 */
int moe_dispatch_backward(const moe_cfg *cfg, const moe_plan *plan,
                          const moe_bf16 *dxperm, moe_bf16 *dx,
                          hipStream_t stream);

/*
 * Dedup encoding of the route map ("Kimi K3 模型结构（8）", 在线规划、零拷贝、
 * 静态 shape: a route entry holds its write position on the destination rank;
 * an entry whose rank already appeared among the same token's earlier
 * entries holds -(position) - 1 instead, so the sender skips its payload).
 * With q = route[t*K + k] and rank d = q / (S*K), for k ascending:
 *   route_enc[t*K + k] = q            if no k' < k of token t has rank d
 *                      = -q - 1       otherwise
 *                      = INT32_MIN    if q < 0 (no plan)
 * route_enc [R*S][K] int32 (caller-allocated, device).
 */
int moe_route_encode(const moe_cfg *cfg, const moe_plan *plan, int32_t *route_enc,
                     hipStream_t stream);

/*
 * Dispatch driven by route_enc (same source): a send pass writes each
 * token's row once per destination rank (entries >= 0); a receive pass then
 * copies, on each rank, the row that arrived for the token into every row
 * -(e) - 1 of that token on that rank.  The result equals moe_dispatch's
 * bit for bit.  x [R*S][H], xperm [R][S*K][H] bf16.
 */
int moe_dispatch_dedup(const moe_cfg *cfg, const int32_t *route_enc,
                       const moe_bf16 *x, moe_bf16 *xperm, hipStream_t stream);

/*
 * First projection of a two-projection SwiGLU expert ("Moonshot AI 开源
 * MoonEP", 核心思想: each expert projection is one contiguous [E+B, H, H']
 * tensor addressed by row index; H' is the expert FFN's intermediate size).
 * cfg->Hp = H'.  W13(r, j) = [W_gate | W_up] is [H][2H'] bf16 (gate columns
 * [0, H'), up columns [H', 2H')), from w13_home [E][H][2H'] for j < E and
 * w13_pref [R][B][H][2H'] otherwise (fill it with moe_prefetch_weight and a
 * cfg whose Hp is 2H').  For ranks r in [rank_begin, rank_end) and every
 * non-empty segment j, with fp32 accumulation:
 *   gate = xperm_seg @ W_gate,  up = xperm_seg @ W_up
 *   act[r][cu[j]:cu[j+1]] = bf16( silu(gate) * up ),  silu(z) = z / (1 + e^-z)
 *   h13[r][cu[j]:cu[j+1]] = [ bf16(gate) | bf16(up) ]  (only if h13 != NULL)
 * act [R][S*K][H'], h13 [R][S*K][2H'] (kept for moe_swiglu_backward),
 * xperm [R][S*K][H].  Rows outside the listed ranks are not written.
 * `workspace` as for moe_grouped_gemm.  Requires H * H' * 4 < 2^32
 * (else MOE_ELIMIT).
 */
int moe_grouped_gemm_swiglu(const moe_cfg *cfg, const moe_bf16 *xperm,
                            const moe_bf16 *w13_home, const moe_bf16 *w13_pref,
                            const int32_t *cu_seqlens, moe_bf16 *act, moe_bf16 *h13,
                            int32_t rank_begin, int32_t rank_end, void *workspace,
                            hipStream_t stream);

/*
 * Gradients of the SwiGLU activation (same source; act = silu(gate) * up).
 * cfg->Hp = H'.  For all R*S*K rows, from the stored h13 = [gate | up] and
 * dact, with s = 1 / (1 + e^-gate) computed in fp32:
 *   dh13[:, :H'] = bf16( dact * up * s * (1 + gate * (1 - s)) )   (d gate)
 *   dh13[:, H':] = bf16( dact * gate * s )                        (d up)
 * h13, dh13 [R][S*K][2H'] bf16, dact [R][S*K][H'] bf16.  dh13 may be h13
 * (in place); it must not overlap dact otherwise.
 */
int moe_swiglu_backward(const moe_cfg *cfg, const moe_bf16 *h13, const moe_bf16 *dact,
                        moe_bf16 *dh13, hipStream_t stream);

/* Host only.  Static text for a MOE_* return code. */
const char *moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_H */
