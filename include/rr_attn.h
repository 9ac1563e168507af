/*
 * rr_attn.h - C ABI of the response-replay attention library for AMD MI355X (gfx950).
 *
 * The library computes, on one GPU, the attention of a replayed response over a
 * stop-gradient resident prompt KV cache plus the response's own causal KV, and its
 * response-only backward:
 *
 *   - Resident prompt state z_p = stopgrad(z_p(theta)) kept as model-native KV pages,
 *     responses replayed against it under autograd:
 *     ai.thesatyajit.com/articles/longstraw-2m-rl, section "The move: change the graph
 *     boundary".  The direct response gradient is kept; the prompt-side term through
 *     z_p(theta) is dropped (same section).
 *   - Attention over sharded KV pages with rank-local softmax statistics composed into
 *     the exact global output; response blocks replayed in reverse; K/V gradient
 *     storage only for what a response backward touches: same page, section "Two
 *     incompatible architectures, same transaction".  On one GPU the prompt chunks play
 *     the part of the ranks.
 *   - Serial replay (G members, one at a time) accumulated up to one update, with
 *     versioned resident state and retry / drop hazards:
 *     networkfinds.com/long-context-rl-is-a-state-lifetime-problem, sections "Account
 *     for memory by lifetime" and "Preserve gradient semantics, not just forward
 *     outputs"; ai.thesatyajit.com/articles/longstraw-2m-rl, section "Serial replay
 *     makes G a schedule, not a memory multiplier".
 *   - Problem sizes P (prompt), R (response), G (group), K (replay microbatch):
 *     networkfinds.com/long-context-rl-is-a-state-lifetime-problem, sections "Why
 *     inference capacity does not imply training capacity" and "Make the prompt
 *     resident and the learning graph selective".
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays unless marked
 *     "host".  The caller owns every buffer; the library allocates and frees no device
 *     memory and keeps no state between calls, except the optional profiling state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Kernels are launched
 *     asynchronously on it; no entry point synchronises except rr_profile_end.
 *   - Every argument is validated before the first launch.  A non-zero return means
 *     nothing was launched (except RR_E_HIP, raised by a failing launch);
 *     rr_last_error() returns a thread-local message describing the failure.  After the
 *     shape checks, every non-NULL tensor pointer is looked up with
 *     hipPointerGetAttributes: memory the GPU cannot access (plain host memory) returns
 *     RR_E_PTR instead of faulting in a kernel.  Host memory pinned through HIP passes.
 *   - Layouts (K = responses in the microbatch, R = R_max = row stride):
 *       q      [K][R][Hq][d_qk]   dtype           (latent: same)
 *       k_r    [K][R][Hkv][d_qk]  dtype           (latent: response latent rows [K][R][d_qk])
 *       v_r    [K][R][Hkv][d_v]   dtype           (latent: NULL; V = first d_v dims of k_r)
 *       d_o    [K][R][Hq][d_v]    dtype
 *       o      [K][R][Hq][d_v]    fp32
 *       lse    [K][R][Hq]         fp32, natural log of the softmax normaliser
 *       dq     [K][R][Hq][d_qk]   fp32
 *       dk_r   [K][R][Hkv][d_qk]  fp32            (latent: [K][R][d_qk])
 *       dv_r   [K][R][Hkv][d_v]   fp32            (latent: [K][R][d_v])
 *       resident K_p [P][Hkv][d_qk], V_p [P][Hkv][d_v] dtype (latent: rows [P][d_qk])
 *     Query head h reads KV head h / (Hq / Hkv).  Row i of response k is valid when
 *     i < r_len[k]; it sees every prompt position and response positions 0..i.
 *     Rows i >= r_len[k] are padding: the forward writes O = 0 and lse = -inf there and
 *     the backward writes (or adds) zero gradients there.
 */
#ifndef RR_ATTN_H
#define RR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------------- */
#define RR_OK              0
#define RR_E_NULL         -1  /* a required pointer is NULL                           */
#define RR_E_SHAPE        -2  /* sizes inconsistent (Hq % Hkv, r_len > R_max, ...)     */
#define RR_E_UNSUPPORTED  -3  /* valid but not built: head dims, dtype combination    */
#define RR_E_WORKSPACE    -4  /* ws NULL or ws_bytes below rr_workspace_bytes()       */
#define RR_E_RANGE        -5  /* member index outside [0, G)                          */
#define RR_E_DUPLICATE    -6  /* member already accumulated in this window (a retry)  */
#define RR_E_STALE        -7  /* gradients of another model version or prompt group   */
#define RR_E_MISSING      -8  /* a member of the window was never accumulated         */
#define RR_E_HIP          -9  /* a HIP call failed; see rr_last_error()               */
#define RR_E_PTR         -10  /* a tensor pointer is memory the GPU cannot access     */
#define RR_E_POISONED    -11  /* an accumulation launch failed part-way: the window's
                                 accumulators hold part of a member; discard the window */

/* ---- enums -------------------------------------------------------------------- */
#define RR_F32   0            /* fp32 inputs, fp32 arithmetic throughout               */
#define RR_BF16  1            /* bf16 inputs, fp32 accumulation                        */

#define RR_OP_FWD 0           /* workspace query for rr_attn_fwd                      */
#define RR_OP_BWD 1           /* workspace query for rr_attn_bwd                      */
#define RR_OP_PROMPT_GRADS 2  /* workspace query for rr_attn_prompt_grads             */

#define RR_MAX_K     64       /* responses per replay microbatch                      */

/* rr_problem.flags */
#define RR_FLAG_SHARD_NO_RESPONSE 1  /* this call holds one shard of the prompt and another
                                        shard owns the response's own keys: the forward
                                        writes the response part as empty (lse = -inf),
                                        the backward forms dq over this shard's prompt keys
                                        only and no dk_r / dv_r (they may be NULL)        */
#define RR_MAX_ACC    8       /* buffers per accumulation window                      */

/* Problem description shared by rr_attn_fwd / rr_attn_bwd / rr_workspace_bytes. */
typedef struct rr_problem {
  int64_t P;        /* resident prompt positions, >= 0 (0: no resident keys, the rows
                       attend to their own causal keys only; k_p / v_p may be NULL)     */
  int64_t chunk;    /* prompt chunk length: the prompt is split into ceil(P/chunk)
                       contiguous chunks, each with its own softmax statistics; >= 1     */
  int32_t R_max;    /* row stride of the per-response tensors, >= 1                     */
  int32_t K;        /* responses in the replay microbatch, 1..RR_MAX_K                  */
  int32_t Hq;       /* query heads                                                      */
  int32_t Hkv;      /* KV heads (1 for latent pages); Hq % Hkv == 0                     */
  int32_t d_qk;     /* query/key head dim: 64 or 128 dense; 576 latent                  */
  int32_t d_v;      /* value head dim: == d_qk dense; 512 latent                        */
  int32_t block;    /* response block length of the reverse backward walk, >= 1         */
  int32_t topk;     /* 0 = dense over all prompt positions; > 0 = per-query top-k       */
  int32_t idx_dim;  /* index-key width of the top-k selection (topk > 0)                */
  int32_t latent;   /* 0 = GQA K/V pages; 1 = latent rows (K = row, V = first d_v dims) */
  int32_t dtype;    /* RR_F32 or RR_BF16                                                */
  float   tau;      /* softmax scale, finite and > 0                                    */
  int32_t flags;    /* RR_FLAG_* bits; 0 for a whole prompt on one device               */
} rr_problem;

/* Resident prompt state (prompt-group lifetime).  Read-only to the library. */
typedef struct rr_resident {
  const void*  k_p;     /* [P][Hkv][d_qk] dtype, or latent rows [P][d_qk]              */
  const void*  v_p;     /* [P][Hkv][d_v] dtype; NULL for latent pages                   */
  const float* k_idx;   /* [P][idx_dim] fp32 index keys (topk > 0), else NULL           */
  int64_t      P;       /* must equal rr_problem.P                                      */
  uint64_t     version; /* identity of the model snapshot the state was captured with   */
} rr_resident;

/* Bytes of caller-provided workspace an operation needs (0 on invalid problems;
   rr_last_error() then says why). */
size_t rr_workspace_bytes(const rr_problem* p, int op);

/* Number of softmax-statistics partials the forward forms: ceil(P/chunk) prompt chunks
   plus one for the response's own causal keys (dense), or 2 (top-k: selected prompt
   rows, then response rows).  0 on invalid problems. */
int32_t rr_num_parts(const rr_problem* p);

/*
 * rr_attn_fwd - exact attention of the replayed response rows.
 *
 * Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
 * architectures, same transaction": each part of the key set (a prompt chunk, then the
 * response's causal keys) is attended separately, keeping its softmax statistics
 * (running max m and sum l, exported as lse_c = m + ln l together with O_c = O~_c / l),
 * and the parts are composed into the exact global output (see rr_lse_merge).
 *
 *   r_len     host [K] int32, 0 <= r_len[k] <= R_max
 *   q_idx     [K][R][idx_dim] fp32 index queries (topk > 0), else NULL
 *   o, lse    outputs (see layouts); both NULL = partials only (export required)
 *   part_o    NULL, or export buffer [n_parts][K][R][Hq][d_v] fp32 (n_parts =
 *   part_lse  rr_num_parts); with part_lse [n_parts][K][R][Hq] fp32.  Exported
 *             partials make the per-chunk statistics available to an external merge;
 *             entries of padding rows (i >= r_len[k]) are unspecified and may be left
 *             unwritten.
 *   topk_idx  topk > 0: output [K][R][topk] int32, the selected prompt positions of
 *             each row in ascending order (-1 in padding rows); else NULL
 *
 * Latent-page top-k variant (latent = 1).  Source: ai.thesatyajit.com/articles/
 * longstraw-2m-rl, section "Two incompatible architectures, same transaction" (GLM
 * instantiation: MLA latent pages of 512 + 64 dims and resident index keys from which
 * the sparse selection is rebuilt).  Row i of response k scores every prompt position j
 * by sigma = q_idx . k_idx_j (fp32), keeps the topk largest (equal scores: the lower
 * position first), and attends, for each of the 64 heads, over those latent rows plus
 * response rows 0..i (key = the 576-wide row, value = its first 512 dims).  Built for
 * bf16, Hq = 64, Hkv = 1, d_qk = 576, d_v = 512, idx_dim = 128, topk a multiple of 32 in
 * [32, min(P, 4096)], R_max a multiple of 8, flags = 0, o and lse required, no partial export; the
 * workspace holds the fp32 scores, K * R_max * P * 4 bytes.
 *   ws        workspace of rr_workspace_bytes(p, RR_OP_FWD) bytes (may be NULL when 0)
 */
int rr_attn_fwd(const rr_problem* p, const rr_resident* kv,
                const void* q, const void* k_r, const void* v_r, const int32_t* r_len,
                const float* q_idx, float* o, float* lse, float* part_o, float* part_lse,
                int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * rr_lse_merge - exact composition of n softmax-statistics partials.
 *
 * Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
 * architectures, same transaction" (rank-local softmax statistics composed into the
 * exact global attention output).  For every row:
 *   lse = ln sum_c exp(lse_c),   O = sum_c exp(lse_c - lse) * O_c,
 * O summed in part order, the normaliser in a fixed order (deterministic).  Parts with lse_c = -inf carry weight 0; a row whose parts are
 * all -inf gets O = 0, lse = -inf.
 *
 *   part_o [n_parts][rows][d_v] fp32, part_lse [n_parts][rows] fp32 (inputs)
 *   o [rows][d_v] fp32, lse [rows] fp32 (outputs; may not alias the inputs)
 */
int rr_lse_merge(int32_t n_parts, int64_t rows, int32_t d_v, const float* part_o,
                 const float* part_lse, float* o, float* lse, void* stream);

/* Identity of the resident state a backward read, written by rr_attn_bwd and checked by
   rr_grad_accum: a member's gradients may only enter the accumulation window of the model
   version and prompt group they were computed against.  Source: networkfinds.com/long-
   context-rl-is-a-state-lifetime-problem, section "Preserve gradient semantics, not just
   forward outputs" (every resident object has an owning model version; versions never
   mix).  Host memory; the caller passes it on unchanged. */
typedef struct rr_grad_tag {
  uint64_t    version;   /* rr_resident.version of the state the backward read           */
  const void* resident;  /* rr_resident.k_p of that state (its identity)                 */
  int64_t     P;         /* rr_resident.P                                                */
  uint64_t    seal;      /* check value the library computes over the three fields above;
                            a tag that no backward wrote (zero-filled, edited, assembled
                            by hand) fails rr_grad_accum                                  */
} rr_grad_tag;

/*
 * rr_attn_bwd - response-only backward.
 *
 * Source: ai.thesatyajit.com/articles/longstraw-2m-rl, sections "The move: change the
 * graph boundary" (only the direct response gradient; the prompt state is a stop-
 * gradient) and "Two incompatible architectures, same transaction" (response blocks
 * replayed in reverse; K/V gradient storage only where a response backward touches).
 * There is no prompt-gradient argument: the resident K/V receives no gradient and no
 * storage for one is ever formed.
 *
 * With L = sum dO . O, per row i, head h and visible key j:
 *   p = exp(tau q.k_j - lse_i), D_i = dO_i . O_i, ds = p (dO_i . v_j - D_i),
 *   dq_i = tau sum_j ds k_j;  dk_r[j] = tau sum ds q_i;  dv_r[j] = sum p dO_i,
 * the last two over the query heads of KV head j's group and rows i >= j.
 *
 *   o, lse      the forward's fp32 outputs for these rows (global statistics; a caller
 *               holding one shard of the prompt passes the merged ones)
 *   topk_idx    topk > 0: the forward's selection [K][R][topk]; else NULL.  Entries
 *               outside [0, P) are clamped into it (no fault; the gradients are then
 *               those of the clamped selection).
 *   accumulate  0: gradients are written (=) to every row the call touches;
 *               1: they are added (+=)
 *   block_idx   -1: whole response: dq of every row, then dk_r/dv_r of the whole walk
 *               over blocks nb-1 .. 0 (nb = ceil(R_max/block); bf16 problems form the
 *               walk's sum in one launch, fp32 problems launch per block, last first).
 *               b >= 0: only block b's query rows:
 *               their dq, and their contributions to dk_r/dv_r of response keys
 *               [0, (b+1)*block).  A caller driving the walk itself zeroes dk_r/dv_r
 *               once and calls b = nb-1 .. 0 with accumulate = 1; after the call for b
 *               the dk_r/dv_r rows of block b are final.
 *   ws          workspace of rr_workspace_bytes(p, RR_OP_BWD) bytes.  On return its first
 *               K * R_max * Hq floats hold D = dO . O, [K][R_max][Hq] fp32, for the rows
 *               the call covered (0 in padding rows; the entries of other rows are
 *               unspecified).
 *   tag         host, may be NULL: on success, the identity of kv (version, k_p, P),
 *               sealed, for rr_grad_accum.  Untouched on failure.
 */
int rr_attn_bwd(const rr_problem* p, const rr_resident* kv,
                const void* q, const void* k_r, const void* v_r, const int32_t* r_len,
                const int32_t* topk_idx, const float* o, const float* lse, const void* d_o,
                float* dq, float* dk_r, float* dv_r, int32_t accumulate, int32_t block_idx,
                void* ws, size_t ws_bytes, rr_grad_tag* tag, void* stream);

/*
 * rr_attn_prompt_grads - full-sequence differential mode: the prompt-side gradient term
 * that the response-only contract drops, for comparing the two paths.
 *
 * Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "The move: change the
 * graph boundary" (a full-sequence gradient is the direct response term plus a term
 * through the prompt state; the contract keeps the first); networkfinds.com/long-context-
 * rl-is-a-state-lifetime-problem, section "Preserve gradient semantics, not just forward
 * outputs" (validate against a conventional run).  rr_attn_bwd never forms this term;
 * a caller asks for it explicitly, with its own output buffers.
 *
 * For every prompt position j, KV head g, and every row i < r_len[k] of every response
 * k of the call, over the query heads h of g's group (no mask: rows see all of the
 * prompt):
 *   p = exp(tau q_ih.k_jg - lse_ih),  D_ih = dO_ih . O_ih,  ds = p (dO_ih.v_jg - D_ih),
 *   dk_p[j][g] = tau sum ds q_ih,     dv_p[j][g] = sum p dO_ih.
 * bf16 problems round p and ds to bf16 before the two products (fp32 accumulation);
 * fp32 problems compute in fp32 throughout.
 *
 *   q, d_o      [K][R][Hq][d] (problem dtype), the rows of rr_attn_bwd
 *   o, lse      the forward's fp32 outputs (global statistics; a caller holding one shard
 *               of the prompt passes the merged ones and gets its shard's gradients)
 *   key_lo, key_hi  the resident positions [key_lo, key_hi) whose gradients are formed,
 *               0 <= key_lo <= key_hi <= P (the whole prompt: 0, P)
 *   dk_p, dv_p  outputs [key_hi - key_lo][Hkv][d] fp32, device, row j - key_lo for
 *               position j; every row is written (=) or added to (+=, accumulate = 1),
 *               e.g. across the members of a group
 *   ws          workspace of rr_workspace_bytes(p, RR_OP_PROMPT_GRADS) bytes: the rows of
 *               each KV head repacked contiguously, with their lse and D
 * Dense pages only (latent = 0; RR_E_UNSUPPORTED otherwise); d_qk = d_v in {64, 128}.
 */
int rr_attn_prompt_grads(const rr_problem* p, const rr_resident* kv, const void* q,
                         const int32_t* r_len, const float* o, const float* lse, const void* d_o,
                         int64_t key_lo, int64_t key_hi, float* dk_p, float* dv_p,
                         int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * rr_lastkv_blend - LastKV previous-chunk blending, the pre-step of a chunk's attention.
 *
 * Source: zefan-cai.github.io/en/blog/lastkv-rl ("In RL, Does the Trainer Evaluate the
 * Policy That Generated the Rollout?"), section "LastKV: making recurrence boundaries part
 * of the policy": chunk c of layer l attends to the last-layer K/V of completed chunks
 * plus its own per-layer K/V (causal); with previous-chunk blending the chunk c-1 enters
 * as x~ = (1 - alpha_{l,g}) x^l_{c-1} + alpha_{l,g} x^L_{c-1}, one gate per layer and KV
 * head.  A caller lays out the resident history of chunk c as [x^L of chunks < c-1; x~ of
 * chunk c-1] (P = c * C positions), passes the chunk's rows as the response (K/V causal),
 * and runs rr_attn_fwd / rr_attn_bwd; rr_attn_prompt_grads over the key range of x~ gives
 * d x~, which rr_lastkv_blend_bwd takes back to the two K/V sources and the gate.
 *
 *   out[r][g][e] = (1 - alpha[g]) x_layer[r][g][e] + alpha[g] x_last[r][g][e]
 * in fp32, stored in `dtype` (bf16: round to nearest even).  Apply once to K, once to V.
 *   rows                    positions of the chunk, >= 0
 *   Hkv, d                  KV heads, head dim (a multiple of 8)
 *   alpha                   device [Hkv] fp32 gates of this layer
 *   x_layer, x_last, x_out  device [rows][Hkv][d] dtype, 16-byte aligned; x_out may alias
 *                           neither input
 */
int rr_lastkv_blend(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                    const void* x_layer, const void* x_last, void* x_out, void* stream);

/*
 * rr_lastkv_blend_bwd - gradients of rr_lastkv_blend from d_out [rows][Hkv][d] fp32:
 *   d_layer = (1 - alpha) d_out,  d_last = alpha d_out,
 *   d_alpha[g] = sum over rows and dims of (x_last - x_layer) d_out  (fixed-order sum).
 * d_layer, d_last: device [rows][Hkv][d] fp32, either may be NULL (not formed); d_alpha:
 * device [Hkv] fp32.  accumulate 0: written; 1: added.
 */
int rr_lastkv_blend_bwd(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                        const void* x_layer, const void* x_last, const float* d_out, float* d_layer,
                        float* d_last, float* d_alpha, int32_t accumulate, void* stream);

/* Update-boundary accumulator for G serially replayed members.
   Source: networkfinds.com/long-context-rl-is-a-state-lifetime-problem, sections
   "Account for memory by lifetime" (gradients accumulate until one update) and
   "Preserve gradient semantics, not just forward outputs" (a retry must not count
   twice, a dropped member must not go unnoticed, no mixing of versions). */
typedef struct rr_accum {
  int32_t  n_bufs;              /* 1..RR_MAX_ACC                                       */
  float*   buf[RR_MAX_ACC];     /* device fp32 accumulators                            */
  int64_t  n[RR_MAX_ACC];       /* elements of each accumulator                        */
  int32_t  G;                   /* members in the window, >= 1                         */
  uint64_t version;             /* model version the window accumulates against       */
  uint8_t* seen;                /* host [G]; seen[g] = 1 once member g is accumulated  */
  /* Written by the library; the caller zero-initialises them when opening a window.    */
  const void* resident;         /* resident (k_p) of the first accepted member; every
                                   later member must have read the same one           */
  int64_t  resident_P;          /* its P                                               */
  int32_t  poisoned;            /* 1 after a launch failed part-way (RR_E_POISONED)    */
} rr_accum;

/*
 * rr_grad_accum - buf[i][e] += scale * grads[i][e] for e < n_elems[i], i < n_bufs.
 * Positions beyond n_elems[i] are untouched (position-aligned accumulation of members
 * with different lengths).
 *   tag      the rr_grad_tag that rr_attn_bwd wrote for this member's gradients
 *   grads    host array [n_bufs] of device fp32 pointers
 *   n_elems  host array [n_bufs]
 * Rejected without any launch: a poisoned window (RR_E_POISONED); member_g outside
 * [0, G) (RR_E_RANGE); tag NULL (RR_E_NULL); a tag that fails its seal (RR_E_STALE: no
 * backward wrote it); tag->version != acc->version (RR_E_STALE: the gradients were
 * computed against a resident state of another model version); a resident other than
 * the window's first member's (RR_E_STALE: prompt groups mixed); a member already seen
 * (RR_E_DUPLICATE, a retry); n_elems[i] > acc->n[i] (RR_E_SHAPE).  On success sets
 * seen[member_g] (and, for the first member, acc->resident / resident_P).  If a launch
 * fails after buffer 0 was added, the window is marked poisoned and RR_E_POISONED is
 * returned: its accumulators hold part of the member, so no retry can make it whole.
 */
int rr_grad_accum(rr_accum* acc, int32_t member_g, const rr_grad_tag* tag,
                  const float* const* grads, const int64_t* n_elems, float scale,
                  void* stream);

/* RR_OK if every member 0..G-1 has been accumulated, else RR_E_MISSING naming the first
   missing member (a dropped branch), or RR_E_POISONED.  Host only. */
int rr_accum_check_complete(const rr_accum* acc);

/* ---- entry point for callers that cannot allocate --------------------------------- */
/*
 * rr_attn_fwd_static - rr_attn_fwd for callers that cannot allocate device memory or size
 * a workspace at call time: code under HIP graph capture that must not allocate, tight
 * serving loops, harnesses that forbid allocation.
 *
 * Same arguments and results as rr_attn_fwd without ws / ws_bytes: the workspace is a
 * static device array of RR_STATIC_SCRATCH_BYTES bytes that the library holds on each GPU
 * it runs on until the process ends.  Calls no hipMalloc or hipFree.  A problem with
 * rr_workspace_bytes(p, RR_OP_FWD) > RR_STATIC_SCRATCH_BYTES (and no partials export)
 * returns RR_E_WORKSPACE before any launch.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (several streams or host threads) race on
 * it, and the caller must order them.  The array keeps the last call's contents; nothing
 * in it needs to start at zero.
 */
#define RR_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int rr_attn_fwd_static(const rr_problem* p, const rr_resident* kv,
                       const void* q, const void* k_r, const void* v_r, const int32_t* r_len,
                       const float* q_idx, float* o, float* lse, float* part_o, float* part_lse,
                       int32_t* topk_idx, void* stream);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* rr_last_error(void);

/* ---- measurement --------------------------------------------------------------- */
/* While profiling is on, every kernel the library launches is bracketed by two HIP
   events recorded on the launch stream.  rr_profile_end waits for them and returns,
   per kernel name, the number of launches and the summed device time.  Not for use
   under stream capture. */
typedef struct rr_profile_entry {
  char    name[48];
  int64_t launches;
  double  total_ms;
} rr_profile_entry;

int rr_profile_begin(void);
int rr_profile_end(rr_profile_entry* out, int32_t max_entries, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* RR_ATTN_H */
