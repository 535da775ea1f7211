/*
 * moe_vq.h -- C ABI of the MoE-VQ routed-expert step on AMD Instinct MI355X (gfx950).
 *
 * One call sequence computes, for n_tokens activations x [T, H]:
 *   route      l = W_r x; p = softmax(l); S = top-k(l); w = p_S / sum p_S
 *   FC1        g = W_g,e x, u = W_u,e x, h = silu(g) * u      (per selected expert e)
 *   FC2        o = W_d,e h
 *   combine    y[t] = sum_i w[t,i] o[t,i]
 * with every expert matrix stored as 2-bit sign-symmetric vector codes (VQ2) or as
 * MXFP4, decoded on the fly.  Sources: the Tandem-vLLM 0.2.0 announcement ("How it
 * works": routed experts kept as 2-bit vector codes, about 2.1 bits per weight, a
 * GPU cache of the most-used experts, nothing skipped or substituted; "Quality vs
 * the official FP4 checkpoint": the 52 most-routed experts per layer kept in FP4)
 * and the vLLM-Moet README ("2-bit experts on vLLM v0.24.0": the codebook is
 * sign-symmetric; "What we changed against official vLLM", row "MoE at decode":
 * router -> FC1 -> FC2 without padding the experts; "Qwen3.8-Flash-Next-FP8": the
 * routed-expert GEMV with silu*up fused).
 *
 * VQ2 format.  A weight matrix [rows][in] is stored as u8 words [rows][in/4] and
 * fp16 scales [rows][in/128].  Word b encodes four consecutive weights of one row:
 *     W[n, 4j+d] = S[n, (4j+d)/128] * (b & 0x80 ? -1 : +1) * CB[b & 0x7F][d]
 * with CB the per-layer fp16 codebook [128][4] (2 + 16/128 = 2.125 bits/weight).
 * MXFP4 format.  u8 [rows][in/2] holding E2M1 elements (low nibble = even index)
 * and u8 E8M0 exponents [rows][in/32]:  W[n,k] = E2M1(q) * 2^(e-127).
 *
 * Slot pool.  All experts live in one device buffer (the pool).  slots[e] gives
 * expert e's byte offset in the pool and its format.  A slot holds six row-major
 * blocks, each starting on a 256-byte boundary relative to the slot start:
 *     VQ2:   codes_gate [I][H/4] | codes_up [I][H/4] | codes_down [H][I/4] |
 *            scales_gate [I][H/128] | scales_up [I][H/128] | scales_down [H][I/128]
 *     MXFP4: q_gate [I][H/2] | q_up [I][H/2] | q_down [H][I/2] |
 *            e8m0_gate [I][H/32] | e8m0_up [I][H/32] | e8m0_down [H][I/32]
 * moe_vq_expert_bytes() returns the slot size.  byte_offset must be a multiple of 256.
 *
 * Conventions.
 *  - Pointers are device memory unless marked [host].  The caller owns every buffer
 *    (pool, slots, router weights, codebook, x, h, y, workspace); the library
 *    allocates and frees nothing and keeps no mutable global state (apart from the
 *    per-thread measurement hook moe_vq_time_next_kernel and the last HIP error).
 *  - stream is a hipStream_t (NULL = the default stream).  Every compute call only
 *    enqueues work on it and returns; nothing synchronises except moe_vq_check().
 *  - Argument errors are returned synchronously, before any HIP call is made.
 *  - Errors found on the device are recorded in the workspace's status word and
 *    reported by moe_vq_check(): an absent expert or a slot outside the pool
 *    (MOE_VQ_ENOTRESIDENT; that contribution is left out of y), or a compute call
 *    made on a workspace routed for other shapes or other activations
 *    (MOE_VQ_EINVAL; the call computes nothing from the experts, and its outputs
 *    must not be used).  Nothing is ever silently skipped (Tandem-vLLM 0.2.0 announcement,
 *    "How it works": nothing is skipped or substituted).
 *  - Calls on one workspace must be stream-ordered: a workspace holds one step.
 *  - Results are deterministic: repeated calls on the same inputs give the same bits.
 */
#ifndef MOE_VQ_H
#define MOE_VQ_H

#include <stddef.h>
#include <stdint.h>

/* Only the moe_vq_* entry points are exported from the shared library; it is built
 * with hidden visibility for everything else. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum moe_vq_status {
  MOE_VQ_OK = 0,
  MOE_VQ_EINVAL = 1,        /* bad argument (null pointer, bad size, bad enum)            */
  MOE_VQ_EUNSUPPORTED = 2,  /* shape or dtype the library does not implement             */
  MOE_VQ_ENOSPACE = 3,      /* workspace smaller than moe_vq_workspace_bytes()            */
  MOE_VQ_EHIP = 4,          /* a HIP runtime call or kernel launch failed                 */
  MOE_VQ_ENOTRESIDENT = 5   /* (device) a selected expert's slot is absent or out of pool */
};

enum moe_vq_dtype { MOE_VQ_F32 = 0, MOE_VQ_BF16 = 1 };

enum moe_vq_format { MOE_VQ_FMT_ABSENT = 0, MOE_VQ_FMT_VQ2 = 1, MOE_VQ_FMT_MXFP4 = 2 };

enum moe_vq_matrix { MOE_VQ_MAT_GATE = 0, MOE_VQ_MAT_UP = 1, MOE_VQ_MAT_DOWN = 2 };

/* Expert slot table entry, device array [n_experts]. */
typedef struct moe_vq_slot {
  uint64_t byte_offset;  /* offset of the slot in the pool, multiple of 256 */
  uint32_t format;       /* enum moe_vq_format                              */
  uint32_t reserved;     /* must be 0                                       */
} moe_vq_slot;

/* [host] Layer descriptor; its pointers are device buffers. */
typedef struct moe_vq_layer {
  int32_t hidden;              /* H, multiple of 128, 128..16384            */
  int32_t inter;               /* I, multiple of 128, 128..16384            */
  int32_t n_experts;           /* E, 1..1024                                */
  int32_t top_k;               /* k, 1..min(E, 32)                          */
  const void *router_w;        /* bf16 [E][H], row-major                    */
  const void *codebook;        /* fp16 [128][4], one per layer              */
  const uint8_t *pool;         /* slot pool                                 */
  uint64_t pool_bytes;         /* size of the pool in bytes                 */
  const moe_vq_slot *slots;    /* [E] expert id -> slot                     */
  float swiglu_limit;          /* SwiGLU clamp L (0: none), see below       */
  const moe_vq_slot *delta_slots; /* [E] FP4 delta cache, or NULL; see below */
  float gate_tau;              /* confidence gate of the delta cache        */
} moe_vq_layer;
/* swiglu_limit: with L > 0 every expert's FC1 output is h = silu(min(g, L)) * clamp(u,
 * -L, L) instead of silu(g) * u, on every path (decode, prefill, the host miss path).
 * The vLLM-Moet README ("Quality vs native", the audit of the W2 path) says the real
 * checkpoint has a SwiGLU clamp that a port must not omit, but gives neither its form
 * nor its constant; this form (gate capped above, up clamped on both sides) is the one
 * read here.  L must be finite and >= 0 (MOE_VQ_EINVAL otherwise).  Zero-initialising
 * the struct leaves the clamp off.
 *
 * delta_slots, gate_tau: the FP4 delta cache and its confidence gate (vLLM-Moet README,
 * "2-bit experts on vLLM v0.24.0", first bullet: a delta cache and a confidence gate
 * bring FP4 back where it matters; "Benchmark results", row glm-5.2-nvfp4: the gate at
 * tau = 0.60).  The pages do not describe the mechanism; the reading here: delta_slots[e]
 * is the slot (in the same pool) of expert e's copy in FP4 (normally MXFP4; format
 * MOE_VQ_FMT_ABSENT: no copy), and a routed pair whose renormalised weight is >= gate_tau
 * and whose expert has a copy is computed from the copy instead of slots[e], on every
 * path (decode and prefill).  Its weight in the combine is unchanged.  With gate_tau >=
 * 0.5 at most one pair of a token passes (its first).  In the workspace, the step's
 * distinct experts (moe_vq_step_info) then count the copies as experts E + e, each listed
 * right after expert e, and a copy whose slot is bad is reported as expert E + e.  NULL (zero-initialised) leaves the cache
 * off.  With delta_slots set, n_experts must be <= 512 and gate_tau finite and >= 0
 * (MOE_VQ_EINVAL otherwise); the host miss path (moe_vq_cpu_experts) does not take such a
 * layer (MOE_VQ_EUNSUPPORTED), and the tier (moe_vq_tier_resolve) manages slots[] only. */

/* [host] Bytes of one expert slot of the given format, 0 if an argument is invalid. */
size_t moe_vq_expert_bytes(int format, int hidden, int inter);

/* [host] Byte offsets, relative to the slot start, of the six blocks of a slot of the
 * given format: offsets[0..2] = gate, up, down payload (VQ2 words or MXFP4 nibbles),
 * offsets[3..5] = gate, up, down scales (fp16 or E8M0), offsets[6] = slot size.
 * Returns MOE_VQ_EINVAL (offsets untouched) for an invalid format or shape. */
int moe_vq_slot_layout(int format, int hidden, int inter, uint64_t offsets[7]);

/* [host] Workspace bytes needed for n_tokens tokens with this layer, 0 if the layer
 * descriptor's sizes are invalid (pointers are not inspected).  The workspace holds
 * the routing worklist, staged activations, per-pair FC2 outputs and the status word. */
size_t moe_vq_workspace_bytes(const moe_vq_layer *layer, int n_tokens);

/* Route n_tokens tokens: router product (bf16 weights, fp32 accumulation), softmax
 * over all experts, top-k (descending logit, equal logits -> lower expert id),
 * renormalised weights, and the per-expert worklist with slot lookups, all on the
 * device.  Source: Tandem-vLLM 0.2.0 announcement, "How it works" (each token's routed
 * experts are looked up in the GPU's expert cache); vLLM-Moet README, "What we changed
 * against official vLLM", row "MoE at decode" (router -> FC1 -> FC2).  The pages do not
 * print the routing function; it is read as a softmax over all logits, renormalised
 * over the chosen k.
 * x: [n_tokens][H] in x_dtype, 16-byte aligned.  Outputs topk_ids [n_tokens][k]
 * (int32) and topk_w [n_tokens][k] (fp32).  Also stages x for FC1 in the workspace,
 * records which x was routed, and resets the status word.  n_tokens == 0 is a no-op;
 * n_tokens <= 65536.  Errors: MOE_VQ_EINVAL (bad argument), MOE_VQ_ENOSPACE (ws_bytes <
 * moe_vq_workspace_bytes), MOE_VQ_EHIP (launch failed); an absent or out-of-pool slot of
 * a selected expert is MOE_VQ_ENOTRESIDENT in the status word. */
int moe_vq_route_topk(const moe_vq_layer *layer, const void *x, int x_dtype, int n_tokens,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* FC1 of every routed (token, expert) pair with SiLU*up fused: for pair p = t*k + i
 * (expert topk_ids[t][i]), h[p][:] = silu(W_g x_t) * (W_u x_t), fp32 [n_tokens*k][I],
 * with W_g and W_u decoded from the expert's codes on the fly.  Source: Tandem-vLLM
 * 0.2.0 announcement, "How it works" (routed experts as 2-bit vector codes); vLLM-Moet
 * README, "2-bit experts on vLLM v0.24.0" (sign-symmetric codebook) and
 * "Qwen3.8-Flash-Next-FP8 on 4x RTX PRO 6000" (silu*up fused into the expert GEMV).
 * x and x_dtype must be the activations moe_vq_route_topk was called with on ws (the
 * call reads the fp16 copy of x that routing staged, and the worklist); otherwise the
 * call computes nothing and sets MOE_VQ_EINVAL in the status word.  h: 16-byte aligned,
 * owned by the caller.  Errors: as moe_vq_route_topk. */
int moe_vq_fc1_silu(const moe_vq_layer *layer, const void *x, int x_dtype, int n_tokens,
                    void *ws, size_t ws_bytes, float *h, void *stream);

/* FC2 and the weighted combine: y[t][:] = sum_i topk_w[t][i] * (W_d h[t*k+i]),
 * fp32 [n_tokens][H], overwritten, with W_d decoded from the codes on the fly and the
 * routing weights of the worklist in ws.  Source: Tandem-vLLM 0.2.0 announcement, "How it
 * works" (expert outputs added back with the routing weights; nothing skipped or
 * substituted); vLLM-Moet README, "What we changed against official vLLM", row "MoE at
 * decode" (no padding rows written back).  h: [n_tokens*k][I] fp32 (any values: FC1's
 * output normally), 16-byte aligned; y 16-byte aligned.  A workspace routed for other
 * shapes sets MOE_VQ_EINVAL in the status word and y is then not valid.  Errors: as
 * moe_vq_route_topk. */
int moe_vq_fc2_combine(const moe_vq_layer *layer, const float *h, int n_tokens,
                       void *ws, size_t ws_bytes, float *y, void *stream);

/* The whole routed-expert step in one call: moe_vq_route_topk, moe_vq_fc1_silu and
 * moe_vq_fc2_combine on ws, in that order on stream, with the same results bit for bit
 * (Tandem-vLLM 0.2.0 announcement, "How it works"; vLLM-Moet README, "What we changed
 * against official vLLM", rows "MoE at decode" and "launch gaps": router -> FC1 -> FC2 in
 * as few launches as possible).  Outputs topk_ids, topk_w (as route), h [n_tokens*k][I]
 * fp32 (as FC1) and y [n_tokens][H] fp32 (as FC2), all caller-owned; x, h and y 16-byte
 * aligned.  Errors: as moe_vq_route_topk; check the status word with moe_vq_check. */
int moe_vq_forward(const moe_vq_layer *layer, const void *x, int x_dtype, int n_tokens,
                   int32_t *topk_ids, float *topk_w, float *h, float *y,
                   void *ws, size_t ws_bytes, void *stream);

/* moe_vq_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same step and
 * the same kernels, with the workspace in a static device array of the library (16 MiB
 * per GPU, held until the process ends) instead of a caller buffer.  It calls no
 * allocating routine.  status (device int32[2], may be NULL) receives the step's status
 * word and offending expert id (as moe_vq_check reports them) at the end of the step, on
 * stream.  Every call on one GPU shares that GPU's array and each call overwrites it:
 * calls that overlap on one GPU (other streams, other threads) race, so they must be
 * serialised by the caller.  Nothing in the array needs clearing between calls (every
 * word a step reads is written earlier in the same step).  Errors: as moe_vq_forward, and
 * MOE_VQ_ENOSPACE when the step's workspace (moe_vq_workspace_bytes for n_tokens) exceeds
 * 16 MiB: 55 tokens at H = 7168, I = 2048, 256 experts, top-8. */
int moe_vq_forward_static(const moe_vq_layer *layer, const void *x, int x_dtype, int n_tokens,
                          int32_t *topk_ids, float *topk_w, float *h, float *y, int32_t *status,
                          void *stream);

/* The shared expert: y[t][:] += S(x_t) for every token, S a SwiGLU MLP that every token
 * passes through with weight 1 besides its routed experts, so that after the routed step
 * y = sum_i w_i E_i(x) + S(x).  Source: the DeepSeek V4 Flash article's llama.cpp
 * comparison, whose GGUF file name marks a quantised shared expert ("SExpQ8"); the pages
 * say no more, and this plain reading (weight 1, added after the routed combine) is the
 * one taken.  shared: a layer descriptor with n_experts = 1 and top_k = 1 whose expert 0
 * is the shared expert, in either slot format (its own pool, or the routed layer's pool
 * and codebook), with its own swiglu_limit; its router_w must point at one bf16 row of H
 * values, whose values do not matter (a single expert always has weight 1).  x, x_dtype,
 * n_tokens: as moe_vq_route_topk.  ws: a workspace of moe_vq_workspace_bytes(shared,
 * n_tokens) bytes (it may be the routed step's workspace once that step is done, if it
 * is large enough).  h: [n_tokens][I] fp32, caller-owned scratch (receives S's FC1
 * output).  y: [n_tokens][H] fp32, read and written (the shared output is added).  Runs
 * route, FC1 and FC2 of the one-expert layer on stream; the same kernels as the routed
 * step.  Errors: MOE_VQ_EINVAL (bad argument, or n_experts != 1 or top_k != 1), as
 * moe_vq_route_topk otherwise; an absent slot is MOE_VQ_ENOTRESIDENT in the status word,
 * and y is then unchanged. */
int moe_vq_shared_expert(const moe_vq_layer *shared, const void *x, int x_dtype, int n_tokens,
                         void *ws, size_t ws_bytes, float *h, float *y, void *stream);

/* Prefill form of FC1 + FC2 + combine for large n_tokens (vLLM-Moet README, "What we
 * changed against official vLLM", rows "MoE at decode" and "prefill": tokens grouped per
 * expert, no padding to a fixed row count).  The routed pairs of each expert are cut into
 * tiles of 64 tokens; FC1 (gate/up, SiLU*up fused) and FC2 (down, routing weight fused)
 * run as fp16 matrix-core (MFMA) products with fp32 accumulation over weights decoded in
 * registers (VQ2: codebook vector times group scale, rounded once to fp16; MXFP4: E2M1
 * values times 2^(e - e_row), e_row the largest exponent of the weight row, with
 * 2^(e_row - 127) applied to the row's fp32 outputs -- exact while e >= e_row - 23).  x is
 * staged as fp16 with one power-of-two factor per token, h with one per routed pair.
 * Requires moe_vq_route_topk on the same x, x_dtype and n_tokens first (it builds the
 * worklist this call reads); other activations set MOE_VQ_EINVAL in the status word and
 * y is then not valid.  x: [n_tokens][H] in x_dtype, 16-byte aligned; y: [n_tokens][H]
 * fp32, 16-byte aligned, overwritten.  Errors: as moe_vq_fc2_combine; an absent expert
 * contributes 0 and is reported by moe_vq_check. */
int moe_vq_prefill_gemm(const moe_vq_layer *layer, const void *x, int x_dtype, int n_tokens,
                        void *ws, size_t ws_bytes, float *y, void *stream);

/* Test hook: decode one matrix (enum moe_vq_matrix) of one expert into out, [rows][in]
 * row-major (the VQ2 and MXFP4 formats above; Tandem-vLLM 0.2.0 announcement, "How it
 * works" and "Quality vs the official FP4 checkpoint").  out_dtype MOE_VQ_F32 gives the exact decoded values, MOE_VQ_BF16 their
 * round-to-nearest-even.  It uses the same LDS decode tables as the FC kernels.  The
 * slot is read on the device: if it is absent or lies outside the pool, out is left
 * untouched and *status_dev (a device int32, may be NULL) is set to
 * MOE_VQ_ENOTRESIDENT, otherwise to MOE_VQ_OK. */
int moe_vq_decode_expert(const moe_vq_layer *layer, int expert, int matrix, int out_dtype,
                         void *out, int32_t *status_dev, void *stream);

/* Synchronise stream, then return the device-side status of the last step run on ws
 * (MOE_VQ_OK, MOE_VQ_ENOTRESIDENT, or MOE_VQ_EINVAL for a refused compute call).  If
 * info is not NULL, *info receives the first offending expert id (or -1). */
int moe_vq_check(const void *ws, void *stream, int32_t *info);

/* Synchronise stream and copy the routing summary of the last step on ws to the host:
 * summary[0] = device status, summary[1] = offending expert or -1, summary[2] = number
 * of distinct selected experts (n_active), summary[3] = routed pairs placed.  If
 * experts is not NULL it receives the n_active distinct expert ids in ascending order of
 * expert (room for n_experts entries; 2 n_experts with an FP4 delta cache, whose copies
 * are listed as E + e, each right after expert e).  layer and n_tokens must match the route call. */
int moe_vq_step_info(const moe_vq_layer *layer, int n_tokens, const void *ws, int32_t summary[4],
                     int32_t *experts, void *stream);

/* Measurement hook for benchmarks (timing the kernels against the pages' throughput
 * figures; Tandem-vLLM 0.2.0 announcement, "Speed").  The next decode FC kernel that a
 * call made on this thread launches -- FC1's in moe_vq_fc1_silu, moe_vq_forward and
 * moe_vq_forward_static, FC2's in moe_vq_fc2_combine, the read of moe_vq_read_probe; not
 * the combine kernel and not prefill -- is launched with hipExtLaunchKernel so that start_event records the
 * kernel's start and stop_event its end (hipEvent_t, created with timing; either may be
 * NULL).  hipEventElapsedTime of the two is then the kernel's own run time, without the
 * dispatch that an event recorded on the stream before the launch also counts.  The
 * hook is per thread, used by one launch, and stays set until a launch uses it; NULL,
 * NULL clears it.  Returns MOE_VQ_OK. */
int moe_vq_time_next_kernel(void *start_event, void *stop_event);

/* Measurement hook: a plain streaming read of bytes (a multiple of 16, >= 16) at buf
 * (16-byte aligned) with 16-byte loads over every compute unit, enqueued on stream, so
 * that the rate the decode kernels reach can be set against what a read alone reaches on
 * the same device (the pages measure their kernels against the hardware's limits; vLLM-Moet
 * README, "What we changed against official vLLM").  sink (device, 4-byte aligned) is
 * written only in a case that does not occur in practice.  Errors: MOE_VQ_EINVAL for bad
 * arguments (before any HIP call), MOE_VQ_EHIP if the launch fails. */
int moe_vq_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* ---- Host-RAM expert tier.  Experts can live in a pinned host pool, with the device
 * pool holding only some of them: a GPU cache of the experts in use in front of the rest
 * (Tandem-vLLM 0.2.0 announcement, "How it works").  When a step selects an expert that
 * is not resident, its slot is copied into a device slot (evicting the least recently
 * used expert that the step does not select) and the step is run again; the result is
 * bit-identical to a run with every expert resident, since the kernels read the same
 * bytes.  All tier state is caller-owned host memory; the library allocates nothing. */
typedef struct moe_vq_tier {
  const uint8_t *host_pool;          /* [host] every expert's slot, pinned (hipHostMalloc) for
                                        asynchronous copies; the slot layout of the device pool */
  const moe_vq_slot *host_slots;     /* [host] [E] expert -> offset in host_pool and format
                                        (MOE_VQ_FMT_ABSENT: not available, never installed)     */
  int32_t n_dev_slots;               /* device slots the tier manages, 1..4096                  */
  const uint64_t *dev_slot_offsets;  /* [host] [n_dev_slots] offsets in the device pool,
                                        multiples of 256, each with room for the largest expert */
  int32_t *dev_slot_expert;          /* [host] [n_dev_slots] state: expert held, -1 = free      */
  uint64_t *dev_slot_stamp;          /* [host] [n_dev_slots] state: last step that used it       */
  moe_vq_slot *slot_mirror;          /* [host] [E] state: the device slot table's contents      */
  uint64_t step;                     /* state: steps resolved so far                            */
  uint32_t *readback;                /* [host] [64 + E] words, pinned (hipHostMalloc), or NULL:
                                        where moe_vq_tier_resolve reads the step's selection;
                                        pinned, that read is one asynchronous copy and one
                                        synchronisation; NULL, a synchronous copy (slower)  */
} moe_vq_tier;

/* [host] Start a tier: every device slot free, every expert absent.  Writes the device
 * slot table slots[E] (the array layer->slots points to) to all-absent and synchronises
 * stream.  Errors: MOE_VQ_EINVAL for a null pointer, a bad size or a device slot offset
 * that is not a multiple of 256 or leaves no room for the largest expert in the pool. */
int moe_vq_tier_init(const moe_vq_layer *layer, moe_vq_tier *tier, moe_vq_slot *slots, void *stream);

/* [host] The tier's decision for one step, without side effects.  active[0..n_active) are
 * the step's distinct experts.  Each active expert that is not resident and is available
 * in the host pool gets a device slot: a free slot first (lowest index), else the slot
 * of the least recently used expert that is not active (oldest stamp, then lowest
 * index).  On return install_expert[i], install_slot[i] and evict_expert[i] (-1 if the
 * slot was free), i < *n_install, list the copies in that order.  Arrays have room for
 * n_active entries.  Returns MOE_VQ_ENOSPACE (nothing listed) if the step selects more
 * experts than the tier has device slots for, MOE_VQ_EINVAL for bad arguments. */
int moe_vq_tier_plan(const moe_vq_tier *tier, int n_experts, const int32_t *active, int n_active,
                     int32_t *install_expert, int32_t *install_slot, int32_t *evict_expert,
                     int *n_install);

/* [host] Resolve the misses of the step last routed on ws: read the step's distinct
 * experts from ws (through tier->readback; this synchronises stream), mark the resident
 * ones as used, then copy every planned expert slot from tier->host_pool into the device
 * pool (asynchronous on stream) and update slots[E] and the tier state.  Synchronises
 * stream again before it returns when it copied anything.  *n_installed (may be NULL) receives the number of experts copied; if it is
 * not 0 the step must be routed again (moe_vq_route_topk) before FC1.  pool and slots
 * are the writable device buffers behind layer->pool and layer->slots.  Errors: as
 * moe_vq_tier_plan, and MOE_VQ_EHIP if a copy fails (the tier state is then updated
 * only for the copies issued before it). */
int moe_vq_tier_resolve(const moe_vq_layer *layer, moe_vq_tier *tier, uint8_t *pool, moe_vq_slot *slots,
                        int n_tokens, const void *ws, void *stream, int32_t *n_installed);

/* [host] The CPU miss path: routed experts computed on the host cores, for the experts
 * of a step that are not resident in the device pool, while the GPU computes the resident
 * ones (Tandem-vLLM 0.2.0 announcement, "How it works": experts that miss the GPU's cache
 * are computed by the CPU in parallel with the GPU; "What you need": an AVX2 or AVX-512
 * CPU).  For every pair p = t*k + i with compute[topk_ids[p]] != 0 it adds
 * topk_w[p] * W_d (silu(W_g x_t) * (W_u x_t)) to y[t], the expert's matrices read from its
 * slot in host_pool (host_slots[e], the device pool's slot layout) and decoded exactly;
 * fp32 products and sums; experts in ascending id, pairs in order.  Only layer's four
 * sizes are read (its pointers are device memory and are not used).  All pointers are
 * host memory: host_pool [host_pool_bytes], host_slots [E], codebook fp16 [128][4], x
 * [n_tokens][H] in x_dtype, topk_ids and topk_w [n_tokens][k], compute u8 [E], y fp32
 * [n_tokens][H] (accumulated, not overwritten).  n_threads host threads (1..256) run
 * the call and are joined before it returns.  Errors: MOE_VQ_EINVAL for a bad argument
 * or an expert id out of range; MOE_VQ_ENOTRESIDENT when an expert to compute has no
 * slot in the host pool (nothing is added then). */
int moe_vq_cpu_experts(const moe_vq_layer *layer, const uint8_t *host_pool, uint64_t host_pool_bytes,
                       const moe_vq_slot *host_slots, const void *codebook, const void *x, int x_dtype,
                       int n_tokens, const int32_t *topk_ids, const float *topk_w, const uint8_t *compute,
                       float *y, int n_threads);

/* [host] Text of the last HIP runtime error seen by a call of this library on the
 * calling thread (the reason behind MOE_VQ_EHIP), or "" if none. */
const char *moe_vq_last_hip_error(void);

/* [host] Static description of a status code. */
const char *moe_vq_strerror(int status);

#ifdef __cplusplus
}
#endif

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif
#endif /* MOE_VQ_H */
