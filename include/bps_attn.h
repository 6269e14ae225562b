/*
 * bps_attn.h - C ABI of the MI355X (gfx950) fused attention library,
 * forward and backward, over packed variable-length (THD) sequences.
 *
 * What it computes (the operation named by "[JAX] Align fused attn backward
 * output gradient sharding and other test strengthening", TransformerEngine
 * PR 3516, Diagram: the fused-attention forward saves its output, the
 * backward turns it and the output gradient into Q/K/V gradients):
 *
 *   S_ij = scale * <q_i, k_j>,  allowed(i, j) decided by the mask below,
 *   P_ij = softmax_j over allowed j,   O_i = sum_j P_ij v_j,
 *   LSE_i = log sum_{allowed j} exp(S_ij)           (natural log),
 *   dV_j = sum_i P_ij dO_i,   dP_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>,
 *   dS_ij = P_ij (dP_ij - Delta_i),
 *   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
 *
 * With grouped-query attention (Hq = g * Hkv) query head h reads key/value
 * head h / g, and dK, dV of a key/value head sum over the g query heads of
 * its group (maxdiffusion PR 485, Code Review and Key Features of the fused
 * backward: q_heads_per_kv_head, dK/dV accumulated across GQA heads).  Query
 * and value head dims may differ (TransformerEngine PR 2358, review of the
 * KV-packed stride: qk_head_dim vs v_head_dim).
 *
 * Mask.  Without segment metadata every pair is allowed, or j <= i when
 * causal (then Sq must equal Skv).  With metadata, each token carries a
 * segment id and a position inside its segment, separately for Q and KV
 * ("[JAX] Fix batcher in FusedAttn primitive for when seg ids bdims != seg
 * pos bdims", TransformerEngine PR 2692, Description); query i may attend
 * key j when ids_q[i] == ids_kv[j] != 0 and, when causal,
 * pos_kv[j] <= pos_q[i].  Id 0 is padding.  A query that attends nothing
 * gets O = 0, LSE = -inf and dQ = 0; a key that nobody attends gets
 * dK = dV = 0 (every output element is written, so callers need no memset;
 * cf. the gradient zeroing for ragged layouts in TransformerEngine PR 2358,
 * Greptile Overview).
 *
 * Routes.  When Q and KV metadata match, each nonzero id is one contiguous
 * run (runs of nonzero ids have increasing ids) and pos is the offset inside
 * the run, the kernels decide the mask from run boundaries alone (the fast
 * route); otherwise they compare ids and positions (the general route).
 * PR 3516 (Changes 3 and 4, Diagram) routes matching metadata to the fast
 * path and differing metadata (cross-attention, rotated ring steps) to the
 * general one.  The check runs on the device per batch row, and both routes
 * give bitwise identical results.
 *
 * Layout.  Token-major BSHD: element (b, s, h, d) of a tensor lives at
 * base + b*stride.batch + s*stride.token + h*stride.head + d (strides in
 * elements, the head-dim axis contiguous).  dQ, dK, dV use the strides of
 * Q, K, V; dO uses the strides of O (the output gradient must share the
 * saved output's layout, the one-GPU form of the sharding alignment in
 * PR 3516, Changes 1).  Packed buffers pass as strided views: Q, K, V of a
 * [B, S, 3, H, D] buffer, or K, V of [B, S, 2, Hkv, D], with the token
 * stride spanning the whole packed row (TransformerEngine PR 2358, review of
 * the KV-packed stride).  Strides the library writes through (O, and for
 * the backward Q, K, V, which dQ, dK, dV share) must not overlap, i.e. no
 * two elements at one address: otherwise ATTN_E_UNSUPPORTED.  The token
 * strides of K and V may not exceed 2^24 elements (the kernels address key
 * tile rows with 32-bit offsets): otherwise ATTN_E_UNSUPPORTED.  LSE is
 * [B, Hq, Sq] fp32, contiguous.  Segment metadata are int32 [B, S],
 * contiguous.
 *
 * Memory and streams.  Every pointer argument except route_out is device
 * memory owned by the caller; the library allocates nothing and keeps no
 * state besides a thread-local error string.  All work is enqueued on the
 * given HIP stream (a hipStream_t passed as void*, NULL = default stream)
 * and nothing synchronises.  The workspace must hold at least the size the
 * matching *_workspace_size query returns for the same descriptor; its
 * contents need no initialisation and are dead after the stream reaches the
 * end of the call.  Calls that share a workspace must be ordered.
 *
 * Errors.  Arguments are validated on the host before any HIP call; on a
 * failure nothing is launched and the status says why (attn_last_error()
 * returns the text).  A failed launch returns ATTN_E_DEVICE.  No C++
 * exception crosses this interface.
 */
#ifndef BPS_ATTN_H
#define BPS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,      /* inconsistent or missing arguments           */
  ATTN_E_UNSUPPORTED = 2,  /* valid request outside what is built         */
  ATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than required  */
  ATTN_E_DEVICE = 4        /* a HIP call or kernel launch failed          */
} attn_status;

typedef enum {
  ATTN_BF16 = 0,           /* bf16 tensors, fp32 accumulation             */
  ATTN_FP32 = 1            /* fp32 tensors, fp32 accumulation             */
} attn_dtype;

/* attn_desc.flags */
enum {
  ATTN_FORCE_GENERAL = 1u << 0,     /* never take the fast route (tests, ring steps) */
  ATTN_REVERSE_SCHEDULE = 1u << 1,  /* visit workgroup tiles in reverse order (tests:
                                       results must not depend on schedule) */
  ATTN_FUSED_BWD = 1u << 2,         /* backward: single-pass form (see below) */
  ATTN_LOG_ROUTE = 1u << 3          /* debug: report fast-route downgrades on stderr
                                       (synchronises; see below) */
};

/* ATTN_LOG_ROUTE: the TransformerEngine page on fused attention sharding
 * (PR 3516, review) asks for a warning when the fast path is not taken.
 * With this flag, a call that prepares segment metadata (attn_fwd and its
 * variants, and the backward's prepare phase) waits for its stream, reads
 * the route every batch row took and writes one line to stderr per row the
 * device moved from the requested fast route to the general route.  It
 * synchronises the stream, so it is for debugging; attn_route_rows gives
 * the same information without a synchronisation. */

/* ATTN_FUSED_BWD: the single-pass backward of the maxdiffusion page on custom
 * splash and ring attention (Key Features: one kernel over key blocks, query
 * blocks inside, computes dQ, dK and dV, and dQ is reduced across key
 * blocks).  The dK/dV kernel, which already forms dS for every allowed
 * (query, key) tile, also multiplies it by K and writes one fp32 dQ partial
 * per (batch row, query head, key tile of 128, query block of 32) into the
 * workspace; the DQ phase then adds each block's partials over key tiles in
 * ascending order and scales them.  So S and dP are formed once instead of
 * twice (five products instead of seven), and, as that page's code review
 * demands of any dQ reduction, no result depends on the order workgroups
 * run in: outputs are bitwise reproducible and dK, dV are bitwise those of
 * the two-kernel backward.  dQ equals the two-kernel dQ up to fp32
 * summation order (a sum of per-tile partials instead of one running sum).
 * Costs: workspace of B * Hq * ceil(Skv / 128) * 64 ceil(Sq / 64) * Dqk * 4
 * bytes more (17.2 GB at B = 1, Hq = 64, S = 8192, Dqk = 128), written and
 * read once per call.  Built for bf16 with Dqk, Dv <= 128 and no bias or soft
 * cap (ATTN_E_UNSUPPORTED otherwise); the ring emulation does not take it.
 * attn_fwd ignores the flag. */

/* Routes.  route_out (host) receives the route the host requested for the
 * call; attn_route_rows (below) gives the route each batch row took on the
 * device, which may fall back from fast to general. */
enum {
  ATTN_ROUTE_DENSE = 0,    /* no metadata: plain or causal mask           */
  ATTN_ROUTE_FAST = 1,     /* fast route requested; a batch row whose
                              metadata fail the device check falls back to
                              the general route                           */
  ATTN_ROUTE_GENERAL = 2
};

typedef struct {
  int64_t batch, token, head;       /* element strides; head dim contiguous */
} attn_strides;

typedef struct {
  int32_t B, Sq, Skv;               /* batch rows, query / key tokens per row */
  int32_t Hq, Hkv;                  /* query heads, key/value heads (Hq % Hkv == 0) */
  int32_t Dqk, Dv;                  /* head dims: bf16 {64,128,192} x {64,128};
                                       fp32 {64,128} x {64,128} */
  int32_t dtype;                    /* attn_dtype */
  int32_t causal;                   /* 0 or 1 */
  float scale;                      /* softmax scale; 0 selects 1/sqrt(Dqk) */
  uint32_t flags;                   /* ATTN_FORCE_GENERAL | ATTN_REVERSE_SCHEDULE |
                                       ATTN_FUSED_BWD | ATTN_LOG_ROUTE */
  attn_strides q, k, v, o;          /* layouts of Q, K, V, O (and dQ, dK, dV, dO) */
} attn_desc;

typedef struct {
  const int32_t* ids_q;    /* [B, Sq] device; required when the struct is given  */
  const int32_t* pos_q;    /* [B, Sq] device; NULL: offset inside the run of ids  */
  const int32_t* ids_kv;   /* [B, Skv] device; NULL: self-attention, KV metadata
                              are Q's (needs Sq == Skv and pos_kv NULL)          */
  const int32_t* pos_kv;   /* [B, Skv] device; NULL: derived from ids_kv          */
} attn_segments;

/* Workspace bytes needed by attn_fwd / attn_bwd for this descriptor and
 * metadata (seg may be NULL).  Returns 0 for an invalid descriptor (the
 * matching call then reports why).  As in the TransformerEngine page that
 * moves every layout onto the non-packed attention calls (PR 2358, Greptile
 * Overview: one workspace-size computation for all layouts), the size
 * depends only on the shapes, dtype, flags and which metadata are given,
 * never on the layout strides, and the caller allocates it. */
size_t attn_fwd_workspace_size(const attn_desc* desc, const attn_segments* seg);
size_t attn_bwd_workspace_size(const attn_desc* desc, const attn_segments* seg);

/* Forward: O [B,Sq,Hq,Dv] (dtype of the inputs) and LSE [B,Hq,Sq] fp32.
 * seg NULL means plain BSHD.  route_out (host, nullable) receives the route. */
attn_status attn_fwd(const attn_desc* desc, const attn_segments* seg,
                     const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     void* workspace, size_t workspace_bytes,
                     void* stream, int32_t* route_out);

/* Backward: from Q, K, V, the saved O and LSE of attn_fwd, and dO, writes
 * dQ, dK, dV (dtype of the inputs).  dK and dV are complete sums over each
 * GQA group; every element is written exactly once by one workgroup, in a
 * fixed order, so results are bitwise reproducible. */
attn_status attn_bwd(const attn_desc* desc, const attn_segments* seg,
                     const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     void* stream, int32_t* route_out);

/* attn_bwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same backward
 * with no workspace argument.  Its scratch (segment metadata, Delta, LSE in
 * base 2) lives in a file-scope device array of 32 MiB that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  It runs on
 * the current device, which must be the one the stream and tensors belong
 * to.  Limits: the workspace attn_bwd would need without split dK/dV walks
 * must fit in 32 MiB (B * Hq * Sq up to about 4 million rows), otherwise
 * ATTN_E_WORKSPACE; ATTN_FUSED_BWD is ATTN_E_UNSUPPORTED.  Small grids that
 * attn_bwd splits into partial walks run unsplit here, so results equal
 * attn_bwd's bitwise when attn_bwd does not split (at least 512 key tiles of
 * 128) and within rounding otherwise.  Every call on one GPU uses that GPU's
 * one array and nothing in it needs to start at zero (each call writes what
 * it reads); calls that overlap on one GPU, on different streams or
 * threads, race on it and must be ordered by the caller.  Tensors, strides,
 * ownership, streams and errors otherwise as attn_bwd. */
attn_status attn_bwd_noalloc(const attn_desc* desc, const attn_segments* seg,
                             const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv,
                             void* stream, int32_t* route_out);

/* Backward in phases, for callers that time or overlap them.  phases is a
 * nonzero OR of the bits below; ATTN_BWD_ALL is attn_bwd.  PREPARE (segment
 * metadata scan, Delta = rowsum(dO * O), LSE in base 2) fills the workspace
 * that DKDV and DQ then read, so it must complete first on the stream (or be
 * ordered before them with events) and the workspace must not change in
 * between; DKDV and DQ are independent of each other and may run on two
 * streams at once, except under ATTN_FUSED_BWD, where DQ sums the partials
 * DKDV writes and must be ordered after it.  Arguments a phase does not use may be NULL (PREPARE uses
 * o, lse, dout; DKDV uses q, k, v, dout, dk, dv; DQ uses q, k, v, dout, dq).
 * Same descriptor, metadata and workspace size rules as attn_bwd. */
enum {
  ATTN_BWD_PREPARE = 1,
  ATTN_BWD_DKDV = 2,
  ATTN_BWD_DQ = 4,
  ATTN_BWD_ALL = 7
};
attn_status attn_bwd_phase(int32_t phases, const attn_desc* desc, const attn_segments* seg,
                           const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes,
                           void* stream, int32_t* route_out);

/* Test helper: writes the mask the kernels apply, mask_out[b][i][j] = 1 when
 * query i may attend key j (uint8 [B,Sq,Skv], device), and, when route_rows
 * is not NULL, the route each batch row takes (int32 [B], device: 0 dense,
 * 1 fast, 2 general).  Uses the same device mask code and the same
 * metadata preparation as attn_fwd; needs attn_fwd_workspace_size bytes. */
attn_status attn_debug_mask(const attn_desc* desc, const attn_segments* seg,
                            uint8_t* mask_out, int32_t* route_rows,
                            void* workspace, size_t workspace_bytes, void* stream);

/* The route each batch row took in the last attn_fwd, attn_bwd(_phase),
 * attn_*_ex or attn_debug_mask call that used this workspace with the same
 * descriptor and metadata: route_rows[b] (int32 [B], device) = 0 dense,
 * 1 fast, 2 general.  The host requests the fast route when Q and KV
 * metadata are shared or, for equal lengths, may match; the metadata kernel
 * then checks each row (matching metadata, contiguous increasing runs,
 * positions equal to run offsets) and runs the general route where the check
 * fails.  This call reports that outcome without a synchronisation: it
 * enqueues one small kernel on `stream` that copies the per-row routes out
 * of the workspace, so it must be ordered after the call it reports on and
 * before the workspace is reused.  The TransformerEngine page on fused
 * attention sharding (PR 3516, review) asks that a caller can tell when the
 * fast path is not taken; this is that report.  Without metadata every row
 * is 0 and the workspace is not read (it may be NULL).  Needs at least
 * attn_fwd_workspace_size bytes of workspace when seg is given. */
attn_status attn_route_rows(const attn_desc* desc, const attn_segments* seg,
                            const void* workspace, size_t workspace_bytes,
                            int32_t* route_rows, void* stream);

/* One-GPU emulation of ring (context-parallel) attention, the long-sequence
 * scheme of the maxdiffusion ring-attention backward page (Summary and Key
 * Features: K, V, dK and dV rotate between devices while each device keeps
 * its queries and accumulates dQ).  Q is cut into cp shards of Sq / cp
 * tokens and KV into cp shards of Skv / cp tokens (both must divide).  At
 * ring step t the emulated device r holds Q shard r and KV shard
 * (r - t) mod cp and runs the fused attention on that pair; steps t > 0 are
 * forced onto the general metadata route, as the TransformerEngine page on
 * fused attention sharding does for rotated ring steps (Changes 3).
 *
 * Segment metadata are those of the whole sequence, as for attn_fwd:
 * positions (given or derived from the ids on the whole row) stay global,
 * so a segment cut by a shard boundary keeps its mask.  Without metadata
 * every token gets id 1 and its index as position, which reproduces the
 * plain or index-causal mask.
 *
 * attn_ring_fwd: per step an output and LSE for the step's keys, merged
 * into O and LSE by log-sum-exp in fp32 (a row no step attends: O = 0,
 * LSE = -inf).  attn_ring_bwd: per step the gradients against the merged O
 * and LSE, which are exact partial sums; dQ of a Q shard and dK, dV of a KV
 * shard are the sums of their step partials, taken in step order in fp32,
 * so the result is deterministic.  Both equal attn_fwd / attn_bwd on the
 * whole sequence up to rounding (each partial is rounded to the tensor
 * dtype once).  Tensors, strides, ownership and errors as for attn_fwd and
 * attn_bwd; cp < 1 or a shard size that does not divide is ATTN_E_INVALID.
 * The workspace holds the shard-major metadata, the step partials (cp
 * copies of O, or of dQ, dK and dV, each as large as the tensor's extent)
 * and one step's attention workspace; its contents are dead after the call. */
size_t attn_ring_fwd_workspace_size(const attn_desc* desc, const attn_segments* seg, int32_t cp);
size_t attn_ring_bwd_workspace_size(const attn_desc* desc, const attn_segments* seg, int32_t cp);
attn_status attn_ring_fwd(const attn_desc* desc, const attn_segments* seg, int32_t cp,
                          const void* q, const void* k, const void* v,
                          void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);
attn_status attn_ring_bwd(const attn_desc* desc, const attn_segments* seg, int32_t cp,
                          const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout,
                          void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Attention variants.  The TransformerEngine page on fused attention
 * backward sharding ("[JAX] Align fused attn backward output gradient
 * sharding and other test strengthening") runs backward cases with a
 * maximum-logit output and a score modification (Changes 5) and returns
 * optional bias gradients next to the Q/K/V gradients (Diagram); the page
 * "[JAX] Make all jax attention calls use non-packed common calls" links a
 * change adding sink attention.  The pages do not define them; the readings
 * taken here are:
 *
 *   x_ij = scale * <q_i, k_j> + bias[b', h, i, j]      (b' = b, or 0 when
 *                                                       one slab is shared)
 *   S_ij = softcap * tanh(x_ij / softcap) if softcap > 0, else x_ij
 *   LSE_i = log(exp(sink[h]) + sum_{allowed j} exp(S_ij))   (no sink term
 *           without sink logits),   P_ij = exp(S_ij - LSE_i)
 *   max_logit[h] = max of S_ij over batch rows and allowed pairs (-inf if
 *                  there is none; the sink is not a pair)
 *   dS_ij = P_ij (dP_ij - Delta_i),  dx_ij = dS_ij * (1 - (S_ij/softcap)^2)
 *           under soft-capping (dS_ij otherwise),
 *   dQ_i = scale sum_j dx_ij k_j,  dK_j = scale sum_i dx_ij q_i,
 *   dbias[b', h, i, j] = sum of dx_ij over the batch rows b that read slab b'
 *                        (0 at pairs the mask removes),
 *   dsink[h] = - sum_{b, i} exp(sink[h] - LSE_{b,h,i}) Delta_{b,h,i}.
 *
 * A query that attends no key has O = 0 and LSE = sink[h] (-inf without a
 * sink).  Every field may be left zero / NULL; with nothing requested the
 * calls are exactly attn_fwd / attn_bwd_phase.  bias (and dbias) are
 * [bias_batch, Hq, Sq, Skv] contiguous, element type of q, 16-byte aligned,
 * entries finite or -inf; sink, max_logit and dsink are [Hq] fp32.  All
 * pointers are device memory owned by the caller.  dbias is written by the
 * PREPARE (zero fill) and DKDV phases, dsink by PREPARE, max_logit by the
 * forward; when bias_batch == 1 < B the per-row dx are summed in fp32 in
 * batch-row order in the workspace, so dbias is bitwise reproducible too.
 * Errors: bias_batch other than 1 or B, dbias without bias, dsink without
 * sink, a negative or non-finite softcap are ATTN_E_INVALID; a misaligned
 * bias / dbias is ATTN_E_UNSUPPORTED. */
typedef struct {
  const void* bias;        /* additive logit bias, or NULL                    */
  int32_t bias_batch;      /* 1 (one slab for every batch row) or B           */
  float softcap;           /* > 0: soft-capping of the logits; 0: none        */
  const float* sink;       /* [Hq] sink logits (natural log), or NULL         */
  float* max_logit;        /* forward output [Hq], or NULL                    */
  void* dbias;             /* backward output, bias's shape and type, or NULL */
  float* dsink;            /* backward output [Hq], or NULL                   */
} attn_variant;

/* Workspace bytes of the variant calls (at least the plain calls' sizes;
 * var may be NULL).  0 for an invalid descriptor or variant. */
size_t attn_fwd_ex_workspace_size(const attn_desc* desc, const attn_segments* seg, const attn_variant* var);
size_t attn_bwd_ex_workspace_size(const attn_desc* desc, const attn_segments* seg, const attn_variant* var);

/* attn_fwd, attn_bwd and attn_bwd_phase with the variants of var applied;
 * same tensors, layouts, ownership, streams and errors. */
attn_status attn_fwd_ex(const attn_desc* desc, const attn_segments* seg, const attn_variant* var,
                        const void* q, const void* k, const void* v,
                        void* o, float* lse,
                        void* workspace, size_t workspace_bytes,
                        void* stream, int32_t* route_out);
attn_status attn_bwd_ex(const attn_desc* desc, const attn_segments* seg, const attn_variant* var,
                        const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        void* stream, int32_t* route_out);
attn_status attn_bwd_ex_phase(int32_t phases, const attn_desc* desc, const attn_segments* seg,
                              const attn_variant* var,
                              const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout,
                              void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes,
                              void* stream, int32_t* route_out);

/* Text of the last non-OK status returned on this thread ("" if none).  The
 * JAX batcher page (PR 2692, Description) shows the failure this replaces: a
 * segment-id / segment-position shape mismatch surfacing as an assertion
 * deep inside the primitive.  Here every argument is checked on the host
 * before any launch, and the message names the argument and the rule it
 * broke. */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BPS_ATTN_H */
