/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet chunked-prefill forward.
 *
 * Operation (FlashQLA talk transcript, "Qwen系列模型线性注意力高性能优化实践",
 * tokendh.com: linear-attention, GDN and sliding-window sections; the API section
 * says the library follows FLA's chunk_gated_delta_rule signature, with varlen
 * support and an automatic intra-card sequence-parallel switch):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   alpha_t = exp(g_t)
 *     o_t = scale * S_t q_t
 *
 * evaluated chunk by chunk (C = 64) through the WY form (chunked-WY section:
 * step 1 is the chunk's K K^T and its inverse, steps 2-4 the projections, the state
 * recurrence and the output).  S_t is dv x dk; the state crossing this ABI is
 * K-major, h = S^T, element [i][j] = S[j][i].
 *
 * Conventions for every entry point
 *   * Pointers marked "device" are device memory on the current HIP device,
 *     owned by the caller, contiguous, 16-byte aligned, and must stay valid until
 *     the work enqueued on `stream` has finished.  Inputs are never written.
 *     Outputs must not alias inputs or each other.
 *   * Tensor layouts are token-major: q, k [B, T, H, dk]; v, o [B, T, H, dv];
 *     g, beta [B, T, H]; states [N, H, dk, dv] fp32.  With packed sequences
 *     (cu_seqlens != NULL) B must be 1 and the N sequences are the slices
 *     [cu_seqlens[n], cu_seqlens[n+1]) of the T axis.
 *   * Every call is asynchronous on `stream` (never synchronises, allocates
 *     nothing) and returns a status code; all argument checks happen before
 *     the first launch, so an error return means nothing was enqueued, except
 *     GDN_ERR_HIP, which reports a failed launch.
 *   * No exceptions cross this boundary.  The library holds no mutable global
 *     state besides a per-device property cache filled once and, per host
 *     thread, the last few plans (keyed by everything a plan depends on).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------- */
enum {
  GDN_OK = 0,
  GDN_ERR_ARG = -1,          /* null pointer, bad dimension, misalignment, bad cu_seqlens */
  GDN_ERR_UNSUPPORTED = -2,  /* dk/dv not in {64,128}, dtype combination not built, or a
                                problem whose launch grids would exceed 2^32 - 1 work-items */
  GDN_ERR_WORKSPACE = -3,    /* workspace missing or smaller than gdn_chunk_fwd_workspace_bytes */
  GDN_ERR_HIP = -4,          /* a kernel launch failed (hipGetLastError) */
  GDN_ERR_SCRATCH = -5       /* gdn_chunk_fwd_noalloc: the problem's workspace exceeds
                                GDN_NOALLOC_SCRATCH_BYTES */
};

/* ---- element types ----------------------------------------------------------- */
enum { GDN_BF16 = 1, GDN_F32 = 2 };

/* Problem description.  N = B without packing, or the number of packed sequences. */
typedef struct gdn_shape {
  int64_t B, T, H, dk, dv;
  int64_t N;
  int32_t qkv_dtype;   /* dtype of q, k, v and o: GDN_BF16 or GDN_F32 */
  int32_t beta_dtype;  /* dtype of beta: GDN_BF16 or GDN_F32 */
  /* Host copy of cu_seqlens (N+1 int32) when sequences are packed, else NULL.
   * Used to size the launch grids without a device-to-host copy; it must hold
   * the same values as the device array passed to the entry points. */
  const int32_t* cu_seqlens_host;
} gdn_shape;

/* Planner options.  A zeroed struct (or NULL) selects the defaults. */
typedef struct gdn_opts {
  /* 1: never split a sequence: one chunk-serial pass per (sequence, head), bitwise
   *    reproducible run to run and independent of the planner.
   * 0 (default): the planner may cut long sequences into segments that run in
   *    parallel (the pages' automatic intra-card sequence parallelism); results
   *    then match the unsplit path within rounding, not bitwise. */
  int32_t no_split;
  int32_t force_segment_chunks; /* >0: split into segments of this many chunks; 0: planner */
  int32_t force_correction;     /* 1: every split head uses the wrong-start correction
                                   (S*, M and the merge) instead of window-lookback starts */
  float window_log_eps;         /* log of the window tolerance; 0 -> log(2^-16) for bf16
                                   q/k/v, log(2^-24) for fp32 */
  int32_t window_max_chunks;    /* longest lookback window in chunks, 1..16; 0 -> 16 */
  float lambda1_us;             /* planner: cost of one chunk step; 0 -> built in */
  float lambda2_us;             /* planner: cost of one merge step; 0 -> built in */
  int32_t value_block;          /* two-kernel path: value columns per workgroup of the fused
                                   forward, 64 or 128; 0 -> planner's choice */
  /* 1: the one-pass forward (bf16 only; each workgroup forms its chunks' inverses
   *    itself and covers all dv value columns), -1: never (the chunk inverse runs
   *    as its own kernel and the fused forward reads it), 0: planner (bf16 -> one
   *    pass, fp32 -> two kernels). */
  int32_t one_pass;
  /* Optional timing hook: NULL, or an array of 2 * GDN_NUM_STAGES events created by
   * the caller (hipEventCreate).  For every stage that runs, stage_events[2*s] and
   * stage_events[2*s+1] are recorded on `stream` from the dispatch of the stage's
   * first and last kernel (hipExtLaunchKernel: that kernel's start and end; a stage
   * with nothing to launch records both at once).  Events of stages that do not run
   * are left untouched, and NULL entries are skipped (so a caller can time one stage
   * alone).  A stop event alone adds nothing to the stream; a start event makes the
   * runtime insert a marker before the kernel, which idles the GPU for a few
   * microseconds.  Recording events is the only effect. */
  hipEvent_t* stage_events;
} gdn_opts;

/* Stages of gdn_chunk_fwd, in launch order, for gdn_opts.stage_events. */
enum {
  GDN_STAGE_INVERSE = 0,    /* step 1: chunk-local gated Gram matrix and its inverse */
  GDN_STAGE_GATE_SCAN = 1,  /* per-(sequence, head) window decision */
  GDN_STAGE_CP_PASS1 = 2,   /* wrong-start states S* and correction matrices M */
  GDN_STAGE_CP_MERGE = 3,   /* recurrence over segments: true segment starts */
  GDN_STAGE_FORWARD = 4,    /* steps 2-4 fused: writes o and the final state */
  GDN_NUM_STAGES = 5
};

/* Workspace size in bytes that gdn_chunk_fwd needs for this problem and options.
 * Returns GDN_OK and writes *bytes, or an error code for an invalid shape. */
int gdn_chunk_fwd_workspace_bytes(const gdn_shape* shape, const gdn_opts* opts, size_t* bytes);

/*
 * The forward pass.
 *   q, k           device, [B,T,H,dk], dtype shape->qkv_dtype; keys are expected
 *                  L2-normalised per token (the GDN contract; not checked)
 *   v              device, [B,T,H,dv], dtype shape->qkv_dtype
 *   g              device, [B,T,H] fp32: log alpha per token (not cumulated), finite, <= 0
 *   beta           device, [B,T,H], dtype shape->beta_dtype, in [0,1]
 *   initial_state  device, [N,H,dk,dv] fp32, or NULL for a zero start
 *   cu_seqlens     device, [N+1] int32 with cu_seqlens[0] = 0, non-decreasing,
 *                  cu_seqlens[N] = T; or NULL (then N = B and each batch row
 *                  is one sequence of length T)
 *   scale          multiplies every output (typically dk^-1/2)
 *   o              device, [B,T,H,dv], dtype shape->qkv_dtype, fully overwritten
 *   final_state    device, [N,H,dk,dv] fp32, fully overwritten; or NULL (not written)
 *   workspace      device scratch of at least gdn_chunk_fwd_workspace_bytes()
 *   stream         HIP stream the work is enqueued on (0 = null stream)
 */
int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                  float scale, void* o, float* final_state, const gdn_shape* shape,
                  const gdn_opts* opts, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * gdn_chunk_fwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The caller passes inputs and
 * outputs exactly as for gdn_chunk_fwd; the scratch the kernels need (what
 * gdn_chunk_fwd_workspace_bytes() reports) comes from a device array built into the
 * library, GDN_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from library load
 * until the process ends.  Its address is looked up once per device (on the first
 * call made with that device current).  The call makes no hipMalloc or hipFree.
 *
 * Limits and sharing:
 *   * a problem whose workspace exceeds GDN_NOALLOC_SCRATCH_BYTES is rejected with
 *     GDN_ERR_SCRATCH before anything is enqueued;
 *   * every call on one GPU uses that GPU's one array: calls that may overlap on one
 *     GPU (different streams, or different host threads without ordering) race and
 *     must be serialised by the caller; calls on one stream are ordered and safe;
 *   * the array keeps the last call's contents; nothing the kernels read from it
 *     needs to start at zero (every region is written by an earlier kernel of the
 *     same call before it is read).
 * Other arguments, results and errors as gdn_chunk_fwd.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* initial_state,
                          const int32_t* cu_seqlens, float scale, void* o, float* final_state,
                          const gdn_shape* shape, const gdn_opts* opts, hipStream_t stream);

/*
 * One stage of gdn_chunk_fwd (the two-level API of the pages: the API section
 * describes a high-level call and a split, lower-level one for frameworks that
 * schedule the pieces themselves).  `stage` is a GDN_STAGE_* value; every other
 * argument has the meaning it has for gdn_chunk_fwd and must be the same in every
 * stage call of one forward pass.  Running stages 0 .. GDN_NUM_STAGES-1 in order on
 * one stream and one workspace gives gdn_chunk_fwd's result bit for bit; between
 * two stages a caller may read, or replace with bytes produced by the same stage
 * elsewhere, the workspace regions below (gdn_chunk_fwd_workspace_region).  A
 * stage that the plan does not need (the split stages when no sequence is split,
 * the gate scan under force_correction) enqueues nothing and returns GDN_OK.
 * Under a one-pass plan (gdn_plan_one_pass) no stage writes T: the one-pass kernel
 * forms it in pass 1 and in the forward itself.  An unsplit plan's GDN_STAGE_INVERSE
 * enqueues nothing; a split plan's forms only the chunk gate sums.  A
 * split one-pass plan also keeps in the workspace a count of the (sequence, head)
 * pairs that take the correction and a list of pass 1's units (the segments of those pairs
 * but each sequence's last) with its length: GDN_STAGE_INVERSE zeroes both counts,
 * GDN_STAGE_GATE_SCAN adds to them and writes the list, GDN_STAGE_CP_PASS1 runs the
 * listed units, and GDN_STAGE_CP_PASS1 and GDN_STAGE_CP_MERGE do nothing when the
 * pair count is zero (a workspace that receives regions from elsewhere runs those
 * two stages first).
 * With packed sequences every stage call first rebuilds, from cu_seqlens, the
 * chunk and segment tables it indexes by (one small launch; gdn_chunk_fwd builds
 * them once), so no stage indexes by anything a caller or an earlier stage left in
 * the workspace: window lengths read back are clamped to the sequence, list entries
 * to the slots and the list's length to its capacity, and every other workspace
 * byte a stage reads is a value.  Each stage reads what the earlier
 * stages of the same pass wrote into the workspace: running a stage on a workspace
 * where they have not run (or ran with other arguments) gives unspecified output
 * values (never an access outside the buffers the arguments describe).
 * Errors as gdn_chunk_fwd; an unknown stage is GDN_ERR_ARG.
 */
int gdn_chunk_fwd_stage(int stage, const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, float scale, void* o, float* final_state,
                        const gdn_shape* shape, const gdn_opts* opts, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Workspace regions that connect the stages.  Segments are numbered over all
 * sequences in order (segment j of sequence n is seg_base(n) + j, where seg_base
 * counts the segments of the earlier sequences; a sequence that is not split, or
 * is empty, has one), and (segment s, head h) is slot s * H + h. */
enum {
  GDN_REGION_CHUNK_INVERSE = 0,  /* T of every chunk-head: [total_chunks, H, 64, 64] in
                                    shape->qkv_dtype, as gdn_chunk_inverse writes it, except
                                    that the (zero) upper-right 32 x 32 quadrant is not
                                    written (GDN_STAGE_INVERSE; empty under a one-pass
                                    plan) */
  GDN_REGION_SEGMENT_WINDOWS = 1, /* per slot int32: the lookback window, in chunks, of the
                                    segment's start: the smallest W <= min(window_max_chunks,
                                    the start's chunk index) whose W chunks before the start
                                    have a gate sum <= window_log_eps - 1e-3 (fp32 sums), or
                                    W = the start's chunk index (the window reaches the
                                    sequence start, where the state is exact); 0 for first
                                    segments and for every slot of a (sequence, head) with a
                                    start that has none, which takes the correction
                                    (GDN_STAGE_GATE_SCAN; read by every later stage) */
  GDN_REGION_SEGMENT_MAPS = 2,   /* per slot the affine map of its segment: the wrong-start
                                    end state S* (dk * dv fp32 per slot, all slots), then,
                                    at a 256-byte aligned offset, the transition M (2 * dk *
                                    dk bf16 per slot, a high and a low part); element order
                                    inside a slot is the kernels' own (GDN_STAGE_CP_PASS1;
                                    read by GDN_STAGE_CP_MERGE).  Slots of a sequence's last
                                    segment, and of heads that take lookback windows, are
                                    not written */
  GDN_REGION_SEGMENT_STARTS = 3, /* per slot the true start state, [slots, dk, dv] fp32,
                                    K-major like initial_state (GDN_STAGE_CP_MERGE; read by
                                    GDN_STAGE_FORWARD for corrected heads) */
  GDN_NUM_REGIONS = 4
};

/* Byte offset and size of a workspace region for this problem and options (both
 * 0 when the plan does not split, for the two segment regions).  Returns GDN_OK,
 * or an error code for an invalid shape, option or region. */
int gdn_chunk_fwd_workspace_region(const gdn_shape* shape, const gdn_opts* opts, int region,
                                   size_t* offset, size_t* bytes);

/*
 * Step 1 alone (chunked-WY section, first step; the pages cut the kernel after
 * it so the sequence-parallel pass can reuse the inverse): for every chunk c
 * (chunks restart at each sequence start; the last one may be partial) and head h,
 *     A = strict_lower(diag(beta) K K^T * Gamma),  Gamma_rs = exp(G_r - G_s) (r >= s),
 *     T = (I + A)^{-1},
 * G the chunk-local cumulative sum of g.  Rows past a partial chunk's end are
 * treated as k = 0, beta = 0, g = 0 (T is the identity there).
 *   t_out  device, [total_chunks, H, 64, 64] in shape->qkv_dtype (bf16 or fp32),
 *          chunk-major in sequence order; total_chunks = sum_n ceil(len_n / 64).
 *   workspace  device scratch; only used with packed sequences, where it must hold
 *          at least gdn_chunk_fwd_workspace_bytes() bytes (NULL allowed otherwise).
 * Other arguments as in gdn_chunk_fwd.
 */
int gdn_chunk_inverse(const void* k, const float* g, const void* beta,
                      const int32_t* cu_seqlens, const gdn_shape* shape, void* t_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The gate scan alone (sliding-window section: a light kernel scans each head's
 * gates to find the heads whose decay allows window-lookback starts).  For every
 * (sequence n, head h) it writes the smallest W in 1..window_max_chunks such that
 * every run of W consecutive chunks of that sequence (partial last chunk: its real
 * tokens) has a gate sum <= window_log_eps - 1e-3, sums formed in fp32; or 0 if
 * no such W exists.  Starting a segment from a zero state W chunks early then
 * changes the state by at most exp(window_log_eps) times its norm (unit keys,
 * beta in [0,1]).
 *   window_out  device, [N, H] int32
 *   workspace   device scratch of at least gdn_gate_scan_workspace_bytes()
 * Other arguments as in gdn_chunk_fwd.
 */
int gdn_gate_scan(const float* g, const int32_t* cu_seqlens, const gdn_shape* shape,
                  const gdn_opts* opts, int32_t* window_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);
int gdn_gate_scan_workspace_bytes(const gdn_shape* shape, size_t* bytes);

/*
 * Backward of gdn_chunk_fwd: the gradients of L = <d_o, o> + <d_final_state,
 * final_state> with respect to q, k, v, g, beta and initial_state, for the forward
 * that gdn_chunk_fwd computes on the same arguments (FlashQLA talk transcript:
 * results and timeline sections, a backward of the forward's chunk structure;
 * algebraic-rewrites section, the K K^T gradient entering K as (dA + dA^T) K).
 * The forward is recomputed inside, so nothing from a forward call is needed: the
 * chunk inverses and the forward's own recurrence over whole sequences (no split)
 * put the state at every chunk start in the workspace.  bf16 q / k / v: a chain
 * kernel walks the chunks in reverse carrying only the state gradient (dv, and the
 * state gradient after every chunk into the workspace), then every (chunk, head)
 * forms dq, dk, dbeta and dg on its own from the two checkpoints, all products on
 * bf16 MFMA with fp32 accumulation.  fp32: one kernel walks the chunks in reverse
 * in plain fp32 and a second adds the value-column blocks' shares.  The reverse walk
 * is serial per sequence, so when (sequence, head, 32 value columns) workgroups
 * would leave most CUs idle it is split into segments (FlashQLA talk transcript: timeline section, the
 * backward's own intra-GPU sequence parallelism): the state gradient's map over a
 * segment is the transpose of the forward's transition M, so the forward's pass 1
 * forms the transposed maps, a pass from a zero gradient at each segment's end the
 * offsets, the merge the true gradient at every segment's end (from d_final_state,
 * segments last to first), and each segment then runs the full backward from it.
 *   q, k, v, g, beta, initial_state, cu_seqlens, scale   as gdn_chunk_fwd
 *   d_o             device, [B,T,H,dv], dtype shape->qkv_dtype: gradient of o
 *   d_final_state   device, [N,H,dk,dv] fp32: gradient of the final state, or NULL (zero)
 *   dq, dk          device, [B,T,H,dk], dtype shape->qkv_dtype, fully overwritten
 *   dv              device, [B,T,H,dv], dtype shape->qkv_dtype, fully overwritten
 *   dg              device, [B,T,H] fp32 (gradient of the log gate), fully overwritten
 *   dbeta           device, [B,T,H], dtype shape->beta_dtype, fully overwritten
 *   d_initial_state device, [N,H,dk,dv] fp32, fully overwritten; or NULL (not written)
 *   opts            NULL or options: force_segment_chunks (> 0: the split's segment
 *                   length in chunks) and no_split as for gdn_chunk_fwd; the rest is
 *                   ignored.  Default: split when each sequence gets at least four
 *                   segments of at least eight chunks and the units still fit the CUs.
 *   workspace       device scratch of at least gdn_chunk_bwd_workspace_bytes() for the
 *                   same shape and options
 * Precision: fp32 inputs, fp32 arithmetic throughout.  bf16 inputs, bf16 MFMA
 * operands with fp32 accumulation as in the forward, except that the operands the
 * gate gradient is most sensitive to (diag(beta) V' in U, in the chunk-start states'
 * recurrence and in the per-chunk kernel, and d U in the states' update) are carried
 * as bf16 hi + lo pairs.  Errors as gdn_chunk_fwd.
 */
int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, float scale,
                  const void* d_o, const float* d_final_state, void* dq, void* dk, void* dv,
                  float* dg, void* dbeta, float* d_initial_state, const gdn_shape* shape,
                  const gdn_opts* opts, void* workspace, size_t workspace_bytes, hipStream_t stream);
int gdn_chunk_bwd_workspace_bytes(const gdn_shape* shape, const gdn_opts* opts, size_t* bytes);

/* Segment length (chunks) the planner picks for gdn_chunk_fwd, or a negative status.
 * When no sequence is split (no_split, a forced length at or above the longest
 * sequence's chunk count, or the planner's own choice) the value is 1073741823
 * (INT_MAX / 2), so every sequence is one segment. */
int64_t gdn_plan_segment_chunks(const gdn_shape* shape, const gdn_opts* opts);

/* The planner's modelled time of one gdn_chunk_fwd call, in microseconds, for the
 * plan it picks (FlashQLA talk transcript, auto-CP section: a cost model decides the
 * split; here per kernel, fitted on MI355X).  corrected_fraction in [0, 1] is the
 * share of (sequence, head) pairs that take the correction (a segment start without a
 * lookback window; they run pass 1 and the merge; force_correction makes it 1); the
 * planner itself, which cannot see the gates, picks the plan with 0.  Uses the
 * current device's CU count. */
int gdn_plan_predict_us(const gdn_shape* shape, const gdn_opts* opts, double corrected_fraction,
                        double* us);

/* 1 if gdn_chunk_fwd runs the one-pass forward for this problem and options (the
 * chunk inverses formed inside the forward kernel), 0 if it runs the chunk inverse
 * and the fused forward as separate kernels, or a negative status. */
int gdn_plan_one_pass(const gdn_shape* shape, const gdn_opts* opts);

/* Total number of chunks (sum over sequences of ceil(len/64)), or a negative status. */
int64_t gdn_total_chunks(const gdn_shape* shape);

/* Human-readable name of a status code (static string). */
const char* gdn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
