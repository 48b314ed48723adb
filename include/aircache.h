/*
 * aircache.h: C ABI of the MI355X (gfx950) AirCache visual KV-cache compression pass.
 *
 * The pass follows the paper-notes page "AirCache: Activating Inter-Modal
 * Relevancy KV Cache Compression for Efficient Large Vision-Language Model
 * Inference" (ICCV 2025):
 *   - "Elite Observation Window" (key design 1): the text-only attention row of
 *     the last text token picks the elite text tokens (threshold alpha times the
 *     row maximum); the elite queries' softmax over the visual keys plus the
 *     elite text keys, mean-pooled over the elite rows, scores every visual
 *     token (I_v);
 *   - "Layer-wise KV Cache Budget Allocation" (key design 2): strength
 *     s_t = sum I_v and skewness s_k of I_v, normalised across layers, give each
 *     layer's budget r_hat = (s'_t + s'_k) / 2 * r;
 *   - the training-free procedure: after prefill has stored every layer's cache,
 *     budgets are computed for all layers at once and the cache is compressed
 *     before decoding.
 *
 * Two calls carry the pass: aircache_plan (scores, statistics, budgets, top-k
 * selection) and aircache_compress (compaction of the kept visual rows and all
 * text rows into a dense per-layer cache). Both are asynchronous on the given
 * HIP stream, never synchronise the host, allocate nothing, and are
 * deterministic (bit-identical results for identical inputs).
 *
 * Where the page leaves a step open, the library takes these readings:
 *   - per-head attention with D = head_dim; query head h reads KV head
 *     h / (n_q_heads / n_kv_heads); the elite set is chosen once per
 *     (layer, sample) from the mean over query heads of the per-head softmax
 *     rows; I_v averages over all query heads and all elite rows;
 *   - the elite rows' softmax runs over the N_v visual keys plus the N_tk elite
 *     text keys only (no causal mask), so s_t < 1;
 *   - s_k uses the sample standard deviation (n - 1); sigma = 0 gives s_k = 0;
 *   - cross-layer normalisation is per sample: s'_t = s_t * L / sum_l s_t;
 *     s_k is shifted by min(0, min_l s_k) and scaled the same way (all layers 1
 *     when the shifted sum is 0); x = (s'_t + s'_k) / 2 * ratio * N_v in double
 *     precision, budget = clamp(floor(x), 0, N_v);
 *   - top-k keeps the budget largest I_v, equal scores to the lower index, and
 *     lists the kept indices in ascending order;
 *   - compacted layout per layer: samples one after another; inside a sample,
 *     [n_kv_heads][budget + N_t][head_dim]: the kept visual rows (ascending),
 *     then all N_t text rows in their original order.
 *
 * Input layout (per layer l, all device memory, contiguous, read-only):
 *   q_txt[l] : [batch][n_q_heads][n_txt][head_dim]            text queries
 *   k[l], v[l]: [batch][n_kv_heads][n_vis + n_txt][head_dim]   visual rows
 *              first, then text rows (the regrouped sequence)
 * Element type: float32 or bfloat16 (aircache_dtype). Pointers must be 16-byte
 * aligned.
 *
 * Errors: every function returns an aircache_status. Arguments are validated
 * on the host before any launch; on AIRCACHE_EINVAL nothing is enqueued.
 * AIRCACHE_EHIP reports a failed HIP launch. Faults inside the kernels surface
 * through the next HIP call or stream synchronisation. Conditions found on the
 * device are OR-ed into plan->status (AIRCACHE_DEV_*), which the caller reads
 * after synchronising. aircache_last_error() returns a thread-local message
 * describing the last failure of the calling thread.
 */
#ifndef AIRCACHE_H
#define AIRCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AIRCACHE_ABI_VERSION 4
#define AIRCACHE_MAX_LAYERS 128

typedef enum {
  AIRCACHE_OK = 0,
  AIRCACHE_EINVAL = 1,      /* invalid argument; nothing was enqueued */
  AIRCACHE_EWORKSPACE = 2,  /* workspace missing or smaller than aircache_workspace_size */
  AIRCACHE_EHIP = 3         /* a HIP runtime call failed */
} aircache_status;

typedef enum { AIRCACHE_F32 = 0, AIRCACHE_BF16 = 1 } aircache_dtype;

/* Device-side condition bits OR-ed into plan->status. */
#define AIRCACHE_DEV_ELITE_OVERFLOW 1 /* some (layer, sample) had more elite tokens than
                                         desc.max_elite; its results are not valid */
#define AIRCACHE_DEV_TIMEOUT 2        /* a bounded wait between workgroups of the chunked
                                         path expired (workspace not zeroed before its
                                         first use, or the device shared with work that
                                         kept workgroups from running); results are not
                                         valid */

typedef struct {
  int32_t n_layers;   /* L, 1 .. AIRCACHE_MAX_LAYERS */
  int32_t batch;      /* B >= 1 */
  int32_t n_q_heads;  /* H_q >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads; /* H_kv >= 1 */
  int32_t head_dim;   /* D: 64 or 128 */
  int32_t n_vis;      /* N_v >= 3 (the skewness needs three values) */
  int32_t n_txt;      /* N_t >= 1 */
  int32_t dtype;      /* aircache_dtype */
  double alpha;       /* elite threshold in [0, 1]; the page uses 0.9 */
  double ratio;       /* r / N_v, the retention ratio in [0, 1] */
  int32_t max_elite;  /* workspace cap on elite tokens per (layer, sample); 0 means n_txt */
  int32_t path;       /* scoring kernels: AIRCACHE_PATH_AUTO (0), _TILED (1), _ROWS (2)
                         _CHUNKED (3) or _SMALL (4); every path computes the same results */
  int32_t budget_mode; /* layer allocation rule, AIRCACHE_BUDGET_*; 0 is the method's */
  int32_t obs_window;  /* observation window: 0 the method's elite window; k > 0 the last
                          min(k, n_txt) text tokens instead (the window ablation of the
                          "Elite Observation Window" section: 16, 32, or all text tokens);
                          -k (1 <= k <= min(n_vis, n_txt)) the last k visual tokens (the
                          ablation's visual window): their rows normalise over the n_vis
                          visual keys only, the query tables then hold every position's
                          query, [batch][n_q_heads][n_vis + n_txt][head_dim] per layer, the
                          plan's elite_idx the window's positions n_vis - k .. n_vis - 1;
                          served by the tiled path (AUTO resolves to it) */
  int32_t select_mode; /* AIRCACHE_SELECT_*: one selection per (layer, sample), the method's
                          (0), or one per KV head (1) */
} aircache_desc;

/* Visual-token selection granularity. SHARED (0): the method's, one top-r_hat
 * per (layer, sample) by I_v over all query heads. PER_KV_HEAD (1): the
 * group-wise top-K of the edge-device survey page (section 10.1 on GQA/MQA,
 * the query heads that share a KV head decide together): KV head g keeps its
 * own top-r_hat by I_v^g, the mean over its G query heads and the elite rows
 * of the same row softmax; the budget r_hat is still set from the I_v over all
 * query heads (plan->iv, s_t, s_k as in SHARED), so every KV head of a
 * (layer, sample) keeps the same number of rows and the compacted layout is
 * unchanged. Served by the TILED and SMALL paths (AUTO picks between them);
 * ROWS and CHUNKED reject it. */
#define AIRCACHE_SELECT_SHARED 0
#define AIRCACHE_SELECT_PER_KV_HEAD 1

/* Layer budget allocation rules. AIRCACHE (0): the method's, r_hat =
 * 0.5 * (s'_t + s'_k) * r ("Layer-wise KV Cache Budget Allocation", the r_hat
 * equation). The others are the variants that section's allocation ablation
 * compares, read as the same equation with one term or none: UNIFORM (1)
 * r_hat = r, STRENGTH (2) r_hat = s'_t * r, SKEWNESS (3) r_hat = s'_k * r, and
 * PYRAMID (4), the table's pyramid allocation (budgets falling with depth, no
 * formula on the page), read as the linear pyramid with the method's mean
 * budget, r_hat = r * 2 (L - l) / (L + 1) for layer l = 0 .. L - 1; each
 * floored and clamped to [0, N_v] as the method's. */
#define AIRCACHE_BUDGET_AIRCACHE 0
#define AIRCACHE_BUDGET_UNIFORM 1
#define AIRCACHE_BUDGET_STRENGTH 2
#define AIRCACHE_BUDGET_SKEWNESS 3
#define AIRCACHE_BUDGET_PYRAMID 4

/* Scoring paths. TILED: column tiles of every (layer, sample, KV head) with
 * the exponentials spilled to the workspace and a separate merge kernel; any
 * size. ROWS: a workgroup per group of up to four 16-row tiles of elite
 * queries keeps their whole rows of logits in registers (n_vis <= 3072).
 * CHUNKED: one persistent launch for the elite sets, scoring, statistics,
 * budgets and top-k (and, from aircache_run, the compaction): once every
 * elite set size is known, each workgroup takes a chunk of the keys (visual,
 * then elite text) of one (layer, sample) for every KV head, chunks narrower
 * where there are more elite rows, and swaps row maxima and sums with the
 * other chunks of its (layer, sample); any n_kv_heads; n_txt <= 1024,
 * n_layers * batch <= 2048 and the per-layer statistics within a CU's LDS.
 * SMALL: one workgroup runs the whole pass (and, from aircache_run, the
 * compaction) sample after sample, for shapes whose keys and text queries of
 * one sample over all layers fit its LDS with the per-wave buffers
 * (n_vis <= 512, n_q_heads * n_txt <= 8192, n_layers <= 51): no waits
 * between workgroups.
 * AUTO picks SMALL, else CHUNKED, else ROWS, else TILED. */
#define AIRCACHE_PATH_AUTO 0
#define AIRCACHE_PATH_TILED 1
#define AIRCACHE_PATH_ROWS 2
#define AIRCACHE_PATH_CHUNKED 3
#define AIRCACHE_PATH_SMALL 4

/* Outputs of aircache_plan; all device pointers, allocated by the caller with
 * the sizes given, written by the library (row-major, [l][b] means index
 * l * batch + b). */
typedef struct {
  int32_t *elite_idx; /* [L][B][N_t] elite text indices, ascending; first n_elite valid */
  int32_t *n_elite;   /* [L][B] N_tk */
  float *iv;          /* [L][B][N_v] visual importance I_v */
  double *s_t;        /* [L][B] strength, sum of I_v */
  double *s_k;        /* [L][B] skewness of I_v */
  double *budget_x;   /* [L][B] budget before the floor (may be NULL) */
  int32_t *budget;    /* [L][B] r_hat, in [0, N_v] */
  int64_t *out_off;   /* [L][B+1] element offset of each sample's segment in the layer's
                         compacted buffer; out_off[l][B] is the layer's total element count */
  int32_t *kept_idx;  /* [L][B][N_v] kept visual indices, ascending; first budget valid;
                         [L][B][H_kv][N_v] with select_mode PER_KV_HEAD */
  int32_t *status;    /* [1] AIRCACHE_DEV_* bits, reset by every aircache_plan call */
  float *iv_head;     /* [L][B][H_kv][N_v] I_v^g per KV head; written (and required) with
                         select_mode PER_KV_HEAD, not read otherwise (may be NULL) */
} aircache_plan_buf;

/* Library version (AIRCACHE_ABI_VERSION). */
int aircache_abi_version(void);

/* Bytes of device workspace aircache_plan needs for this descriptor, or 0 if
 * the descriptor is invalid (aircache_last_error() says why). The workspace is
 * caller-owned scratch that must be zero-filled before its first use with a
 * descriptor; the library keeps it valid across calls with that descriptor
 * (its counters end every call at zero and its records carry a call count).
 * Zero it again before using it with a different descriptor. One workspace
 * must not be used by two calls that can run concurrently. */
size_t aircache_workspace_size(const aircache_desc *desc);

/* Largest compacted element count per layer (every visual row kept): the
 * worst-case capacity of each k_out[l] / v_out[l] buffer in elements. */
int64_t aircache_max_compacted_elems(const aircache_desc *desc);

/* The scoring path aircache_plan takes for this descriptor:
 * AIRCACHE_PATH_TILED, _ROWS, _CHUNKED or _SMALL (desc->path AIRCACHE_PATH_AUTO
 * resolved), or -1 for an invalid descriptor (aircache_last_error says why).
 * Host only; no device work. */
int32_t aircache_resolved_path(const aircache_desc *desc);

/* Kernel launches aircache_run makes for this descriptor: 1 when the chunked
 * or the small path compacts inside its launch, more when aircache_run falls
 * back to aircache_plan then aircache_compress; -1 for an invalid descriptor.
 * Host only; no device work. */
int32_t aircache_run_launches(const aircache_desc *desc);

/* Scores, statistics, budgets and top-k selection for all layers: the first
 * four steps of the pass on the AirCache paper-notes page.
 *   - elite set and I_v: "Elite Observation Window" (the Att, k, A_vtk and
 *     I_v equations);
 *   - s_t, s_k and the budget r_hat: "Layer-wise KV Cache Budget Allocation"
 *     (the s_t, s_k and r_hat equations, normalised across layers);
 *   - the top-r_hat selection per layer and the rule that budgets are set
 *     once, after prefill, for all layers together: the training-free
 *     procedure (the section on losses and training strategy).
 * Arguments:
 *   q_txt, k : host arrays of n_layers device pointers (layout above)
 *   plan     : output buffers (see aircache_plan_buf)
 *   workspace: device scratch of ws_bytes >= aircache_workspace_size(desc)
 *   stream   : a hipStream_t (NULL: the default stream)
 * The elite selection, scoring and statistics read K and the text queries
 * once; the budget of every layer waits for all layers of its sample, as the
 * procedure on the page prescribes. */
int aircache_plan(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                  const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream);

/* Compaction: the compress step of the training-free procedure on the
 * AirCache paper-notes page (the section on losses and training strategy:
 * after the budgets are set, each layer keeps its selected visual KV and all
 * text KV for decoding). For every (layer, sample, KV head) copy the kept
 * visual rows (plan->kept_idx, ascending) and then all text rows of K and V
 * into k_out[l] / v_out[l] at plan->out_off[l][b]. Bit-exact copies.
 *   k, v        : host arrays of n_layers device pointers (inputs, read-only)
 *   k_out, v_out: host arrays of n_layers device pointers to buffers of at
 *                 least out_off[l][B] elements (aircache_max_compacted_elems is
 *                 always enough); they must not overlap the inputs
 *   plan        : the buffers filled by aircache_plan on the same stream (only
 *                 budget, out_off and kept_idx are read) */
int aircache_compress(const aircache_desc *desc, const aircache_plan_buf *plan,
                      const void *const *k, const void *const *v, void *const *k_out,
                      void *const *v_out, void *stream);

/* The whole pass in one call: aircache_plan then aircache_compress, with the
 * same arguments, results and checks as the two calls on the same stream.
 * Where the chunked path serves the descriptor (aircache_resolved_path) and
 * 5 * n_layers <= 256, one launch does both: the compaction of a (layer,
 * sample) starts as soon as its top-k is out, on workgroups that have
 * finished their scoring work, instead of in a second kernel after the last
 * top-k; the small path's one workgroup also compacts in its launch.
 * Otherwise the two calls are made in order.
 *   q_txt, k, v : host arrays of n_layers device pointers (inputs, read-only)
 *   plan        : output buffers (see aircache_plan_buf), all filled
 *   k_out, v_out: compacted outputs as for aircache_compress
 *   workspace   : as for aircache_plan */
int aircache_run(const aircache_desc *desc, const void *const *q_txt, const void *const *k, const void *const *v,
                 const aircache_plan_buf *plan, void *const *k_out, void *const *v_out, void *workspace,
                 size_t ws_bytes, void *stream);

/* int8 quantisation of the compacted cache, one scale per (layer, sample, KV
 * head) for K and one for V, after the token compression (the UniCache blog,
 * section 6.3 on stacking quantisation with compression: compress first,
 * then quantise; a per-head scale, the head's largest absolute value over the
 * quantisation range). Read as the symmetric range [-127, 127]: per head
 * segment x (its r_hat + n_txt rows of the compacted layout), s = max|x| / 127
 * and code = round-half-to-even(x / s), both in float32 (one correctly
 * rounded division each), s = 0 and every code 0 for an all-zero segment;
 * the value is code * s.
 *   plan        : budget and out_off as written by aircache_plan
 *   k_out, v_out: the compacted buffers of aircache_compress / aircache_run
 *   kq, vq      : host arrays of n_layers device pointers to int8 buffers of
 *                 out_off[l][B] bytes, the same layout as k_out / v_out
 *                 (16-byte aligned)
 *   k_scale, v_scale: device float buffers [L][B][H_kv]
 * Segments whose budget or offset lie outside the buffers (a plan this
 * library did not write) are skipped. */
int aircache_quantize_i8(const aircache_desc *desc, const aircache_plan_buf *plan, const void *const *k_out,
                         const void *const *v_out, int8_t *const *kq, int8_t *const *vq, float *k_scale,
                         float *v_scale, void *stream);

/* aircache_run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same pass, results and checks as aircache_run, with the library's own
 * scratch in place of the caller's workspace. The scratch is a static device
 * array of AIRCACHE_NOALLOC_SCRATCH_BYTES per GPU, held from the library's
 * first use on that GPU until the process ends; this call allocates nothing
 * (no hipMalloc, no allocating library routine). A descriptor whose
 * aircache_workspace_size exceeds that size is rejected with
 * AIRCACHE_EINVAL before anything is enqueued. On a GPU's first call, and on
 * every call whose descriptor differs from the previous call's on that GPU,
 * the part of the scratch the descriptor uses is zeroed first by a kernel on
 * the same stream; otherwise the scratch keeps what the last call left, as a
 * workspace does across aircache_run calls. Every call on one GPU shares that
 * GPU's scratch: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. The remaining arguments
 * are those of aircache_run. */
#define AIRCACHE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int aircache_run_noalloc(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                         const void *const *v, const aircache_plan_buf *plan, void *const *k_out,
                         void *const *v_out, void *stream);

/* Decode attention over the compacted cache, the consumer of the compacted
 * per-layer cache: the KV-cache primer page (devpress.csdn.net), section 2.1
 * "到底缓存什么？", the o_t equation, with one new query per query head and no
 * mask. For every layer l, sample b and query head h, with KV head
 * g = h / (n_q_heads / n_kv_heads) and the n = budget[l][b] + n_txt rows of
 * head g in the (l, b) segment that aircache_compress / aircache_run wrote
 * ([n_kv_heads][n][head_dim] at out_off[l][b]):
 *   o[l][b][h] = softmax(q_dec[l][b][h] . K^T / sqrt(head_dim)) V
 * in float32 arithmetic.
 *   q_dec       : host array of n_layers device pointers, each [B][H_q][D] in
 *                 the descriptor's dtype (read-only)
 *   plan        : only budget and out_off are read (device), as aircache_plan
 *                 or aircache_run left them on the same stream
 *   k_out, v_out: the compacted buffers (read-only)
 *   o           : host array of n_layers device pointers, each [B][H_q][D]
 *                 float32 (written)
 *   workspace   : device scratch of ws_bytes >= aircache_decode_workspace_size
 *                 (no zeroing needed; every word read is written first)
 * All device pointers 16-byte aligned. A workgroup's threads own eight
 * output elements of one query head each: at most 32 query heads per KV head
 * for head_dim 128, 64 for head_dim 64 (AIRCACHE_EINVAL beyond). A segment
 * whose budget or offset is
 * out of range (a plan not written by this library) gives NaN rows instead
 * of reading outside the buffers. */
size_t aircache_decode_workspace_size(const aircache_desc *desc);
int aircache_decode(const aircache_desc *desc, const void *const *q_dec, const aircache_plan_buf *plan,
                    const void *const *k_out, const void *const *v_out, float *const *o, void *workspace,
                    size_t ws_bytes, void *stream);

/* Decode attention over the int8 cache that aircache_quantize_i8 wrote: the
 * same attention as aircache_decode (the primer page's o_t equation) with
 * every cached value read as code * scale, the scale of its (layer, sample,
 * KV head) for K or for V. The codes' dot products with the query are formed
 * in float32 (the codes are exact) and multiplied by the K scale; the
 * weighted sum of V codes is multiplied by the V scale.
 *   kq, vq      : host arrays of n_layers device pointers to the int8 codes,
 *                 the compacted layout of aircache_quantize_i8 (read-only)
 *   k_scale, v_scale: device float [L][B][H_kv] (read-only)
 *   q_dec, plan, o, workspace: as for aircache_decode (the same workspace
 *                 size, aircache_decode_workspace_size)
 * Errors and limits as for aircache_decode; NULL scales are AIRCACHE_EINVAL. */
int aircache_decode_i8(const aircache_desc *desc, const void *const *q_dec, const aircache_plan_buf *plan,
                       const int8_t *const *kq, const int8_t *const *vq, const float *k_scale, const float *v_scale,
                       float *const *o, void *workspace, size_t ws_bytes, void *stream);

/* Prefill attention of one layer with the pass's scoring fused in: the
 * attention is the KV-cache primer page's (devpress.csdn.net) section 2.1
 * o_t equation at every position t of the regrouped sequence (visual tokens
 * first, then text), each position attending to the keys 0..t:
 *   o[b][h][t] = softmax(q[b][h][t] . K_g[0..t]^T / sqrt(head_dim)) V_g[0..t],
 * g = h / (n_q_heads / n_kv_heads), float32 accumulation, the probabilities
 * rounded to bfloat16 for the product with V, the output rounded to bfloat16.
 * The same call writes layer `layer`'s rows of the plan as aircache_plan
 * would (elite set, I_v, s_t, s_k; the AirCache paper-notes page, "Elite
 * Observation Window" and the strength and skewness equations): the elite
 * rows' logits against the visual keys are taken from the attention itself,
 * so the visual keys are read once. The call for the last layer also computes
 * the budgets and the top-r_hat selection of every layer ("Layer-wise KV Cache
 * Budget Allocation"), after which the plan is complete and aircache_compress
 * compacts the cache.
 *   layer       : 0 .. n_layers - 1; the calls for one pass are made for the
 *                 layers 0, 1, .., n_layers - 1 in this order on one stream
 *                 (layer 0 opens the pass and clears plan->status)
 *   q           : device [batch][n_q_heads][n_vis + n_txt][head_dim], every
 *                 position's query (the text rows are the pass's q_txt)
 *   k, v        : device [batch][n_kv_heads][n_vis + n_txt][head_dim]
 *   o           : device [batch][n_q_heads][n_vis + n_txt][head_dim] (written;
 *                 must not overlap q, k or v)
 *   plan        : as for aircache_plan (every output pointer but budget_x may
 *                 be used; iv_head with AIRCACHE_SELECT_PER_KV_HEAD)
 *   workspace   : device scratch of ws_bytes >=
 *                 aircache_prefill_workspace_size(desc), kept by the caller
 *                 across the layer calls of one pass (two layers' scoring
 *                 terms, sized for max_elite elite rows per (layer, sample),
 *                 plus the pass's counters; no zeroing needed). With
 *                 max_elite = 0 the cap is n_txt, which for long text makes
 *                 this large (batch 8, n_txt 1024, n_vis 3072: 5.6 GB)
 * bfloat16 only (AIRCACHE_EINVAL for float32); head_dim 64 or 128; all
 * pointers 16-byte aligned. The descriptor's path is ignored; max_elite caps
 * the elite rows that are scored per (layer, sample) as on the other paths
 * (overflow is flagged in plan->status). */
size_t aircache_prefill_workspace_size(const aircache_desc *desc);
int aircache_prefill_layer(const aircache_desc *desc, int32_t layer, const void *q, const void *k, const void *v,
                           void *o, const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream);

/* The same prefill attention of one layer without the scoring: o only, no
 * plan and no workspace (arguments as for aircache_prefill_layer). */
int aircache_prefill_attention(const aircache_desc *desc, const void *q, const void *k, const void *v, void *o,
                               void *stream);

/* Instrumented variants of aircache_plan / aircache_compress / aircache_run for
 * timing individual kernels. events is a host array of hipEvent_t handles created by
 * the caller: events[i] is recorded on the stream just before the i-th kernel
 * of the call and events[n_events - 1] after the last one. n_events must be
 * AIRCACHE_PLAN_KERNELS + 1 (kernels: elite_select, cross_score, finalize,
 * topk_select), AIRCACHE_COMPRESS_KERNELS + 1 (kernel: kv_gather) or
 * AIRCACHE_RUN_KERNELS + 1 (the whole pass); NULL events gives the plain call.
 * Results are identical to the plain calls. */
#define AIRCACHE_PLAN_KERNELS 4
#define AIRCACHE_COMPRESS_KERNELS 1
#define AIRCACHE_RUN_KERNELS 1 /* aircache_run_profiled: events bracket the whole pass */
int aircache_plan_profiled(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                           const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream,
                           void *const *events, int n_events);
int aircache_compress_profiled(const aircache_desc *desc, const aircache_plan_buf *plan,
                               const void *const *k, const void *const *v, void *const *k_out,
                               void *const *v_out, void *stream, void *const *events, int n_events);
int aircache_run_profiled(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                          const void *const *v, const aircache_plan_buf *plan, void *const *k_out,
                          void *const *v_out, void *workspace, size_t ws_bytes, void *stream,
                          void *const *events, int n_events);

/* Text of an aircache_status value. */
const char *aircache_strerror(int status);

/* Message describing the calling thread's last failure ("" if none). */
const char *aircache_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AIRCACHE_H */
