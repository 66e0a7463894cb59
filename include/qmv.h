/*
 * qmv.h -- C ABI of libqmv, the MI355X (gfx950) quantized matrix-vector library.
 *
 * What it computes (the pages' statement of the problem):
 *   - Weights are ternary, five trits per byte with one fp32 scale per matrix
 *     ("Gemma 3 1B at 114 tokens per second on a laptop CPU", sections
 *     "Step 1: a kernel for 1.6-bit weights" and "Step 2: making a ternary
 *     Gemma"), or int8 with one symmetric per-tensor scale (cpp20gemma README,
 *     "Architecture & implementation").
 *   - Activations are rounded to int8 with one scale per token ("Step 2";
 *     llama2.c tour, "Key ideas & tradeoffs": activations quantised at run
 *     time).
 *   - Dot products are exact int32 sums; the two scales are applied once,
 *     after the sum (cpp20gemma, "Architecture & implementation").
 *   - Many tokens ("lanes") can share one pass over the weights ("Many users
 *     at once"; "Step 1": prompt tokens go through each matrix in one pass).
 *   - The output layer is a bf16 matrix-vector product followed by a greedy
 *     choice of the first maximum ("Step 3: the output layer became the
 *     bottleneck"; llama2.c tour, "Sampling").
 *
 * Conventions (apply to every call):
 *   - Pointers are DEVICE pointers unless marked "host".  Every buffer is owned
 *     by the caller; the library never allocates or frees device memory.
 *     Scratch memory is passed in as `workspace` (except for
 *     qmv_lmhead_argmax_static, whose scratch is a fixed array in the
 *     library's code object).
 *   - Calls are asynchronous: host-side arguments are validated synchronously;
 *     on a validation failure the call returns a negative status and enqueues
 *     nothing.  Otherwise the work is enqueued on `stream` (a hipStream_t;
 *     NULL = the null stream) and the call returns QMV_OK, or QMV_EHIP if the
 *     HIP runtime reported an error when enqueuing.
 *   - There are no device-side error reports apart from the optional invalid
 *     trit counter of qmv_pack_ternary and the status word of qmv_ffn_decode;
 *     read them after synchronising.
 *   - Non-finite fp32 inputs are outside the contract.
 *   - State: the library keeps one record per device, filled once on the
 *     first call that needs it (the compute-unit count, the kernels'
 *     dynamic-LDS limit, the device address of qmv_lmhead_argmax_static's
 *     scratch array), and nothing else between calls.  A plan (qmv_plan_*)
 *     is host memory the caller owns through its handle.  Calls on different
 *     streams with different buffers and workspaces may run concurrently.
 *
 * Device weight layout (both weight types): a row's bytes are cut into
 * 16-byte chunks and chunk c of every row is stored before chunk c+1 of any
 * row, i.e. byte j of row r lives at ((j / 16) * n + r) * 16 + (j % 16).
 * Row byte counts are padded to a multiple of 16.
 *   - ternary: row bytes = ceil(k/5); byte j holds columns 5j..5j+4 as the
 *     base-3 number sum_i (t[5j+i] + 1) * 3^i (0..242); columns >= k and the
 *     padding bytes hold trit 0 (a padding byte is 121).
 *   - int8: row bytes = k int8 codes, zero padded.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call (0 = success). */
enum {
    QMV_OK = 0,
    QMV_EINVAL = -1,        /* null pointer, negative size or bad flag */
    QMV_ESHAPE = -2,        /* sizes inconsistent or beyond the supported range */
    QMV_EVALUE = -3,        /* a host-side value is out of range (e.g. a non-finite scale) */
    QMV_EHIP = -4,          /* the HIP runtime reported an error */
    QMV_EUNSUPPORTED = -5,  /* unknown weight type */
    QMV_EWORKSPACE = -6     /* workspace missing or too small */
};

/* Weight types. */
enum {
    QMV_W_TERNARY5 = 1,     /* five trits per byte, one fp32 scale per matrix */
    QMV_W_INT8 = 2,         /* int8 codes, one fp32 scale per tensor */
    QMV_W_INT8_G128 = 3     /* int8 codes, one fp32 scale per QMV_WEIGHT_GROUP columns of a row */
};

/* Group sizes of the group-scaled path (QMV_W_INT8_G128 and
 * qmv_quantize_act_grouped). */
#define QMV_WEIGHT_GROUP 128
#define QMV_ACT_GROUP 32

/* Limits. */
#define QMV_MAX_GEMV_M 16            /* tokens per qmv_gemv problem */
#define QMV_MAX_K (1 << 20)          /* input columns */
#define QMV_MAX_N (1 << 24)          /* output rows */

/* A packed weight matrix (host struct describing device memory). */
typedef struct qmv_weight {
    int32_t wtype;          /* QMV_W_TERNARY5, QMV_W_INT8 or QMV_W_INT8_G128 */
    int32_t reserved;       /* must be 0 */
    int64_t n;              /* output rows */
    int64_t k;              /* input columns */
    const void* data;       /* device, qmv_packed_bytes(wtype, n, k) bytes, 16-byte aligned */
    const float* scale;     /* device, 1 fp32; QMV_W_INT8_G128: [n][ceil(k/128)] fp32 */
} qmv_weight;

/* One matrix-times-activations problem: y[m][n] = (x8[m][:] . W[n][:]) * sx[m] * scale.
 * For QMV_W_INT8_G128 weights the activations carry one scale per 32 columns
 * and y[m][n] = sum_h (scale[n][h/4] * sx[m][h]) * D_h, D_h the exact int32 dot
 * of columns 32h .. 32h+31 (see qmv_pack_int8_grouped). */
typedef struct qmv_problem {
    qmv_weight w;
    const int8_t* x8;       /* device, [m][k] int8, row-major, natural column order */
    const float* sx;        /* device, [m] fp32 per-token scales; QMV_W_INT8_G128: [m][ceil(k/32)] */
    int64_t m;              /* tokens (lanes) */
    float* y;               /* device, [m][n] fp32, row-major */
    int32_t* acc;           /* device, [m][n] int32 exact dot products; NULL = not wanted (must be NULL
                               for QMV_W_INT8_G128) */
} qmv_problem;

/* Library version string and status names (static strings). */
const char* qmv_version(void);
const char* qmv_status_str(int32_t status);

/* Bytes of a packed matrix in the device layout: n * roundup(ceil(k/5), 16)
 * for QMV_W_TERNARY5, n * roundup(k, 16) for QMV_W_INT8 and QMV_W_INT8_G128;
 * -1 on bad input. */
int64_t qmv_packed_bytes(int32_t wtype, int64_t n, int64_t k);

/*
 * qmv_pack_ternary -- trits -> five trits per byte ("Step 1": 3^5 = 243 codes
 * fit in a byte; "Step 2": one scale per matrix).
 *   trits     [n][k] int8 in {-1, 0, +1}, row-major.  A value outside the set
 *             is packed as 0 and counted in *bad_count.
 *   scale     the matrix scale (host value, finite) -> written to *scale_out.
 *   packed    qmv_packed_bytes(QMV_W_TERNARY5, n, k) bytes, 16-byte aligned.
 *   scale_out 1 fp32.
 *   bad_count nullable; 1 int32, zeroed and then incremented in-stream.
 *   desc_out  nullable host struct, filled in on success.
 * One-time preparation, not part of the per-token path.
 */
int32_t qmv_pack_ternary(const int8_t* trits, int64_t n, int64_t k, float scale, void* packed,
                         float* scale_out, int32_t* bad_count, qmv_weight* desc_out, void* stream);

/*
 * qmv_pack_int8 -- fp32 weights -> int8 codes with one per-tensor scale
 * (cpp20gemma, "Architecture & implementation"):
 *   scale = max(max|w|, 1e-9) / 127 (fp32, correctly rounded),
 *   code  = clip(round_half_even(w / scale), -128, 127) (IEEE fp32 division).
 *   w         [n][k] fp32, row-major, finite.
 *   packed    qmv_packed_bytes(QMV_W_INT8, n, k) bytes, 16-byte aligned.
 *   scale_out 1 fp32 (also used as the in-stream max cell while packing).
 *   desc_out  nullable host struct.
 */
int32_t qmv_pack_int8(const float* w, int64_t n, int64_t k, void* packed, float* scale_out,
                      qmv_weight* desc_out, void* stream);

/*
 * qmv_pack_int8_grouped -- fp32 weights -> int8 codes in groups of
 * QMV_WEIGHT_GROUP (128) consecutive columns of a row, one fp32 scale per group
 * (gemma.cpp tour, "Weights, Blobs, and the .sbs Format": int8 groups of 128
 * sharing one scale).  Each group is quantised by qmv_pack_int8's rule; the
 * last group of a row may be shorter; groups never span rows.
 *   w       [n][k] fp32, row-major, finite.
 *   packed  qmv_packed_bytes(QMV_W_INT8_G128, n, k) bytes, 16-byte aligned:
 *           row-major int8, each row padded with zero bytes to roundup(k, 16)
 *           (unlike QMV_W_INT8, rows are not chunk-interleaved).
 *   scales  [n][ceil(k/128)] fp32, written in-stream.
 *   desc_out nullable host struct (wtype QMV_W_INT8_G128, scale = scales).
 * Limits: k <= 65536, n <= 2^20, n * roundup(k, 16) < 2^31 (QMV_ESHAPE).
 * For the activations of such a matrix use qmv_quantize_act_grouped.
 */
int32_t qmv_pack_int8_grouped(const float* w, int64_t n, int64_t k, void* packed, float* scales,
                              qmv_weight* desc_out, void* stream);

/*
 * qmv_quantize_act_grouped -- int8 activations with one scale per
 * QMV_ACT_GROUP (32) consecutive columns of a row ("Gemma 3 1B at 114 tokens
 * per second on a laptop CPU", "A side finding: Gemma 4 E4B in 4-bit": one
 * activation scale per 32 values instead of one per token), each group by
 * qmv_quantize_act's rule; the last group of a row may be shorter.
 *   x [m][k] fp32 row-major, finite.   x8 [m][k] int8.   sx [m][ceil(k/32)] fp32.
 * Pair with QMV_W_INT8_G128 weights in qmv_gemv: activation group h lies in
 * weight group h / 4, its dot product is exact in int32 and both scales are
 * applied after it; y is summed over h in fp32 (within (ceil(k/32) + 3) * 2^-24
 * of sum_h |term| of the exact result).  Such problems take acc = NULL and
 * need m * (roundup(k, 32) + 4 * ceil(k/32)) <= 160 KB (activations staged in
 * LDS); otherwise QMV_EINVAL / QMV_ESHAPE.
 */
int32_t qmv_quantize_act_grouped(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, void* stream);

/*
 * qmv_quantize_act -- per-token int8 activation quantisation ("Step 2": the
 * inputs of every layer are rounded to int8; same formula as qmv_pack_int8,
 * one scale per row).
 *   x   [m][k] fp32 row-major, finite.   x8 [m][k] int8.   sx [m] fp32.
 *   A row of zeros gets sx = 1e-9/127 and all-zero codes.
 */
int32_t qmv_quantize_act(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, void* stream);

/* One activation set of qmv_quantize_act_many (host struct describing device memory). */
typedef struct qmv_act {
    const float* x;         /* device, [m][k] fp32 row-major, finite */
    int64_t m;              /* rows (tokens) */
    int64_t k;              /* columns */
    int8_t* x8;             /* device, [m][k] int8 codes */
    float* sx;              /* device, [m] fp32 scales */
} qmv_act;

#define QMV_MAX_ACT_SETS 8           /* activation sets per qmv_quantize_act_many call */

/*
 * qmv_quantize_act_many -- qmv_quantize_act over up to QMV_MAX_ACT_SETS sets of
 * activations of different widths in one launch (a decode step's inputs of
 * every width at once); each set's codes and scales are bit-identical to
 * qmv_quantize_act on that set.
 *   acts  host array of `count` sets, 1 <= count <= QMV_MAX_ACT_SETS.
 * EINVAL for a NULL array or pointer, ESHAPE for a bad count or shape or more
 * than 2^31 - 1 rows in all.
 */
int32_t qmv_quantize_act_many(const qmv_act* acts, int32_t count, void* stream);

/*
 * qmv_rmsnorm_quantize -- RMSNorm, then the same per-token quantisation, in one
 * pass (llama2.c tour, "Step 1" / "Step 6": o = weight * (x / rms), rms =
 * sqrt(mean(x^2) + eps); the normalised row never goes to memory).
 *   x      [m][k] fp32 row-major, finite.   weight [k] fp32.   eps >= 0.
 *   x8/sx  as qmv_quantize_act, of o.
 * fp32 throughout, in a fixed order so results are reproducible: the sum of
 * squares is 256 partial sums (partial t over j = t, t + 256, ... in order)
 * added pairwise (t += t + s, s = 128 .. 1); r = 1 / sqrt(ss / k + eps) with
 * correctly rounded division and root; o = weight * (r * x); no fused
 * multiply-adds.  EVALUE for a negative or non-finite eps.
 */
int32_t qmv_rmsnorm_quantize(const float* x, const float* weight, int64_t m, int64_t k, float eps, int8_t* x8,
                             float* sx, void* stream);

/* Gate activations of qmv_glu_quantize. */
enum {
    QMV_ACT_GELU_TANH = 1,  /* 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), the GeGLU gate */
    QMV_ACT_SILU = 2        /* v / (1 + exp(-v)), the SwiGLU gate */
};

/*
 * qmv_glu_quantize -- the gated feed-forward's middle step and the
 * quantisation for the down projection in one pass (llama2.c tour, "Step 5":
 * act(gate) * up; Gemma uses a GeLU gate): h = act(gate) * up per element, then
 * per-row int8 codes and scales of h as qmv_quantize_act.
 *   gate, up [m][n] fp32, finite.   x8 [m][n].   sx [m].
 * fp32 with the device's exp / tanh.  EINVAL for an unknown act.
 */
int32_t qmv_glu_quantize(const float* gate, const float* up, int64_t m, int64_t n, int32_t act, int8_t* x8, float* sx,
                         void* stream);

/* ---- The feed-forward half of a layer stack in one persistent launch ---------- */

/* One layer of qmv_ffn_decode (host struct describing device memory). */
typedef struct qmv_ffn_layer {
    qmv_weight gate;        /* QMV_W_TERNARY5, n = inter, k = hidden */
    qmv_weight up;          /* QMV_W_TERNARY5, n = inter, k = hidden */
    qmv_weight down;        /* QMV_W_TERNARY5, n = hidden, k = inter */
    const float* norm;      /* device, [hidden] fp32 RMSNorm weights */
} qmv_ffn_layer;

/* End status of a qmv_ffn_decode call (written to its status word). */
enum {
    QMV_FFN_OK = 0,
    QMV_FFN_CANCELLED = 1,  /* the cancel word was nonzero at a wait */
    QMV_FFN_TIMEOUT = 2     /* a wait ran out of polls (e.g. workgroups not all resident) */
};

#define QMV_FFN_LAUNCH_LAYERS 32     /* layers per kernel launch; more layers take more launches */
#define QMV_FFN_TRACE_STAMPS 12      /* trace stamps per layer (qmv_ffn_decode) */
#define QMV_FFN_MAX_HIDDEN 8192
#define QMV_FFN_MAX_INTER 65536

/* Workspace bytes of qmv_ffn_decode (-1 on bad sizes). */
int64_t qmv_ffn_workspace_bytes(int64_t hidden, int64_t inter);

/* Workgroups of one qmv_ffn_decode launch on the current device (the trace's
 * first dimension), or a negative status. */
int32_t qmv_ffn_grid(int32_t* grid /* host */);

/*
 * qmv_ffn_decode -- for one token, the feed-forward half of nlayers decoder
 * layers (llama2.c tour, "forward": Step 5 and the residual connection after
 * it; gemma.cpp tour, "The Forward Pass, Layer by Layer"), each layer being
 *     x8, sx = qmv_rmsnorm_quantize(h, norm, eps)
 *     g, u   = qmv_gemv of gate and up against (x8, sx)
 *     q8, sq = qmv_glu_quantize(g, u, act)
 *     y      = qmv_gemv of down against (q8, sq)
 *     h      = h + y                                   (fp32 add)
 * with results identical bit for bit to that chain of calls.  All layers run
 * in one kernel launch (QMV_FFN_LAUNCH_LAYERS per launch) whose steps wait for
 * each other inside the kernel: the launch needs every one of its workgroups
 * resident at once (qmv_ffn_grid of them; the kernel shares the GPU with no
 * other work on other streams for the duration).
 *   layers     host, nlayers >= 1 entries, every layer of the same hidden and
 *              inter (1 <= hidden <= QMV_FFN_MAX_HIDDEN, 1 <= inter <=
 *              QMV_FFN_MAX_INTER); weights ternary, 16-byte aligned.
 *   h          device, [hidden] fp32, finite: the residual stream, updated in
 *              place.
 *   eps        RMSNorm epsilon (>= 0, finite).   act  QMV_ACT_*.
 *   workspace  >= qmv_ffn_workspace_bytes(hidden, inter) bytes, 256-byte
 *              aligned, zero-filled before its first use; every launch leaves
 *              it zero-filled again (also when it stops early), so calls on
 *              one stream may share it; calls that overlap must not.
 *   cancel     nullable: a device word, or host memory the device can read
 *              (hipHostMalloc); while it is nonzero every wait stops the launch
 *              (status QMV_FFN_CANCELLED).
 *   spin_limit polls per wait before the launch stops with QMV_FFN_TIMEOUT
 *              (0 = 2^20, about a second; a wait normally takes a few polls).
 *   status     device, 1 int32, required: QMV_FFN_OK or the first QMV_FFN_*
 *              error of the call; on an error the launches after it do
 *              nothing and h is unspecified (its input, or the state after
 *              some of the layers).
 *   trace      nullable (then nlayers <= QMV_FFN_LAUNCH_LAYERS): device
 *              uint64 [grid][1 + QMV_FFN_TRACE_STAMPS * nlayers] in ticks of the
 *              device's 100 MHz constant clock: each workgroup's start, then
 *              per layer: 0 layer start; for a workgroup with a gate/up task
 *              (32 rows of both, workgroup b takes rows 32 b ..) 1 down sums of
 *              the previous layer gathered, 2 RMSNorm's scale known, 3 codes
 *              written, 4 their staged form ready, 5 gate/up and GLU values
 *              written; for a workgroup with a down task (workgroup b takes task
 *              b) 6 its GLU inputs gathered, 7 staged, 8 dots done, 9 the atomic
 *              adds acknowledged (its completion mark follows); 10 layer end;
 *              11 (a count, not a time) the poll rounds of the layer's waits.
 *              Stamps a workgroup does not reach are 0.
 * EINVAL / ESHAPE / EUNSUPPORTED / EVALUE / EWORKSPACE on bad arguments.
 */
int32_t qmv_ffn_decode(const qmv_ffn_layer* layers /* host */, int32_t nlayers, float* h, float eps, int32_t act,
                       void* workspace, int64_t ws_bytes, const int32_t* cancel, int64_t spin_limit,
                       int32_t* status, uint64_t* trace, void* stream);

/* Workspace bytes for this problem list (-1 on bad input); the workspace
 * must be 256-byte aligned.  qmv_workspace_bytes covers both qmv_gemv and
 * qmv_gemm_prefill (the larger need of the calls that accept the list);
 * the other two are each call's own need. */
int64_t qmv_workspace_bytes(const qmv_problem* probs /* host */, int32_t count);
int64_t qmv_gemv_workspace_bytes(const qmv_problem* probs /* host */, int32_t count);
int64_t qmv_prefill_workspace_bytes(const qmv_problem* probs /* host */, int32_t count);

/*
 * qmv_gemv -- grouped weight-streaming matrix-vector products for 1..16 tokens
 * ("On a CPU, speed is bytes": every weight byte is read once per step;
 * "Many users at once": one read of each byte serves every lane).
 *   probs     host array of `count` problems (1 <= count); each problem has
 *             1 <= m <= QMV_MAX_GEMV_M, its own weights, activations and
 *             outputs.  All problems of one weight type run in one kernel
 *             launch (one launch per type present).
 *   workspace device, >= qmv_gemv_workspace_bytes(probs, count) bytes; the
 *             call schedules the list, uploads the schedule into the
 *             workspace in-stream and launches.  For the same list launched
 *             again (a decode loop) make a plan once instead (qmv_plan_*).
 * y (and acc when non-NULL) are written for every problem.  x8/acc must not
 * alias y.  Results are exact in acc and do not depend on the grouping.
 * QMV_W_INT8_G128 problems are summed in fp32 over their activation groups
 * (see qmv_quantize_act_grouped).  The upload copies from host memory that is
 * released on return, so the call is refused (QMV_EUNSUPPORTED) while
 * `stream` is being captured into a graph; capture qmv_plan_launch instead.
 */
int32_t qmv_gemv(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, void* stream);

/*
 * qmv_gemm_prefill -- the same products for any number of tokens, computed
 * with int8 matrix cores ("Step 1": all prompt tokens go through each weight
 * matrix in one pass).  Ternary weights only.  Same arguments and results as
 * qmv_gemv, with 1 <= m <= 65536 per problem.  The workspace also holds the
 * kernel's tile tickets (zeroed by the upload, left at zero by every launch),
 * so launches that share a workspace must not overlap in time.
 */
int32_t qmv_gemm_prefill(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, void* stream);

/*
 * Plans: one problem list scheduled once and launched many times, as a decode
 * loop with fixed buffers does (the schedule and tile tables depend only on
 * the list and the device).  A plan is host memory owned by the caller
 * through its handle; it is made for the device current at qmv_plan_create
 * and must be used with streams of that device.
 *   kind      QMV_PLAN_GEMV (the launches of qmv_gemv), QMV_PLAN_PREFILL
 *             (those of qmv_gemm_prefill), or QMV_PLAN_GEMV_DOT (qmv_gemv's
 *             products with vector dot-product instructions only, no matrix
 *             cores: a comparison point), or QMV_PLAN_GEMV_SKIP_ZERO
 *             (qmv_gemv's products, with the one- and two-token ternary
 *             kernel skipping every 20-column activation unit that is zero
 *             for all tokens -- the work of "What is next": skipping groups
 *             of zero inputs; exact, since such units add nothing; the
 *             weights are still read); the list is validated as by the
 *             corresponding call.  Results are identical across the kinds.
 *   qmv_plan_workspace_bytes  exact workspace bytes of the plan.
 *   qmv_plan_upload  copies the plan's tables into `workspace` (in-stream,
 *             from the plan's host memory, which lives until
 *             qmv_plan_destroy).  Once per workspace, before its first launch.
 *   qmv_plan_launch  enqueues the kernels only (no copies, no allocation, no
 *             device queries): safe to capture in a graph.  Launches that
 *             share a workspace must not overlap in time.  The buffers named
 *             in the list must still be valid.
 * EINVAL for a null plan or handle pointer or an unknown kind, EWORKSPACE for
 * a missing, misaligned or small workspace, EHIP with no usable device.
 */
typedef struct qmv_plan qmv_plan;
enum { QMV_PLAN_GEMV = 1, QMV_PLAN_PREFILL = 2, QMV_PLAN_GEMV_DOT = 3, QMV_PLAN_GEMV_SKIP_ZERO = 4 };
int32_t qmv_plan_create(int32_t kind, const qmv_problem* probs /* host */, int32_t count, qmv_plan** plan);
int64_t qmv_plan_workspace_bytes(const qmv_plan* plan);
int32_t qmv_plan_upload(const qmv_plan* plan, void* workspace, int64_t ws_bytes, void* stream);
int32_t qmv_plan_launch(const qmv_plan* plan, void* workspace, int64_t ws_bytes, void* stream);
void qmv_plan_destroy(qmv_plan* plan);

/* Workspace bytes of qmv_lmhead_argmax for a v x k head. */
int64_t qmv_lmhead_workspace_bytes(int64_t v, int64_t k);

/*
 * qmv_lmhead_argmax -- output layer and greedy choice ("Step 3": score every
 * vocabulary row against the final hidden state; llama2.c "Sampling": greedy
 * keeps the first maximum).
 *   w_bf16    [v][k] bf16 bit patterns, row-major, 16-byte aligned.
 *   x         [k] fp32 hidden state.
 *   logit[r]  = sum_c float(w[r][c]) * x[c], accumulated in fp32.
 *   idx       1 int32: smallest r with the largest logit.
 *   max_logit nullable, 1 fp32: that logit.
 *   logits    nullable, [v] fp32: every logit.
 *   workspace >= qmv_lmhead_workspace_bytes(v, k) bytes, 256-byte aligned.
 */
int32_t qmv_lmhead_argmax(const uint16_t* w_bf16, const float* x, int64_t v, int64_t k, int32_t* idx,
                          float* max_logit, float* logits, void* workspace, int64_t ws_bytes,
                          void* stream);

/*
 * qmv_lmhead_argmax_static -- qmv_lmhead_argmax without a workspace, for
 * callers that cannot allocate device memory (code under graph capture,
 * serving loops that forbid allocation).  Same arguments and results; the
 * per-workgroup maxima go to a scratch array of 256 KiB that the library
 * holds on each device until the process ends, so v <= 2^21 rows (else
 * QMV_ESHAPE).  Every call on one device shares that array: calls that
 * overlap in time on one device race.  Nothing is allocated or freed; EHIP
 * with no usable device.
 */
int32_t qmv_lmhead_argmax_static(const uint16_t* w_bf16, const float* x, int64_t v, int64_t k, int32_t* idx,
                                 float* max_logit, float* logits, void* stream);

/*
 * The sketch head ("Step 3": candidates first, exact scores only for them).
 * For each token:
 *   1. the T = min(32, k) hidden dimensions with the largest |x| (ties to the
 *      lower index) are scored exactly for every word;
 *   2. the other dimensions are scored from the sign bits of the table: in
 *      rank order they form 4 groups (floor((k-T)/4) each, the last takes the
 *      rest), and group g adds c * mean|x|_g * (agreeing - disagreeing signs),
 *      c being the mean |w| of the table (a sign bit is set for a value < 0);
 *      the score is fp32: a = fma(w, x, a) over the exact dimensions in index
 *      order, then a = fma(weight_g, agreement_g, a) for g = 0..3;
 *   3. the candidates are the words whose score falls in the top bins that
 *      hold at least min(1024, v) words, a bin being the top 13 bits of the
 *      score's order-preserving key (a sixteenth of an octave), the bins
 *      searched being the 256 below the highest non-empty one (16 octaves;
 *      if they hold fewer words, every word is a candidate); only they are
 *      scored exactly (as in qmv_lmhead_argmax) and the first maximum among
 *      them is the choice.
 * Two launches per token (scores; cut, rescoring and choice).
 * Limits: 8 <= k <= 8192, k % 8 == 0, 1 <= v <= QMV_MAX_N.
 */
int64_t qmv_sketch_bytes(int64_t v, int64_t k);            /* -1 on bad shape */
int64_t qmv_sketch_workspace_bytes(int64_t v, int64_t k);  /* -1 on bad shape */

/*
 * qmv_sketch_build -- one-time preparation from the output layer's weights:
 * the sign bits (word d/32 of row r at (d/32)*vp + r), a dimension-major bf16
 * copy [k][vp] and c, in `sketch` (256-byte aligned, >= qmv_sketch_bytes);
 * vp = v rounded up to a multiple of 1024, rows v..vp-1 zero in both tables.
 *   w_bf16  [v][k] bf16 bit patterns, row-major, 16-byte aligned, finite.
 * Not part of the per-token path.  EINVAL / ESHAPE / EWORKSPACE as above.
 */
int32_t qmv_sketch_build(const uint16_t* w_bf16, int64_t v, int64_t k, void* sketch, int64_t sketch_bytes,
                         void* stream);

/*
 * qmv_lmhead_sketch_argmax -- the greedy choice through the sketch head.
 *   w_bf16     the same table the sketch was built from (exact rescoring).
 *   x          [k] fp32 hidden state, finite, 16-byte aligned.
 *   idx        1 int32: the chosen word.
 *   max_logit  nullable, 1 fp32: its exact logit.
 *   candidates nullable, 1 int32: how many words were rescored.
 *   scores     nullable, [v] fp32: every word's approximate score (step 1+2).
 *   workspace  >= qmv_sketch_workspace_bytes(v, k) bytes, 256-byte aligned,
 *              zero-filled before its first use; it carries state from one
 *              call to the next and every call leaves it ready for the next
 *              (also for other shapes).  Calls that share it must not
 *              overlap; if a launch fails (QMV_EHIP), zero it again.
 */
int32_t qmv_lmhead_sketch_argmax(const uint16_t* w_bf16, const void* sketch, const float* x, int64_t v,
                                 int64_t k, int32_t* idx, float* max_logit, int32_t* candidates, float* scores,
                                 void* workspace, int64_t ws_bytes, void* stream);

/*
 * qmv_read_probe -- a measurement aid, not part of the method: reads `bytes`
 * of `data` once with 16-byte loads (grid-stride, the access pattern that
 * reads fastest on this GPU) and folds them into a word written to *out only
 * when it equals a fixed key.  Timing it beside qmv_gemv gives the achievable
 * HBM read rate on the same buffers.
 *   data  device, 16-byte aligned; bytes a multiple of 16 (0 = no-op).
 *   out   device, 1 uint32 (normally left untouched).
 */
int32_t qmv_read_probe(const void* data, int64_t bytes, uint32_t* out, void* stream);

/*
 * qmv_mfma_probe -- a measurement aid, not part of the method: every wave of
 * four workgroups per compute unit issues iters x 6 (kind 0:
 * v_mfma_i32_16x16x64_i8) or iters x 8 (kind 1: v_mfma_i32_32x32x32_i8)
 * independent int8 matrix instructions on register operands and folds the
 * results into a word written to *out only when it equals a fixed key.  *ops
 * (host) receives the int8 operations of the launch (2 per multiply-add);
 * ops / time is the matrix cores' rate on this machine, the yardstick of
 * qmv_gemm_prefill.
 *   1 <= iters <= 2^20.   EINVAL otherwise.
 */
int32_t qmv_mfma_probe(int32_t kind, int32_t iters, uint32_t* out, int64_t* ops /* host */, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
