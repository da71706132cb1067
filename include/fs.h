/*
 * fs.h -- C ABI of the per-rank state-sharding engine (FSDP / ZeRO-3 full
 * sharding) for AMD Instinct MI355X (gfx950).
 *
 * The engine plans the shard layout of one FSDP group, packs bf16 (or fp32)
 * parameters into it and unpacks them out of it (the all-gather copy-in and
 * copy-out), averages N logical ranks' gradient slices times grad_acc
 * micro-steps into this rank's fp32 shard (the local part of the
 * reduce-scatter), and runs the mixed-precision AdamW step on that shard.
 * All N ranks are logical: their buffers live on one GPU.
 *
 * Sources, cited by page title and section:
 *   "FSDP1 vs FSDP2" (blog.vllbc.top, visual reading)      -- [FvF]
 *   "Data parallelism, ZeRO and FSDP" (hs-black.github.io)  -- [DPZ]
 *   "ZeRO/FSDP explainer" (AI infra KB, M036)              -- [KB]
 *
 * Conventions for every call:
 *   - Device buffers are owned by the caller.  The library allocates no
 *     device memory and never synchronizes the device, except fs_plan_upload
 *     and fs_reshard_upload (set-up calls that wait for their own copies).
 *   - Pointers named "device" point to GPU memory; pointers named "host" to
 *     CPU memory.  Every device pointer must be aligned to its element size
 *     (2 bytes for bf16, 4 for fp32); 16-byte alignment is not required but
 *     is the fast path.
 *   - Work is issued asynchronously on `stream` (NULL = the null stream) as
 *     kernel launches only -- no copies, allocations or waits -- so the calls
 *     can be captured into a HIP graph.  A call launches one kernel, or
 *     several in sequence on `stream`: the reduces and the fused step one
 *     per pass of up to 32 terms, and over long buffers one per sub-range
 *     (32M elements for the reduce and the fused step, 16M for the bf16
 *     reduce dtype, 64M for AdamW), which measured faster than one launch
 *     over the whole buffer.
 *   - fs_plan_info, fs_plan_param, fs_plan_segments, fs_plan_upload,
 *     fs_plan_destroy, the fs_reshard_info/upload/destroy calls and
 *     fs_last_error are infrastructure around the method's steps (reading a
 *     plan back, placing its tables in device memory, reporting errors); no
 *     passage of the pages defines them.
 *   - Long launches of the reduces, AdamW, the unpack, the re-shard and the
 *     cast pack reserve LDS they never use, to limit how many of their workgroups share
 *     a CU (fewer concurrent HBM streams run faster); a kernel that another
 *     stream runs at the same time finds correspondingly less LDS on those
 *     CUs.
 *   - Inputs and outputs must not overlap, except the in-place AdamW state.
 *   - Errors are reported by return code (fs_status); the call then has
 *     launched nothing.  fs_last_error() describes the last failure of the
 *     calling thread.  No call aborts the process.
 */
#ifndef FS_H
#define FS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FS_OK = 0,
    FS_E_INVAL = -1,       /* bad argument: N < 1, NULL pointer, rank out of range, ... */
    FS_E_UNSUPPORTED = -2, /* a layout the method does not define (e.g. use_orig_params in FSDP2) */
    FS_E_DTYPE = -3,       /* unknown dtype */
    FS_E_OVERFLOW = -4,    /* a size does not fit in int64, or exceeds one launch's grid or the scratch array */
    FS_E_ALIGN = -5,       /* a pointer not aligned to its element size */
    FS_E_HIP = -6,         /* the HIP runtime reported an error */
    FS_E_NOMEM = -7        /* host memory for the plan could not be allocated */
} fs_status;

typedef enum { FS_BF16 = 0, FS_FP32 = 1 } fs_dtype;

typedef enum {
    FS_FSDP1_FLAT = 1,      /* FlatParameter: flatten, pad, chunk(N)   [FvF section 03] */
    FS_FSDP2_PER_PARAM = 2  /* each parameter chunked on dim 0          [FvF section 03] */
} fs_mode;

typedef struct fs_plan_s *fs_plan_t;       /* opaque; host memory owned by the library */
typedef struct fs_reshard_s *fs_reshard_t; /* opaque; host memory owned by the library */

/* Summary of a plan.  Counts are in elements of the plan's dtype. */
typedef struct {
    int32_t mode;            /* fs_mode */
    int32_t dtype;           /* fs_dtype */
    int32_t world;           /* N */
    int32_t use_orig_params; /* FSDP1 only */
    int32_t grad_acc;        /* micro-steps per optimizer step */
    int32_t n_params;
    int32_t elem_bytes;      /* 2 (bf16) or 4 (fp32) */
    int32_t bopt;            /* optimizer bytes per parameter the engine keeps: 12 (fp32 master, m, v) */
    int64_t total_numel;     /* sum of the parameters' element counts */
    int64_t flat_numel;      /* FSDP1: L, the flat length with alignment pads; FSDP2: 0 (there is no flat) */
    int64_t shard_numel;     /* elements per rank: c = ceil(L/N) (FSDP1) or T = sum ceil(d0_i/N)*row_i (FSDP2) */
    int64_t gathered_numel;  /* N * shard_numel: the all-gather output */
    int64_t align_pad;       /* FSDP1: alignment pad elements inside the flat (0 without use_orig_params) */
    int64_t tail_pad;        /* FSDP1: N*c - L (world / chunk pad); FSDP2: N*T - total_numel (per-parameter chunk pads) */
    int64_t n_segments;      /* copy segments of the lowered layout (see fs_segment_t) */
    int64_t workspace_bytes; /* device bytes fs_plan_upload needs */
    /* Per-rank resident bytes of params + grads + optimizer state
     * [FvF section 01 ledger; DPZ section 9; KB section 03]:
     * ideal  = P*(2b + bopt)/N, plus 4P/N for the fp32 gradient accumulator when grad_acc > 1;
     * padded = shard_numel*(2b + bopt), plus 4*shard_numel when grad_acc > 1.  b = elem_bytes. */
    double ledger_ideal_bytes;
    double ledger_padded_bytes;
    /* The same group under the other data-parallel schemes, per rank [FvF
     * section 01 and strategy ledger; DPZ section 9]; P = total_numel,
     * b = elem_bytes, bopt = 12, A = 4 B of fp32 gradient accumulator when
     * grad_acc > 1 (kept for the whole gradient under DDP and ZeRO-1, for the
     * own 1/N under ZeRO-2): */
    double ledger_ddp_bytes;          /* P(2b + bopt) (+ A*P) */
    double ledger_zero1_bytes;        /* 2Pb + P*bopt/N (+ A*P) */
    double ledger_zero2_bytes;        /* Pb + P(b + bopt)/N (+ A*P/N) */
    double peak_full_shard_bytes;     /* ideal ZeRO-3 bytes + P*b while the group is gathered */
    double comm_full_shard_bytes;     /* 3P(N-1)/N * b per step (AG forward, AG backward, RS) */
    double comm_shard_grad_op_bytes;  /* 2P(N-1)/N * b per step (one AG, one RS) */
} fs_plan_info_t;

/* One contiguous run of a parameter inside the gathered buffer.  Elements
 * [src_off, src_off+len) of parameter `param` occupy gathered elements
 * [dst_off, dst_off+len), which lie in rank `rank`'s shard.  Every gathered
 * element not covered by a segment is a pad (zero after fs_pack). */
typedef struct {
    int64_t dst_off;
    int64_t src_off;
    int64_t len;
    int32_t param;
    int32_t rank;
} fs_segment_t;

/* Layout of one parameter.  FSDP1: `start` is its flat offset, the FSDP2
 * fields are 0.  FSDP2: `start` is -1; chunk_rows = ceil(d0/N), row = product
 * of dims 1.., pre = offset of its chunk inside every rank's shard. */
typedef struct {
    int64_t numel;
    int64_t start;
    int64_t chunk_rows;
    int64_t row;
    int64_t pre;
} fs_param_layout_t;

typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    int32_t reserved; /* set to 0 */
    int64_t step;     /* t >= 1, the step being taken */
} fs_adamw_hparams_t;

/*
 * fs_plan -- plan the shard layout of one FSDP group (host only, no GPU call).
 *
 *   n_params        number of parameters in the group, >= 0.
 *   ndim   (host)   n_params dimension counts, each 0..8 (0 = a scalar).
 *   dims   (host)   the shapes, concatenated (sum of ndim entries), each >= 0.
 *   dtype           FS_BF16 or FS_FP32: the dtype of the parameters being
 *                   packed; it sets FSDP1's alignment unit a = 16/bytes.
 *   world           N >= 1 logical ranks.
 *   use_orig_params FSDP1 only (0 or 1); must be 0 for FSDP2.
 *   mode            FS_FSDP1_FLAT or FS_FSDP2_PER_PARAM.
 *   grad_acc        >= 1; recorded for the ledger.
 *   out    (host)   receives the plan; release it with fs_plan_destroy.
 *
 * FSDP1 [FvF section 03; Table 3]: parameters are flattened and concatenated
 * in order; with use_orig_params each parameter after the first starts on a
 * multiple of a = 16/bytes elements (at most a-1 pad elements before it);
 * every rank holds c = ceil(L/N) elements of the flat (world pad to a
 * multiple of N with use_orig_params; torch.chunk padded to chunks[0]
 * without).  FSDP2 [FvF section 03; Table 3]: parameter i is chunked on dim 0
 * into ceil(d0_i/N) rows per rank (torch.chunk semantics, trailing ranks may
 * get fewer or no rows, padded with zeros to the full chunk); the group's
 * shards are concatenated per rank, so the gathered buffer is [N][T].  A 0-d
 * parameter counts as shape [1].  All pads are zero.
 *
 * Errors: FS_E_INVAL (n_params < 0, world < 1, grad_acc < 1, ndim out of
 * range, negative dim, NULL pointers), FS_E_UNSUPPORTED (use_orig_params with
 * FSDP2), FS_E_DTYPE, FS_E_OVERFLOW (sizes beyond int64), FS_E_NOMEM.
 */
int fs_plan(int32_t n_params, const int32_t *ndim, const int64_t *dims,
            fs_dtype dtype, int32_t world, int32_t use_orig_params,
            fs_mode mode, int32_t grad_acc, fs_plan_t *out);

/* fs_plan_info -- fill *out (host) with the plan's summary. */
int fs_plan_info(fs_plan_t plan, fs_plan_info_t *out);

/* fs_plan_param -- layout of parameter i (0 <= i < n_params) into *out (host). */
int fs_plan_param(fs_plan_t plan, int32_t i, fs_param_layout_t *out);

/* fs_plan_segments -- copy up to `cap` segments, ordered by dst_off, into
 * out (host); *n (host) receives the total count.  out may be NULL when cap
 * is 0 (to query the count). */
int fs_plan_segments(fs_plan_t plan, fs_segment_t *out, int64_t cap, int64_t *n);

/*
 * fs_plan_upload -- copy the plan's device tables (segments and tile index)
 * into `workspace` (device memory of the current device, at least
 * info.workspace_bytes bytes, 16-byte aligned; FS_E_INVAL for host or
 * another device's memory) and bind that workspace to the plan for later
 * fs_pack/fs_unpack calls, which must then run with the same current device
 * (FS_E_INVAL otherwise).  Blocks until the copy has finished.  The workspace must stay
 * allocated and unmodified while the plan is used; calls that use one plan
 * on different streams at once are fine (the tables are read only).
 */
int fs_plan_upload(fs_plan_t plan, void *workspace, size_t bytes, hipStream_t stream);

/* fs_plan_destroy -- free the plan's host memory (NULL is a no-op). */
void fs_plan_destroy(fs_plan_t plan);

/*
 * fs_plan_twin -- a plan with the same element positions as `plan` and
 * elements of `dtype` (host only, not uploaded): every element of the twin's
 * gathered buffer and shards holds the same parameter element as in plan's.
 * It lays out state kept beside the parameters, element for element: the
 * fp32 master, m and v of a group's bf16 parameters [DPZ sections 1 and 9.1:
 * each rank updates its own slice of them].  FSDP1's use_orig_params
 * alignment follows the parameter dtype [FvF section 03], so a plan made
 * directly with FS_FP32 places those elements differently; the twin's pack,
 * unpack, re-shard and fs_load_local move the state where the bf16 plan's
 * elements are.  For FSDP2, and FSDP1 without use_orig_params, the twin
 * equals the plan made with `dtype`.
 *
 *   plan           any plan.
 *   dtype          FS_BF16 or FS_FP32: the twin's element type.
 *   out   (host)   receives the twin; release it with fs_plan_destroy.
 * info of the twin: the plan's, with dtype, elem_bytes, workspace_bytes and
 * the ledger fields (computed with the twin's element size) replaced.
 * Errors: FS_E_INVAL (NULL), FS_E_DTYPE, FS_E_OVERFLOW, FS_E_NOMEM.
 */
int fs_plan_twin(fs_plan_t plan, fs_dtype dtype, fs_plan_t *out);

/*
 * fs_pack -- the all-gather copy-in [FvF section 03: FSDP2 copies each
 * parameter's shard into the group's concatenated all-gather input; FSDP1's
 * flat is chunked].
 *
 *   params (device) array of n_params device pointers; parameter i holds
 *                   numel_i contiguous elements of the plan's dtype.
 *   out    (device) rank < 0: the whole gathered buffer, gathered_numel
 *                   elements (what the all-gather delivers to every rank);
 *                   rank r: rank r's shard only, shard_numel elements.
 *                   Every pad element is written as zero.
 *   rank            -1, or 0 <= rank < N.
 * Errors: FS_E_INVAL (plan not uploaded, rank out of range, NULL pointers),
 * FS_E_ALIGN (out not aligned to the element size), FS_E_OVERFLOW (more
 * tiles than one launch's grid holds), FS_E_HIP.
 */
int fs_pack(fs_plan_t plan, const void *const *params, void *out, int32_t rank,
            hipStream_t stream);

/*
 * fs_unpack -- the all-gather copy-out [FvF section 03: the flat metadata
 * (FSDP1) or the per-parameter chunks (FSDP2) view the gathered buffer back
 * as the original parameters].
 *
 *   gathered (device) gathered_numel elements laid out by the plan.
 *   params   (device) array of n_params device pointers, outputs of numel_i
 *                     elements each.  Pad elements of `gathered` are not read.
 * Errors: as fs_pack.
 */
int fs_unpack(fs_plan_t plan, const void *gathered, void *const *params,
              hipStream_t stream);

/*
 * fs_reshard_plan -- plan moving one group's gathered buffer from plan `src`
 * (N ranks) to plan `dst` (N' ranks; FSDP1 or FSDP2 on either side), host
 * only.  Every parameter element goes from its place in src's gathered
 * buffer to its place in dst's; dst's pads are written as zero.  Sources:
 * [FvF] memory and engineering section (FSDP2's shards are the sharded state
 * dict; FSDP1 must unshard to save one); the FSDP tutorial page (m.xxqk.cn),
 * section 3.3 (sharded checkpoints do not carry over between card counts:
 * they must be re-sharded).  With fp32 plans the same call re-shards fp32
 * optimizer state (master, m, v).
 * Errors: FS_E_INVAL (NULL, different parameter lists), FS_E_DTYPE
 * (different element sizes), FS_E_OVERFLOW, FS_E_NOMEM.
 */
int fs_reshard_plan(fs_plan_t src, fs_plan_t dst, fs_reshard_t *out);

/* fs_reshard_info -- device workspace bytes and copy-segment count (either
 * output may be NULL). */
int fs_reshard_info(fs_reshard_t r, int64_t *workspace_bytes, int64_t *n_segments);

/* fs_reshard_upload -- as fs_plan_upload, for a reshard plan. */
int fs_reshard_upload(fs_reshard_t r, void *workspace, size_t bytes, hipStream_t stream);

/*
 * fs_reshard -- dst_gathered (device, dst's gathered_numel elements) <- the
 * re-sharded src_gathered (device, src's gathered_numel elements).  Pads of
 * src are not read.  Errors: FS_E_INVAL (not uploaded, NULL, overlapping
 * buffers), FS_E_ALIGN, FS_E_OVERFLOW (more tiles than one launch's grid
 * holds), FS_E_HIP.
 */
int fs_reshard(fs_reshard_t r, const void *src_gathered, void *dst_gathered, hipStream_t stream);

/* fs_reshard_destroy -- free a reshard plan (NULL is a no-op). */
void fs_reshard_destroy(fs_reshard_t r);

/*
 * fs_load_local -- import rank `rank`'s part of a sharded state dict into its
 * shard buffer [FvF, memory and engineering section: FSDP2's shards are the
 * sharded state dict, saved and loaded per rank without communication; the
 * FSDP tutorial page (m.xxqk.cn), section 3.3: sharded checkpoints are
 * loaded rank by rank].  The inverse of viewing a shard's local pieces: with
 * the plan's fp32 twin (fs_plan_twin) the same call restores master, m or v.
 *
 *   rank            0 <= rank < N.
 *   pieces (device) array of n_params device pointers; entry i points to the
 *                   rank's local piece of parameter i: the run of its
 *                   elements that fs_plan_segments lists on this rank (FSDP2:
 *                   the rank's torch.chunk dim-0 chunk; FSDP1: the flattened
 *                   parameter's elements inside the rank's flat shard), in
 *                   element order, contiguous, aligned to the element size.
 *                   Entries of parameters the rank holds none of are not read.
 *   shard  (device) shard_numel elements of the plan's dtype; every element
 *                   that no piece covers (a pad) is written as zero.
 * Same kernels and tables as fs_pack with rank = r.
 * Errors: FS_E_INVAL (plan not uploaded, rank out of range, NULL pointers),
 * FS_E_ALIGN (shard not aligned to the element size), FS_E_OVERFLOW, FS_E_HIP.
 */
int fs_load_local(fs_plan_t plan, int32_t rank, const void *const *pieces, void *shard,
                  hipStream_t stream);

/*
 * fs_reduce_shard -- this rank's averaged fp32 gradient shard [DPZ section
 * 2.1: sum the ranks' gradients, then divide by N; DPZ sections 1 and 9.2:
 * fp32 accumulation over micro-steps on the own shard; DPZ section 5: the
 * 1/grad_acc factor is already in each micro-step's loss].
 *
 *   n              elements of the shard (>= 0).
 *   world          N >= 1.
 *   grad_acc       A >= 1.
 *   slices (host)  array of A*N device pointers; slices[j*N + k] is logical
 *                  rank k's bf16 gradient at micro-step j, restricted to this
 *                  rank's shard (n elements).
 *   out   (device) n fp32 values: for each element the A*N terms are added in
 *                  fp32 one by one in slice order, starting from the first
 *                  term, and the sum is divided once by N (IEEE division).
 *                  The result is bit-exact and deterministic.
 * Errors: FS_E_INVAL (n < 0, world < 1, grad_acc < 1, NULL pointers, out
 * overlapping a slice), FS_E_ALIGN, FS_E_OVERFLOW, FS_E_HIP.
 */
int fs_reduce_shard(int64_t n, int32_t world, int32_t grad_acc,
                    const uint16_t *const *slices, float *out,
                    hipStream_t stream);

/*
 * fs_reduce_shard_ex -- fs_reduce_shard with a choice of reduce dtype [FvF
 * mixed-precision section: reduce_dtype sets the precision of the gradient
 * reduction; DPZ section 9.2: the own fp32 shard accumulates the bf16
 * gradients the reduce-scatter delivers].
 *
 *   reduce_dtype   FS_FP32: identical to fs_reduce_shard.
 *                  FS_BF16: for each micro-step j, the N terms are added in
 *                  fp32 in rank order and divided once by N, the quotient is
 *                  rounded to bf16 (nearest even) -- what a bf16
 *                  reduce-scatter delivers -- and the micro-step values are
 *                  accumulated in fp32 starting from the first.  Needs
 *                  world <= 32.  Bit-exact and deterministic.
 *   other arguments as fs_reduce_shard.
 * Errors: those of fs_reduce_shard; FS_E_DTYPE for another reduce_dtype;
 * FS_E_UNSUPPORTED for world > 32 with FS_BF16.
 */
int fs_reduce_shard_ex(int64_t n, int32_t world, int32_t grad_acc,
                       fs_dtype reduce_dtype, const uint16_t *const *slices,
                       float *out, hipStream_t stream);

/*
 * fs_pack_cast -- the all-gather copy-in with the parameter-dtype cast at
 * the all-gather boundary [FvF mixed-precision section: the all-gather casts
 * the parameters to param_dtype, the optimizer keeps the original dtype].
 *
 *   plan           a plan made with dtype FS_BF16 (the param_dtype; FSDP1
 *                  alignment follows it), uploaded.
 *   params (device) array of n_params device pointers to parameters stored
 *                  as `param_dtype`.
 *   param_dtype    FS_FP32: every element is written as the
 *                  round-to-nearest-even bf16 of its value (NaN stays a
 *                  quiet NaN); FS_BF16: identical to fs_pack.
 *   out, rank      as fs_pack (bf16 output).
 * Errors: those of fs_pack; FS_E_DTYPE; FS_E_UNSUPPORTED for any other
 * dtype pair.
 */
int fs_pack_cast(fs_plan_t plan, const void *const *params, fs_dtype param_dtype,
                 void *out, int32_t rank, hipStream_t stream);

/*
 * fs_adamw_step -- one mixed-precision AdamW step over the shard [DPZ
 * section 1: moments first, then the parameter; DPZ section 9.1: update the
 * own fp32 parameters, then turn them into bf16; KB section 04].
 *
 *   n                     elements (>= 0).
 *   master, exp_avg, exp_avg_sq (device, fp32, in place): theta, m, v.
 *   grad       (device)   n gradients of grad_dtype (FS_FP32 or FS_BF16).
 *   param_bf16 (device)   n bf16 outputs (the rank's slice of the next
 *                         all-gather input), or NULL to skip.
 *   hp         (host)     hyperparameters; step t >= 1.
 * Update, evaluated in double from the fp32 values and rounded to fp32 only
 * when stored:
 *   m' = b1*m + (1-b1)*g;  v' = b2*v + (1-b2)*g*g;
 *   theta' = theta*(1 - lr*wd) - lr*(m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps);
 *   param_bf16 = round-to-nearest-even bf16 of the stored fp32 theta'.
 * Errors: FS_E_INVAL (n < 0, NULL pointers, step < 1, betas outside [0,1),
 * two of master, exp_avg, exp_avg_sq, grad and param_bf16 sharing memory),
 * FS_E_DTYPE, FS_E_ALIGN, FS_E_OVERFLOW (n beyond one launch), FS_E_HIP.
 */
int fs_adamw_step(int64_t n, float *master, float *exp_avg, float *exp_avg_sq,
                  const void *grad, fs_dtype grad_dtype, uint16_t *param_bf16,
                  const fs_adamw_hparams_t *hp, hipStream_t stream);

/*
 * fs_reduce_adamw_step -- the reduce and the AdamW step fused into one pass
 * over the shard [DPZ section 9.2: the own 1/N fp32 gradient feeds the update
 * of the own fp32 parameters; KB section 04: optimizer step over the local
 * shard].  The averaged gradient is not written to memory unless asked for.
 *
 *   n, world, grad_acc, slices: as fs_reduce_shard.
 *   master, exp_avg, exp_avg_sq, param_bf16, hp: as fs_adamw_step (fp32
 *                  gradient).
 *   grad_out (device, fp32, n, nullable): also receives the averaged
 *                  gradient.  Required when world*grad_acc > 32 (it holds
 *                  the partial sums between passes).
 * Results: theta, m, v and param_bf16 are bit-identical to fs_reduce_shard
 * followed by fs_adamw_step(grad_dtype = FS_FP32); grad_out to
 * fs_reduce_shard's output.  HBM traffic per element: 2*A*N + 26 bytes
 * (+4 with grad_out) instead of 2*A*N + 34.
 * Errors: those of fs_reduce_shard and fs_adamw_step; FS_E_INVAL also for an
 * output overlapping a slice or another output, or more than 32 terms
 * without grad_out.
 */
int fs_reduce_adamw_step(int64_t n, int32_t world, int32_t grad_acc,
                         const uint16_t *const *slices, float *master,
                         float *exp_avg, float *exp_avg_sq, uint16_t *param_bf16,
                         float *grad_out, const fs_adamw_hparams_t *hp,
                         hipStream_t stream);

/*
 * fs_reduce_adamw_step_noalloc -- fs_reduce_adamw_step with grad_out = NULL
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): with more
 * than 32 terms the partial sums that fs_reduce_adamw_step keeps in the
 * caller's grad_out go to a scratch array the library holds on each GPU
 * instead (FS_NOALLOC_MAX_NUMEL fp32 elements, 64 MiB, held until the process
 * ends).  Allocates and frees nothing.  Same arguments, results (bit for bit)
 * and errors as fs_reduce_adamw_step, plus FS_E_OVERFLOW when more than 32
 * terms meet n > FS_NOALLOC_MAX_NUMEL.  Calls on one GPU share the scratch
 * array: calls that overlap in time on one GPU race.
 */
#define FS_NOALLOC_MAX_NUMEL 16777216
int fs_reduce_adamw_step_noalloc(int64_t n, int32_t world, int32_t grad_acc,
                                 const uint16_t *const *slices, float *master,
                                 float *exp_avg, float *exp_avg_sq, uint16_t *param_bf16,
                                 const fs_adamw_hparams_t *hp, hipStream_t stream);

/* fs_last_error -- message for the calling thread's last failed call
 * (empty string if none).  The pointer stays valid until the next call. */
const char *fs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FS_H */
