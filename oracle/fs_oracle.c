/*
 * fs_oracle.c -- CPU oracle for the per-rank state-sharding engine.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this file's library.  It
 * shares no code, header, table or helper with the HIP library: the two are
 * written independently so that one can check the other.
 *
 * Everything here is a plain, slow, element-by-element loop that follows the
 * pages' definitions in their own order.  Sources (page title, then section):
 *
 *   "FSDP1 vs FSDP2" (visual reading, blog.vllbc.top)
 *        -- section 03 (the two representations): FlatParameter alignment
 *           padding, world-size padding, flatten().chunk(N); FSDP2 dim-0
 *           ceil(s_i/N) chunks and group concatenation.
 *        -- Table 3 (worked example: parameters of 3 and 5 elements, N=4).
 *   "Data parallelism, ZeRO and FSDP" (hs-black.github.io)
 *        -- section 1 (16 B/param mixed-precision recipe; fp32 gradient
 *           accumulation; Adam updates the moments first, then the params),
 *        -- section 2.1 (gradients are summed, then divided by N_d),
 *        -- section 5 (the 1/grad_acc factor sits in the loss),
 *        -- section 9.1/9.2 (rank updates its own fp32 slice, then casts it
 *           to bf16; fp32 accumulation of the reduce-scatter output).
 *
 * Floating-point environment: build with -ffp-contract=off and without
 * -ffast-math, so each C operator below is one IEEE operation with
 * round-to-nearest-even and denormals preserved.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes):
 *   - every pad element is bit-zero;
 *   - FSDP1 alignment is measured in elements from the flat start and applies
 *     to every parameter after the first, empty ones included; there is no
 *     trailing alignment after the last parameter;
 *   - FSDP1 shard length is ceil(L/N) in both use_orig_params modes (world
 *     padding to a multiple of N, or torch.chunk padded to chunks[0]);
 *   - FSDP2 shards dim 0 with torch.chunk semantics, a 0-d parameter counts
 *     as shape [1], and the group's gathered buffer is rank-major [N][T];
 *   - the reduce sums the A*N terms in the fixed order (micro-step outer,
 *     rank inner), starting from the first term, then divides once by N;
 *   - AdamW is computed in double from the fp32 inputs and rounded to fp32
 *     only when stored; the bf16 copy is the RNE rounding of the stored fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * The same source also builds with -fopenmp (liboracle_omp.so, used only to
 * time the oracle on every host core): ELEMENT_LOOP marks loops whose
 * iterations write disjoint outputs and share no accumulator, so running them
 * on several threads changes no arithmetic and no result.
 */
#ifdef _OPENMP
#define ELEMENT_LOOP _Pragma("omp parallel for schedule(static)")
#else
#define ELEMENT_LOOP
#endif

/* Threads the element loops use (1 in the single-threaded build). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

uint16_t oracle_bf16_round(float f); /* defined with the number formats below */

/* ------------------------------------------------------------------------ */
/* Layouts                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * FSDP1 FlatParameter layout ["FSDP1 vs FSDP2", section 03 and Table 3].
 * Parameters are flattened and concatenated in order.  With use_orig_params
 * the start of every parameter after the first is padded up to a multiple of
 * a = 16 / elem_bytes elements (16-byte boundary, at most a-1 pad elements).
 * The flat of length L is then cut into N equal chunks of c = ceil(L/N)
 * elements: with use_orig_params by padding the whole flat to a multiple of N,
 * without it by torch.chunk(N) and padding every chunk to chunks[0].numel().
 *
 * Outputs: start[i] (flat offset of parameter i), *flat_len (L, before the
 * world/chunk pad) and *shard (c).  Returns 0, or -1 on bad arguments.
 */
int oracle_fsdp1_layout(int32_t n_params, const int64_t *numel,
                        int32_t elem_bytes, int32_t world,
                        int32_t use_orig_params, int64_t *start,
                        int64_t *flat_len, int64_t *shard)
{
    if (n_params < 0 || world < 1 || (elem_bytes != 2 && elem_bytes != 4))
        return -1;
    int64_t a = use_orig_params ? (16 / elem_bytes) : 1;
    int64_t off = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        if (numel[i] < 0)
            return -1;
        if (i > 0) {
            int64_t pad = (a - off % a) % a; /* pad *before* parameter i */
            off += pad;
        }
        start[i] = off;
        off += numel[i];
    }
    *flat_len = off;
    /* c = ceil(L / N): the chunk length every rank stores. */
    *shard = (off + world - 1) / world;
    return 0;
}

/*
 * FSDP2 per-parameter layout ["FSDP1 vs FSDP2", section 03: each parameter is chunked on
 * dim 0 into ceil(s_i/N) rows per rank, padding belongs to that parameter
 * alone, an empty parameter gets empty chunks; the group's shards are
 * concatenated into one all-gather input].
 *
 * Inputs: d0[i] (dim-0 extent, 1 for a 0-d parameter) and row[i] (product of
 * the remaining dims).  Outputs: chunk_rows[i] = ceil(d0/N), pre[i] (offset of
 * parameter i's chunk inside one rank's shard) and *shard (T = sum of
 * chunk_rows[i]*row[i]).  Returns 0, or -1 on bad arguments.
 */
int oracle_fsdp2_layout(int32_t n_params, const int64_t *d0,
                        const int64_t *row, int32_t world,
                        int64_t *chunk_rows, int64_t *pre, int64_t *shard)
{
    if (n_params < 0 || world < 1)
        return -1;
    int64_t t = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        if (d0[i] < 0 || row[i] < 0)
            return -1;
        chunk_rows[i] = (d0[i] + world - 1) / world;
        pre[i] = t;
        t += chunk_rows[i] * row[i];
    }
    *shard = t;
    return 0;
}

/*
 * Gathered-buffer index of element e of parameter i.  The gathered buffer is
 * the all-gather output: N shards of `shard` elements, rank-major.
 *   FSDP1: flat index start[i] + e (the flat *is* the gathered buffer).
 *   FSDP2: element e lies in row e / row[i]; that row belongs to rank
 *          r = row_index / chunk_rows[i] at local row row_index - r*chunk_rows[i]
 *          of parameter i's chunk, which begins at r*T + pre[i].
 */
static int64_t fsdp1_index(const int64_t *start, int32_t i, int64_t e)
{
    return start[i] + e;
}

static int64_t fsdp2_index(const int64_t *chunk_rows, const int64_t *row,
                           const int64_t *pre, int64_t shard, int32_t i,
                           int64_t e)
{
    int64_t rw = row[i];
    int64_t row_index = e / rw;
    int64_t col = e % rw;
    int64_t r = row_index / chunk_rows[i];
    int64_t local_row = row_index - r * chunk_rows[i];
    return r * shard + pre[i] + local_row * rw + col;
}

/*
 * Layout descriptor passed in from Python.  mode 1 = FSDP1 (uses start),
 * mode 2 = FSDP2 (uses chunk_rows, row, pre).  numel[i] is parameter i's
 * element count in both modes.
 */
typedef struct {
    int32_t mode;
    int32_t n_params;
    int32_t world;
    int32_t elem_bytes;
    int64_t shard;
    const int64_t *numel;
    const int64_t *start;
    const int64_t *chunk_rows;
    const int64_t *row;
    const int64_t *pre;
} oracle_layout;

static int64_t gathered_index(const oracle_layout *L, int32_t i, int64_t e)
{
    if (L->mode == 1)
        return fsdp1_index(L->start, i, e);
    return fsdp2_index(L->chunk_rows, L->row, L->pre, L->shard, i, e);
}

/* Index table for tests: out[k] for k over the parameters' elements in order
 * (parameter 0's elements, then parameter 1's, ...). */
void oracle_index_map(const oracle_layout *L, int64_t *out)
{
    int64_t k = 0;
    for (int32_t i = 0; i < L->n_params; ++i)
        for (int64_t e = 0; e < L->numel[i]; ++e)
            out[k++] = gathered_index(L, i, e);
}

/* Gathered index of sampled elements: out[k] = index of element elem[k] of
 * parameter param[k]. */
void oracle_index_at(const oracle_layout *L, int64_t n, const int32_t *param,
                     const int64_t *elem, int64_t *out)
{
    for (int64_t k = 0; k < n; ++k)
        out[k] = gathered_index(L, param[k], elem[k]);
}

/*
 * All-gather copy-in ["FSDP1 vs FSDP2", section 03, and the FSDP2 group
 * concatenation]:
 * start from a zero-filled output and copy every parameter element to its
 * place.  rank < 0 writes the whole gathered buffer (N * shard elements);
 * rank r writes only shard r, into an output of `shard` elements.
 * Elements are copied as raw bytes, so NaN payloads survive.
 */
void oracle_pack(const oracle_layout *L, const void *const *params, void *out,
                 int32_t rank)
{
    const int64_t w = L->elem_bytes;
    int64_t lo = 0, hi = (int64_t)L->world * L->shard;
    if (rank >= 0) {
        lo = (int64_t)rank * L->shard;
        hi = lo + L->shard;
    }
    memset(out, 0, (size_t)((hi - lo) * w));
    for (int32_t i = 0; i < L->n_params; ++i) {
        const unsigned char *p = (const unsigned char *)params[i];
        ELEMENT_LOOP
        for (int64_t e = 0; e < L->numel[i]; ++e) {
            int64_t x = gathered_index(L, i, e);
            if (x >= lo && x < hi)
                memcpy((unsigned char *)out + (x - lo) * w, p + e * w,
                       (size_t)w);
        }
    }
}

/*
 * Copy-in with the parameter-dtype cast at the all-gather boundary ["FSDP1 vs
 * FSDP2", section on mixed precision: the all-gather casts the parameters to
 * param_dtype while the optimizer keeps the original dtype].  The layout is
 * the bf16 one (elem_bytes 2); the parameters are fp32 and every element is
 * written as the round-to-nearest-even bf16 of its value; pads are zero.
 */
void oracle_pack_cast(const oracle_layout *L, const float *const *params,
                      uint16_t *out, int32_t rank)
{
    int64_t lo = 0, hi = (int64_t)L->world * L->shard;
    if (rank >= 0) {
        lo = (int64_t)rank * L->shard;
        hi = lo + L->shard;
    }
    for (int64_t x = 0; x < hi - lo; ++x)
        out[x] = 0;
    for (int32_t i = 0; i < L->n_params; ++i)
        for (int64_t e = 0; e < L->numel[i]; ++e) {
            int64_t x = gathered_index(L, i, e);
            if (x >= lo && x < hi)
                out[x - lo] = oracle_bf16_round(params[i][e]);
        }
}

/*
 * All-gather copy-out: read every parameter element back from its place in
 * the gathered buffer (the inverse of oracle_pack with rank < 0).  Pad
 * elements are never read.
 */
void oracle_unpack(const oracle_layout *L, const void *gathered,
                   void *const *params)
{
    const int64_t w = L->elem_bytes;
    for (int32_t i = 0; i < L->n_params; ++i) {
        unsigned char *p = (unsigned char *)params[i];
        ELEMENT_LOOP
        for (int64_t e = 0; e < L->numel[i]; ++e) {
            int64_t x = gathered_index(L, i, e);
            memcpy(p + e * w, (const unsigned char *)gathered + x * w,
                   (size_t)w);
        }
    }
}

/*
 * Re-shard one group's gathered buffer from layout Ls (N ranks) to layout Ld
 * (N' ranks, either mode) ["FSDP1 vs FSDP2", memory and engineering
 * section: FSDP2's shards are the sharded state dict; the FSDP tutorial page
 * (m.xxqk.cn), section 3.3: sharded checkpoints must be re-sharded to load at
 * another card count]: start from a zero-filled output and copy every
 * parameter element from its place under Ls to its place under Ld.
 */
void oracle_reshard(const oracle_layout *Ls, const oracle_layout *Ld,
                    const void *src, void *dst)
{
    const int64_t w = Ld->elem_bytes;
    memset(dst, 0, (size_t)((int64_t)Ld->world * Ld->shard * w));
    for (int32_t i = 0; i < Ld->n_params; ++i)
        for (int64_t e = 0; e < Ld->numel[i]; ++e)
            memcpy((unsigned char *)dst + gathered_index(Ld, i, e) * w,
                   (const unsigned char *)src + gathered_index(Ls, i, e) * w,
                   (size_t)w);
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * binary32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quiet
 * bit set, sign and upper payload kept); infinities and overflow follow the
 * usual rounding (values that round past the largest bf16 become inf).
 */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;       /* the bits that survive */
    uint32_t dropped = u & 0xffffu; /* the 16 bits cut off */
    if (dropped > 0x8000u || (dropped == 0x8000u && (keep & 1u)))
        keep += 1; /* a carry into the exponent is the correct rounding */
    return (uint16_t)keep;
}

void oracle_bf16_round_array(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t e = 0; e < n; ++e)
        out[e] = oracle_bf16_round(in[e]);
}

/* ------------------------------------------------------------------------ */
/* Reduce-scatter local averaging                                            */
/* ------------------------------------------------------------------------ */

/*
 * This rank's averaged gradient shard ["Data parallelism, ZeRO and FSDP",
 * section 2.1: sum the ranks' gradients, then divide by N_d; sections 1 and
 * 9.2: accumulate in fp32 over the micro-steps on the own 1/N_d; section 5:
 * the 1/grad_acc factor
 * is already in each micro-step's loss, so the engine only sums over them].
 *
 * slices[j*world + k] is rank k's gradient at micro-step j, restricted to
 * this rank's shard: n bf16 values.  For every element the A*N terms are
 * added one by one in fp32 in that order, starting from the first term, and
 * the sum is divided once by N (one IEEE division).
 */
void oracle_reduce(int64_t n, int32_t world, int32_t grad_acc,
                   const uint16_t *const *slices, float *out)
{
    const int32_t terms = world * grad_acc;
    ELEMENT_LOOP
    for (int64_t e = 0; e < n; ++e) {
        float acc = bf16_to_float(slices[0][e]);
        for (int32_t t = 1; t < terms; ++t) {
            float g = bf16_to_float(slices[t][e]);
            acc = acc + g;
        }
        out[e] = acc / (float)world;
    }
}

/*
 * The same averaging with a bf16 reduce dtype ["FSDP1 vs FSDP2", section on
 * mixed precision: reduce_dtype sets the precision of the gradient reduction;
 * "Data parallelism, ZeRO and FSDP", section 9.2: the own 1/N_d fp32 buffer accumulates the bf16 gradients the
 * reduce-scatter delivers].  Per micro-step j the N ranks' terms are added in
 * fp32 in rank order and divided once by N -- the reduce-scatter's average --
 * and that average is delivered as bf16 (round to nearest even); the
 * micro-step averages are then accumulated in fp32, starting from the first.
 */
void oracle_reduce_bf16rs(int64_t n, int32_t world, int32_t grad_acc,
                          const uint16_t *const *slices, float *out)
{
    ELEMENT_LOOP
    for (int64_t e = 0; e < n; ++e) {
        float acc = 0.0f;
        for (int32_t j = 0; j < grad_acc; ++j) {
            float s = bf16_to_float(slices[j * world][e]);
            for (int32_t k = 1; k < world; ++k)
                s = s + bf16_to_float(slices[j * world + k][e]);
            float delivered = bf16_to_float(oracle_bf16_round(s / (float)world));
            acc = (j == 0) ? delivered : acc + delivered;
        }
        out[e] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Mixed-precision AdamW on the shard                                        */
/* ------------------------------------------------------------------------ */

/*
 * One AdamW step over this rank's shard ["Data parallelism, ZeRO and FSDP",
 * section 1: Adam updates the first and second moments, then the parameter;
 * section 9.1: the rank updates its own fp32 parameters and then turns them
 * into bf16; "ZeRO/FSDP explainer", section 04: optimizer_step over the local sharded states, AdamW built on
 * the sharded parameters].
 *
 * Update (decoupled weight decay scaled by lr), all in double:
 *   m'     = beta1*m + (1-beta1)*g
 *   v'     = beta2*v + (1-beta2)*g*g
 *   m_hat  = m' / (1 - beta1^t)
 *   v_hat  = v' / (1 - beta2^t)
 *   theta' = theta*(1 - lr*wd) - lr * m_hat / (sqrt(v_hat) + eps)
 * theta', m', v' are rounded to fp32 when stored; param_bf16 (if not NULL)
 * receives the RNE bf16 rounding of the stored fp32 theta'.
 *
 * grad_is_bf16 selects the gradient format (bf16 bits or fp32).
 */
void oracle_adamw(int64_t n, float *master, float *exp_avg, float *exp_avg_sq,
                  const void *grad, int32_t grad_is_bf16, uint16_t *param_bf16,
                  float lr, float beta1, float beta2, float eps,
                  float weight_decay, int64_t step)
{
    const double b1 = beta1, b2 = beta2;
    const double bias1 = 1.0 - pow(b1, (double)step);
    const double bias2 = 1.0 - pow(b2, (double)step);
    const double lr_d = lr, eps_d = eps, wd_d = weight_decay;
    ELEMENT_LOOP
    for (int64_t e = 0; e < n; ++e) {
        double g = grad_is_bf16 ? (double)bf16_to_float(((const uint16_t *)grad)[e])
                                : (double)((const float *)grad)[e];
        double theta = master[e];
        double m = exp_avg[e];
        double v = exp_avg_sq[e];

        double m_new = b1 * m + (1.0 - b1) * g;
        double v_new = b2 * v + (1.0 - b2) * g * g;
        double m_hat = m_new / bias1;
        double v_hat = v_new / bias2;
        double theta_new = theta * (1.0 - lr_d * wd_d) -
                           lr_d * m_hat / (sqrt(v_hat) + eps_d);

        master[e] = (float)theta_new;
        exp_avg[e] = (float)m_new;
        exp_avg_sq[e] = (float)v_new;
        if (param_bf16)
            param_bf16[e] = oracle_bf16_round(master[e]);
    }
}
