// fs_plan.cpp -- host planner: shard layouts, segment lowering, tile index.
//
// Layout rules (page "FSDP1 vs FSDP2", section 03 and Table 3):
//   FSDP1 FlatParameter: parameters flattened and concatenated in order; with
//     use_orig_params every parameter after the first starts on a multiple of
//     a = 16/bytes(dtype) elements (at most a-1 pad elements); the flat of
//     length L is split into N equal shards of c = ceil(L/N) elements (world
//     pad to a multiple of N with use_orig_params, chunk(N) padded to
//     chunks[0] without -- the same c).
//   FSDP2 per-parameter: parameter i is chunked on dim 0, ceil(d0_i/N) rows
//     per rank with torch.chunk semantics (later ranks may get fewer or no
//     rows), each chunk padded to the full row count; every rank's shard
//     concatenates its chunks in parameter order, and the group's all-gather
//     output is rank-major [N][T].
// Memory ledger ("FSDP1 vs FSDP2" section 01; "Data parallelism, ZeRO and
// FSDP" section 9; "ZeRO/FSDP explainer" section 03): per-rank bytes
// P(2b + bopt)/N, plus 4P/N for an fp32 gradient accumulator.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "fs_plan_impl.h"

using fsi::Segment;
using fsi::Tile;

namespace fsi {

static thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

}  // namespace fsi

extern "C" const char *fs_last_error(void) { return fsi::g_err; }

namespace {

constexpr int64_t kMaxI64 = INT64_MAX;

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_add_overflow(a, b, out); }

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

}  // namespace

// Cut the grid of blocks [lo + k*vec, lo + (k+1)*vec) covering [lo, hi) into
// tiles of at most tile_blocks blocks that overlap at most kTileSegs segments.
// `segs` is sorted by vx and non-overlapping.
void fsi::build_tiles(const std::vector<Segment> &segs, int64_t lo, int64_t hi, int vec, int tile_blocks,
                      std::vector<Tile> &out) {
    if (hi <= lo) return;
    const int64_t nblocks = ceil_div(hi - lo, vec);
    const int64_t nseg = (int64_t)segs.size();
    // first segment whose end lies beyond x
    auto first_ending_after = [&](int64_t from, int64_t x) {
        int64_t a = from, b = nseg;
        while (a < b) {
            int64_t m = (a + b) / 2;
            if (segs[m].vx + segs[m].len <= x) a = m + 1; else b = m;
        }
        return a;
    };
    // first segment starting at or beyond x
    auto first_starting_at = [&](int64_t from, int64_t x) {
        int64_t a = from, b = nseg;
        while (a < b) {
            int64_t m = (a + b) / 2;
            if (segs[m].vx < x) a = m + 1; else b = m;
        }
        return a;
    };
    int64_t s0 = first_ending_after(0, lo);
    int64_t b0 = 0;
    while (b0 < nblocks) {
        int64_t x0 = lo + b0 * vec;
        s0 = first_ending_after(s0, x0);
        int64_t b1 = std::min<int64_t>(nblocks, b0 + tile_blocks);
        if (s0 + fsi::kTileSegs < nseg) {
            // keep the (kTileSegs+1)-th segment out of this tile
            int64_t cut = (segs[s0 + fsi::kTileSegs].vx - lo) / vec;
            if (cut < b1) b1 = cut;
        }
        int64_t x1 = std::min(hi, lo + b1 * vec);
        int64_t s1 = first_starting_at(s0, x1);
        Tile t;
        t.x_begin = x0;
        t.nblk = (int32_t)(b1 - b0);
        t.seg_lo = (int32_t)s0;
        t.nseg = (int32_t)(s1 - s0);
        t.run_buf = -1;
        t.run_src = 0;
        t.run_dst = 0;
        const int64_t x_full = lo + b1 * vec;   // end of the tile's last block
        if (t.nseg == 1 && segs[s0].vx <= x0 && segs[s0].vx + segs[s0].len >= x_full) {
            t.run_buf = segs[s0].buf;
            t.run_src = segs[s0].src_off + (x0 - segs[s0].vx);
        }
        out.push_back(t);
        b0 = b1;
    }
}

namespace {

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

// The tables that depend on the element size: the unpack view (parameters
// end to end on 16-byte boundaries), the tile grids, the workspace layout
// and the size-dependent summary fields.  p->params, p->pack_segs and the
// position fields of p->info are set; bad_alloc propagates to the caller.
static void finalize_plan(fs_plan_s *p, fs_dtype dtype) {
    const int64_t eb = dtype == FS_BF16 ? 2 : 4;
    const int vec = (int)(16 / eb);
    p->vec = vec;
    const int32_t n_params = p->info.n_params, world = p->info.world;
    const int64_t shard = p->info.shard_numel, gathered = p->info.gathered_numel;
    const std::vector<Segment> &ps = p->pack_segs;
    p->bufinfo.clear();
    p->unpack_segs.clear();
    p->pack_tiles_all.clear();
    p->pack_tiles_rank.clear();
    p->rank_tile_off.clear();
    p->unpack_tiles.clear();
    p->ws = fsi::WorkspaceLayout{};
    // ---- unpack view: parameters laid end to end on 16-byte boundaries
    p->bufinfo.resize(n_params);
    int64_t vb = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        p->bufinfo[i].vbase = vb;
        p->bufinfo[i].numel = p->params[i].numel;
        vb += align_up(p->params[i].numel, vec);
    }
    p->unpack_segs.reserve(ps.size());
    for (const Segment &s : ps)
        p->unpack_segs.push_back(Segment{p->bufinfo[s.buf].vbase + s.src_off, s.vx, s.len, s.buf, s.rank});
    std::sort(p->unpack_segs.begin(), p->unpack_segs.end(),
              [](const Segment &a, const Segment &b) { return a.vx < b.vx; });

    // ---- tiles
    // Per-rank grids (anchored at each shard's start).  When every shard
    // starts on a 16-byte block of the gathered buffer, their concatenation
    // is also a grid anchored at 0 and serves the all-ranks pack: one table.
    p->rank_tile_off.push_back(0);
    p->pack_tiles_rank.reserve((size_t)world * (size_t)(ceil_div(ceil_div(shard, vec), fsi::kCopyTileBlocks) + 1));
    for (int32_t r = 0; r < world; ++r) {
        fsi::build_tiles(ps, (int64_t)r * shard, (int64_t)(r + 1) * shard, vec, fsi::kCopyTileBlocks,
                         p->pack_tiles_rank);
        p->rank_tile_off.push_back((int64_t)p->pack_tiles_rank.size());
    }
    const bool shared_grid = world == 1 || shard % vec == 0;
    if (!shared_grid) {
        p->pack_tiles_all.reserve((size_t)(ceil_div(ceil_div(gathered, vec), fsi::kCopyTileBlocks) + 1));
        fsi::build_tiles(ps, 0, gathered, vec, fsi::kCopyTileBlocks, p->pack_tiles_all);
    }
    p->unpack_tiles.reserve((size_t)(ceil_div(ceil_div(vb, vec), fsi::kCopyTileBlocks) + 1));
    fsi::build_tiles(p->unpack_segs, 0, vb, vec, fsi::kCopyTileBlocks, p->unpack_tiles);
    for (Tile &t : p->unpack_tiles)
        if (t.run_buf >= 0) t.run_dst = t.x_begin - p->bufinfo[t.run_buf].vbase;

    // ---- workspace layout (each table on a 256-byte boundary)
    fsi::WorkspaceLayout &w = p->ws;
    int64_t off = 0;
    auto place = [&](int64_t count, int64_t elem, int64_t *o, int64_t *n) {
        *o = off;
        *n = count;
        off = align_up(off + count * elem, 256);
    };
    place((int64_t)ps.size(), sizeof(Segment), &w.pack_segs, &w.n_pack_segs);
    place((int64_t)p->unpack_segs.size(), sizeof(Segment), &w.unpack_segs, &w.n_unpack_segs);
    place((int64_t)p->pack_tiles_all.size(), sizeof(Tile), &w.pack_tiles_all, &w.n_pack_tiles_all);
    place((int64_t)p->pack_tiles_rank.size(), sizeof(Tile), &w.pack_tiles_rank, &w.n_pack_tiles_rank);
    if (shared_grid) {   // the all-ranks launch reads the per-rank table
        w.pack_tiles_all = w.pack_tiles_rank;
        w.n_pack_tiles_all = w.n_pack_tiles_rank;
    }
    place((int64_t)p->unpack_tiles.size(), sizeof(Tile), &w.unpack_tiles, &w.n_unpack_tiles);
    place((int64_t)p->bufinfo.size(), sizeof(fsi::BufInfo), &w.bufinfo, &w.n_bufinfo);
    place((int64_t)p->local_first.size(), sizeof(int64_t), &w.local_first, &w.n_local_first);
    w.total_bytes = std::max<int64_t>(off, 256);

    // ---- summary: element type, workspace and ledger
    fs_plan_info_t &I = p->info;
    I.dtype = dtype;
    I.elem_bytes = (int32_t)eb;
    I.workspace_bytes = w.total_bytes;
    const double b = (double)eb, bopt = (double)I.bopt, Pd = (double)I.total_numel, Nd = (double)world;
    const double acc = I.grad_acc > 1 ? 4.0 : 0.0;   // fp32 gradient accumulator
    const double per_param = 2.0 * b + bopt + acc;
    I.ledger_ideal_bytes = Pd * per_param / Nd;
    I.ledger_padded_bytes = (double)shard * per_param;
    I.ledger_ddp_bytes = Pd * (2.0 * b + bopt) + acc * Pd;
    I.ledger_zero1_bytes = 2.0 * Pd * b + Pd * bopt / Nd + acc * Pd;
    I.ledger_zero2_bytes = Pd * b + Pd * (b + bopt) / Nd + acc * Pd / Nd;
    I.peak_full_shard_bytes = I.ledger_ideal_bytes + Pd * b;
    I.comm_full_shard_bytes = 3.0 * Pd * (Nd - 1.0) / Nd * b;
    I.comm_shard_grad_op_bytes = 2.0 * Pd * (Nd - 1.0) / Nd * b;
}

extern "C" int fs_plan(int32_t n_params, const int32_t *ndim, const int64_t *dims,
                       fs_dtype dtype, int32_t world, int32_t use_orig_params,
                       fs_mode mode, int32_t grad_acc, fs_plan_t *out) {
    fsi::clear_error();
    if (!out) return fsi::fail(FS_E_INVAL, "fs_plan: out is NULL");
    *out = nullptr;
    if (n_params < 0) return fsi::fail(FS_E_INVAL, "fs_plan: n_params < 0");
    if (n_params > 0 && (!ndim || !dims)) return fsi::fail(FS_E_INVAL, "fs_plan: ndim/dims is NULL");
    if (world < 1) return fsi::fail(FS_E_INVAL, "fs_plan: world must be >= 1 (got %d)", world);
    if (grad_acc < 1) return fsi::fail(FS_E_INVAL, "fs_plan: grad_acc must be >= 1 (got %d)", grad_acc);
    if (dtype != FS_BF16 && dtype != FS_FP32) return fsi::fail(FS_E_DTYPE, "fs_plan: unknown dtype %d", (int)dtype);
    if (mode != FS_FSDP1_FLAT && mode != FS_FSDP2_PER_PARAM)
        return fsi::fail(FS_E_INVAL, "fs_plan: unknown mode %d", (int)mode);
    if (use_orig_params != 0 && use_orig_params != 1)
        return fsi::fail(FS_E_INVAL, "fs_plan: use_orig_params must be 0 or 1");
    if (mode == FS_FSDP2_PER_PARAM && use_orig_params)
        return fsi::fail(FS_E_UNSUPPORTED, "fs_plan: use_orig_params is an FSDP1 option; FSDP2 shards every parameter on dim 0");

    fs_plan_s *p = new (std::nothrow) fs_plan_s();
    if (!p) return fsi::fail(FS_E_NOMEM, "fs_plan: out of host memory");
    try {
        const int64_t eb = dtype == FS_BF16 ? 2 : 4;
        const int vec = (int)(16 / eb);
        p->vec = vec;
        p->params.resize(n_params);
        memset(&p->info, 0, sizeof p->info);

        // ---- shapes -> numel, d0, row
        int64_t di = 0, total = 0;
        std::vector<int64_t> d0(n_params), row(n_params);
        for (int32_t i = 0; i < n_params; ++i) {
            if (ndim[i] < 0 || ndim[i] > 8) {
                delete p;
                return fsi::fail(FS_E_INVAL, "fs_plan: parameter %d has ndim %d (0..8 allowed)", i, ndim[i]);
            }
            int64_t n = 1, r = 1;
            for (int32_t k = 0; k < ndim[i]; ++k) {
                int64_t d = dims[di + k];
                if (d < 0) {
                    delete p;
                    return fsi::fail(FS_E_INVAL, "fs_plan: parameter %d has a negative dim", i);
                }
                if (!mul_ok(n, d, &n) || (k > 0 && !mul_ok(r, d, &r))) {
                    delete p;
                    return fsi::fail(FS_E_OVERFLOW, "fs_plan: parameter %d numel overflows int64", i);
                }
            }
            d0[i] = ndim[i] ? dims[di] : 1;   // a 0-d parameter counts as [1]
            row[i] = r;
            di += ndim[i];
            p->params[i].numel = n;
            if (!add_ok(total, n, &total)) {
                delete p;
                return fsi::fail(FS_E_OVERFLOW, "fs_plan: total numel overflows int64");
            }
        }

        // ---- layout
        int64_t shard = 0, flat = 0, align_pad = 0;
        if (mode == FS_FSDP1_FLAT) {
            const int64_t a = use_orig_params ? vec : 1;   // 16 bytes / element size
            int64_t off = 0;
            for (int32_t i = 0; i < n_params; ++i) {
                if (i > 0) {
                    int64_t aligned = align_up(off, a);
                    align_pad += aligned - off;
                    off = aligned;
                }
                p->params[i].start = off;
                if (!add_ok(off, p->params[i].numel, &off) || off > kMaxI64 - 64) {
                    delete p;
                    return fsi::fail(FS_E_OVERFLOW, "fs_plan: flat length overflows int64");
                }
            }
            flat = off;
            shard = ceil_div(flat, world);
        } else {
            int64_t t = 0;
            for (int32_t i = 0; i < n_params; ++i) {
                fs_param_layout_t &pl = p->params[i];
                pl.start = -1;
                pl.chunk_rows = ceil_div(d0[i], world);
                pl.row = row[i];
                pl.pre = t;
                int64_t part;
                if (!mul_ok(pl.chunk_rows, row[i], &part) || !add_ok(t, part, &t)) {
                    delete p;
                    return fsi::fail(FS_E_OVERFLOW, "fs_plan: shard length overflows int64");
                }
            }
            shard = t;
        }
        int64_t gathered, gathered_bytes;
        if (!mul_ok(shard, world, &gathered) || !mul_ok(gathered, eb, &gathered_bytes) ||
            gathered > kMaxI64 - 64) {
            delete p;
            return fsi::fail(FS_E_OVERFLOW, "fs_plan: gathered size overflows int64");
        }

        // ---- segments, split at rank boundaries, in gathered order
        std::vector<Segment> &ps = p->pack_segs;
        if (mode == FS_FSDP1_FLAT) {
            for (int32_t i = 0; i < n_params; ++i) {
                int64_t s = p->params[i].start, n = p->params[i].numel, e = 0;
                while (e < n) {
                    int64_t x = s + e;
                    int32_t r = (int32_t)(x / shard);
                    int64_t len = std::min(n - e, (int64_t)(r + 1) * shard - x);
                    ps.push_back(Segment{x, e, len, i, r});
                    e += len;
                }
            }
        } else {
            for (int32_t r = 0; r < world; ++r) {
                for (int32_t i = 0; i < n_params; ++i) {
                    const fs_param_layout_t &pl = p->params[i];
                    int64_t first = (int64_t)r * pl.chunk_rows;
                    int64_t rows = std::max<int64_t>(0, std::min(pl.chunk_rows, d0[i] - first));
                    int64_t len = rows * pl.row;
                    if (len > 0)
                        ps.push_back(Segment{(int64_t)r * shard + pl.pre, first * pl.row, len, i, r});
                }
            }
        }

        if ((int64_t)ps.size() > INT32_MAX) {
            delete p;
            return fsi::fail(FS_E_OVERFLOW, "fs_plan: too many copy segments");
        }
        // A parameter's elements on one rank form one run in both layouts
        // (FSDP1 cuts the flat at rank boundaries, FSDP2 gives each rank one
        // dim-0 chunk), so the rank's local piece of parameter i starts at the
        // run's first parameter element: the state-dict import reads it there.
        p->local_first.assign((size_t)world * (size_t)n_params, 0);
        for (const Segment &sg : ps) p->local_first[(size_t)sg.rank * (size_t)n_params + (size_t)sg.buf] = sg.src_off;

        // ---- summary (positions), then the element-size-dependent tables
        fs_plan_info_t &I = p->info;
        I.mode = mode;
        I.world = world;
        I.use_orig_params = use_orig_params;
        I.grad_acc = grad_acc;
        I.n_params = n_params;
        I.bopt = 12;
        I.total_numel = total;
        I.flat_numel = mode == FS_FSDP1_FLAT ? flat : 0;
        I.shard_numel = shard;
        I.gathered_numel = gathered;
        I.align_pad = align_pad;
        I.tail_pad = mode == FS_FSDP1_FLAT ? gathered - flat : gathered - total;
        I.n_segments = (int64_t)ps.size();
        finalize_plan(p, dtype);
    } catch (const std::bad_alloc &) {
        delete p;
        return fsi::fail(FS_E_NOMEM, "fs_plan: out of host memory");
    }
    *out = p;
    return FS_OK;
}

extern "C" int fs_plan_info(fs_plan_t plan, fs_plan_info_t *out) {
    fsi::clear_error();
    if (!plan || !out) return fsi::fail(FS_E_INVAL, "fs_plan_info: NULL argument");
    *out = plan->info;
    return FS_OK;
}

extern "C" int fs_plan_param(fs_plan_t plan, int32_t i, fs_param_layout_t *out) {
    fsi::clear_error();
    if (!plan || !out) return fsi::fail(FS_E_INVAL, "fs_plan_param: NULL argument");
    if (i < 0 || i >= plan->info.n_params)
        return fsi::fail(FS_E_INVAL, "fs_plan_param: index %d out of range", i);
    *out = plan->params[i];
    return FS_OK;
}

extern "C" int fs_plan_segments(fs_plan_t plan, fs_segment_t *out, int64_t cap, int64_t *n) {
    fsi::clear_error();
    if (!plan || !n) return fsi::fail(FS_E_INVAL, "fs_plan_segments: NULL argument");
    if (cap < 0 || (cap > 0 && !out)) return fsi::fail(FS_E_INVAL, "fs_plan_segments: bad output buffer");
    const int64_t total = (int64_t)plan->pack_segs.size();
    *n = total;
    for (int64_t k = 0; k < std::min(cap, total); ++k) {
        const Segment &s = plan->pack_segs[k];
        out[k] = fs_segment_t{s.vx, s.src_off, s.len, s.buf, s.rank};
    }
    return FS_OK;
}

extern "C" void fs_plan_destroy(fs_plan_t plan) { delete plan; }

// The same element positions with another element type: the parameter list,
// segments and per-rank pieces are copied, the element-size tables rebuilt.
extern "C" int fs_plan_twin(fs_plan_t plan, fs_dtype dtype, fs_plan_t *out) {
    fsi::clear_error();
    if (!plan || !out) return fsi::fail(FS_E_INVAL, "fs_plan_twin: NULL argument");
    *out = nullptr;
    if (dtype != FS_BF16 && dtype != FS_FP32) return fsi::fail(FS_E_DTYPE, "fs_plan_twin: unknown dtype %d", (int)dtype);
    int64_t bytes;
    if (!mul_ok(plan->info.gathered_numel, dtype == FS_BF16 ? 2 : 4, &bytes))
        return fsi::fail(FS_E_OVERFLOW, "fs_plan_twin: gathered size overflows int64");
    fs_plan_s *p = new (std::nothrow) fs_plan_s();
    if (!p) return fsi::fail(FS_E_NOMEM, "fs_plan_twin: out of host memory");
    try {
        p->info = plan->info;
        p->params = plan->params;
        p->pack_segs = plan->pack_segs;
        p->local_first = plan->local_first;
        finalize_plan(p, dtype);
    } catch (const std::bad_alloc &) {
        delete p;
        return fsi::fail(FS_E_NOMEM, "fs_plan_twin: out of host memory");
    }
    *out = p;
    return FS_OK;
}

// ---------------------------------------------------------------- reshard --
//
// Re-shard one group from plan `src` (N ranks, one mode) to plan `dst` (N'
// ranks, same or other mode): every parameter element moves from its place
// in src's gathered buffer to its place in dst's.  Sources: "FSDP1 vs FSDP2",
// memory and engineering section (FSDP2's shards are the sharded state dict,
// FSDP1 must unshard for one); the FSDP tutorial page (m.xxqk.cn), section
// 3.3 (sharded checkpoints do not carry over between card counts as they
// are -- they must be re-sharded).  Both plans must list the same
// parameters with the same element size.  Lowering: for each parameter, the
// two plans' runs over its elements are intersected into pieces (dst
// gathered offset, src gathered offset, length), merged when contiguous in
// both, sorted by destination, and tiled like a pack.

extern "C" int fs_reshard_plan(fs_plan_t src, fs_plan_t dst, fs_reshard_t *out) {
    fsi::clear_error();
    if (!src || !dst || !out) return fsi::fail(FS_E_INVAL, "fs_reshard_plan: NULL argument");
    *out = nullptr;
    if (src->info.n_params != dst->info.n_params)
        return fsi::fail(FS_E_INVAL, "fs_reshard_plan: the plans list %d and %d parameters", src->info.n_params,
                         dst->info.n_params);
    if (src->info.elem_bytes != dst->info.elem_bytes)
        return fsi::fail(FS_E_DTYPE, "fs_reshard_plan: the plans have different element sizes");
    const int32_t np = src->info.n_params;
    for (int32_t i = 0; i < np; ++i)
        if (src->params[i].numel != dst->params[i].numel)
            return fsi::fail(FS_E_INVAL, "fs_reshard_plan: parameter %d has %lld vs %lld elements", i,
                             (long long)src->params[i].numel, (long long)dst->params[i].numel);
    fs_reshard_s *r = new (std::nothrow) fs_reshard_s();
    if (!r) return fsi::fail(FS_E_NOMEM, "fs_reshard_plan: out of host memory");
    try {
        r->elem_bytes = src->info.elem_bytes;
        r->vec = 16 / r->elem_bytes;
        r->src_gathered = src->info.gathered_numel;
        r->dst_gathered = dst->info.gathered_numel;
        // runs of each parameter, in parameter-element order: (gathered offset, param offset, len)
        auto runs_of = [np](const fs_plan_s *p) {
            std::vector<std::vector<Segment>> by(np);
            for (const Segment &sg : p->pack_segs) by[sg.buf].push_back(sg);
            for (auto &v : by)
                std::sort(v.begin(), v.end(), [](const Segment &a, const Segment &b) { return a.src_off < b.src_off; });
            return by;
        };
        const auto sr = runs_of(src), dr = runs_of(dst);
        std::vector<Segment> pieces;
        for (int32_t i = 0; i < np; ++i) {
            size_t a = 0, b = 0;
            int64_t off = 0;
            const int64_t n = src->params[i].numel;
            while (off < n) {
                const Segment &s0 = sr[i][a], &d0 = dr[i][b];
                const int64_t ls = s0.src_off + s0.len - off, ld = d0.src_off + d0.len - off;
                const int64_t len = std::min(ls, ld);
                Segment pc{d0.vx + (off - d0.src_off), s0.vx + (off - s0.src_off), len, 0, d0.rank};
                if (!pieces.empty()) {
                    Segment &q = pieces.back();
                    if (q.vx + q.len == pc.vx && q.src_off + q.len == pc.src_off) {
                        q.len += len;
                        pc.len = 0;
                    }
                }
                if (pc.len) pieces.push_back(pc);
                off += len;
                if (len == ls) ++a;
                if (len == ld) ++b;
            }
        }
        std::sort(pieces.begin(), pieces.end(), [](const Segment &x, const Segment &y) { return x.vx < y.vx; });
        if ((int64_t)pieces.size() > INT32_MAX) {
            delete r;
            return fsi::fail(FS_E_OVERFLOW, "fs_reshard_plan: too many copy segments");
        }
        r->segs = std::move(pieces);
        fsi::build_tiles(r->segs, 0, r->dst_gathered, r->vec, fsi::kCopyTileBlocks, r->tiles);
        r->ws_segs = 0;
        r->ws_tiles = align_up((int64_t)r->segs.size() * (int64_t)sizeof(Segment), 256);
        r->ws_bytes = std::max<int64_t>(256, r->ws_tiles + align_up((int64_t)r->tiles.size() * (int64_t)sizeof(Tile), 256));
    } catch (const std::bad_alloc &) {
        delete r;
        return fsi::fail(FS_E_NOMEM, "fs_reshard_plan: out of host memory");
    }
    *out = r;
    return FS_OK;
}

extern "C" int fs_reshard_info(fs_reshard_t r, int64_t *workspace_bytes, int64_t *n_segments) {
    fsi::clear_error();
    if (!r) return fsi::fail(FS_E_INVAL, "fs_reshard_info: NULL argument");
    if (workspace_bytes) *workspace_bytes = r->ws_bytes;
    if (n_segments) *n_segments = (int64_t)r->segs.size();
    return FS_OK;
}

extern "C" void fs_reshard_destroy(fs_reshard_t r) { delete r; }
