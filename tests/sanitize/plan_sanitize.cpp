// plan_sanitize.cpp -- host-only driver for a sanitizer build (AddressSanitizer
// and UndefinedBehaviorSanitizer) of the library's planner (fs_plan.cpp) and
// of the oracle (oracle/fs_oracle.c).  Test infrastructure: it links both only
// to compare them.  It runs the integer code that decides every index the
// kernels use -- layouts, segment lowering, tile building, the re-shard piece
// intersection, the twin of the other element size -- over exhaustive tiny
// parameter lists, the workload shapes and the documented error paths, and
// checks the planner's element map against the oracle's.  Exit status 0 and a final "ok" line mean clean.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/fs.h"

extern "C" {
typedef struct {
    int32_t mode, n_params, world, elem_bytes;
    int64_t shard;
    const int64_t *numel, *start, *chunk_rows, *row, *pre;
} oracle_layout;
int oracle_fsdp1_layout(int32_t n_params, const int64_t *numel, int32_t elem_bytes, int32_t world,
                        int32_t use_orig_params, int64_t *start, int64_t *flat_len, int64_t *shard);
int oracle_fsdp2_layout(int32_t n_params, const int64_t *d0, const int64_t *row, int32_t world,
                        int64_t *chunk_rows, int64_t *pre, int64_t *shard);
void oracle_index_map(const oracle_layout *L, int64_t *out);
}

static long g_checked = 0;
static int g_fail = 0;

#define EXPECT(cond, ...)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            if (g_fail++ < 20) {                           \
                fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
                fprintf(stderr, __VA_ARGS__);              \
                fputc('\n', stderr);                       \
            }                                              \
        }                                                  \
    } while (0)

struct Shapes {
    std::vector<int32_t> ndim;
    std::vector<int64_t> dims;
};

// Planner's element map: gathered index of every parameter element, in order.
static std::vector<int64_t> plan_map(fs_plan_t p, const fs_plan_info_t &I) {
    std::vector<int64_t> numel(I.n_params), off(I.n_params + 1, 0);
    for (int32_t i = 0; i < I.n_params; ++i) {
        fs_param_layout_t pl;
        fs_plan_param(p, i, &pl);
        numel[i] = pl.numel;
        off[i + 1] = off[i] + pl.numel;
    }
    // large plans: segment bounds and per-parameter coverage only (an element
    // map of a Llama block would be 200M entries)
    const bool small = off[I.n_params] <= (1 << 22);
    std::vector<int64_t> map(small ? off[I.n_params] : 0, -1), covered(I.n_params, 0);
    int64_t n = 0;
    fs_plan_segments(p, nullptr, 0, &n);
    std::vector<fs_segment_t> segs(n > 0 ? n : 1);
    fs_plan_segments(p, segs.data(), n, &n);
    for (int64_t k = 0; k < n; ++k) {
        const fs_segment_t &s = segs[k];
        EXPECT(s.len > 0 && s.param >= 0 && s.param < I.n_params && s.src_off >= 0 &&
               s.src_off + s.len <= numel[s.param], "segment %lld out of range", (long long)k);
        EXPECT(s.dst_off / I.shard_numel == s.rank && (s.dst_off + s.len - 1) / I.shard_numel == s.rank,
               "segment %lld crosses its rank", (long long)k);
        covered[s.param] += s.len;
        if (!small) continue;
        for (int64_t e = 0; e < s.len; ++e) {
            int64_t &slot = map[off[s.param] + s.src_off + e];
            EXPECT(slot == -1, "element placed twice");
            slot = s.dst_off + e;
        }
    }
    for (int32_t i = 0; i < I.n_params; ++i) EXPECT(covered[i] == numel[i], "parameter %d covered %lld of %lld", i,
                                                    (long long)covered[i], (long long)numel[i]);
    return map;
}

static void check_case(const Shapes &sh, fs_dtype dt, int32_t world, int32_t uo, fs_mode mode,
                       fs_plan_t *keep = nullptr) {
    const int32_t np = (int32_t)sh.ndim.size();
    fs_plan_t p = nullptr;
    int rc = fs_plan(np, sh.ndim.data(), sh.dims.data(), dt, world, uo, mode, 1, &p);
    EXPECT(rc == FS_OK, "fs_plan rc %d: %s", rc, fs_last_error());
    if (rc != FS_OK) return;
    fs_plan_info_t I;
    fs_plan_info(p, &I);
    std::vector<int64_t> got = plan_map(p, I);
    // oracle
    const int32_t eb = dt == FS_BF16 ? 2 : 4;
    std::vector<int64_t> numel(np), d0(np), row(np), start(np + 1), cr(np + 1), pre(np + 1);
    int64_t di = 0;
    for (int32_t i = 0; i < np; ++i) {
        int64_t n = 1, r = 1;
        for (int32_t k = 0; k < sh.ndim[i]; ++k) {
            n *= sh.dims[di + k];
            if (k) r *= sh.dims[di + k];
        }
        d0[i] = sh.ndim[i] ? sh.dims[di] : 1;
        row[i] = r;
        numel[i] = n;
        di += sh.ndim[i];
    }
    int64_t flat = 0, shard = 0;
    oracle_layout L;
    memset(&L, 0, sizeof L);
    if (mode == FS_FSDP1_FLAT) {
        oracle_fsdp1_layout(np, numel.data(), eb, world, uo, start.data(), &flat, &shard);
        L.mode = 1;
    } else {
        oracle_fsdp2_layout(np, d0.data(), row.data(), world, cr.data(), pre.data(), &shard);
        L.mode = 2;
    }
    L.n_params = np;
    L.world = world;
    L.elem_bytes = eb;
    L.shard = shard;
    L.numel = numel.data();
    L.start = start.data();
    L.chunk_rows = cr.data();
    L.row = row.data();
    L.pre = pre.data();
    EXPECT(I.shard_numel == shard, "shard %lld vs oracle %lld", (long long)I.shard_numel, (long long)shard);
    if (!got.empty()) {
        std::vector<int64_t> want(got.size());
        oracle_index_map(&L, want.data());
        for (size_t k = 0; k < got.size(); ++k) EXPECT(got[k] == want[k], "element %zu: %lld vs %lld", k,
                                                       (long long)got[k], (long long)want[k]);
    }
    // the twin of the other element size places every element where p does
    fs_plan_t t = nullptr;
    rc = fs_plan_twin(p, dt == FS_BF16 ? FS_FP32 : FS_BF16, &t);
    EXPECT(rc == FS_OK, "fs_plan_twin rc %d: %s", rc, fs_last_error());
    if (rc == FS_OK) {
        fs_plan_info_t TI;
        fs_plan_info(t, &TI);
        EXPECT(TI.gathered_numel == I.gathered_numel && plan_map(t, TI) == got, "the twin moves elements");
        fs_plan_destroy(t);
    }
    ++g_checked;
    if (keep) *keep = p;
    else fs_plan_destroy(p);
}

static void reshard_pair(const Shapes &sh, fs_dtype dt, int32_t n1, fs_mode m1, int32_t uo1, int32_t n2,
                         fs_mode m2, int32_t uo2) {
    fs_plan_t a = nullptr, b = nullptr;
    check_case(sh, dt, n1, uo1, m1, &a);
    check_case(sh, dt, n2, uo2, m2, &b);
    if (!a || !b) {
        fs_plan_destroy(a);
        fs_plan_destroy(b);
        return;
    }
    fs_reshard_t r = nullptr;
    int rc = fs_reshard_plan(a, b, &r);
    EXPECT(rc == FS_OK, "fs_reshard_plan rc %d: %s", rc, fs_last_error());
    int64_t wb = 0, ns = 0;
    if (r) fs_reshard_info(r, &wb, &ns);
    EXPECT(!r || wb >= 256, "reshard workspace");
    fs_reshard_destroy(r);
    fs_plan_destroy(a);
    fs_plan_destroy(b);
}

int main() {
    // exhaustive: 1..3 one-dimensional parameters of 0..9 elements
    for (int np = 1; np <= 3; ++np) {
        int total = 1;
        for (int k = 0; k < np; ++k) total *= 10;
        for (int code = 0; code < total; ++code) {
            Shapes sh;
            int c = code;
            for (int k = 0; k < np; ++k) {
                sh.ndim.push_back(1);
                sh.dims.push_back(c % 10);
                c /= 10;
            }
            for (int32_t N = 1; N <= 8; ++N)
                for (fs_dtype dt : {FS_BF16, FS_FP32}) {
                    check_case(sh, dt, N, 1, FS_FSDP1_FLAT);
                    check_case(sh, dt, N, 0, FS_FSDP1_FLAT);
                    check_case(sh, dt, N, 0, FS_FSDP2_PER_PARAM);
                }
        }
    }
    // two-dimensional FSDP2 pairs, and 0-d parameters
    for (int a0 = 0; a0 <= 9; ++a0)
        for (int a1 = 1; a1 <= 3; ++a1)
            for (int b0 = 0; b0 <= 9; ++b0)
                for (int32_t N = 1; N <= 8; ++N) {
                    Shapes sh;
                    sh.ndim = {2, 0, 2};
                    sh.dims = {a0, a1, b0, 2};
                    check_case(sh, FS_BF16, N, 0, FS_FSDP2_PER_PARAM);
                    check_case(sh, FS_FP32, N, 0, FS_FSDP1_FLAT);
                }
    // re-shard between ranks counts and modes
    for (int code = 0; code < 200; ++code) {
        Shapes sh;
        sh.ndim = {2, 1, 1};
        sh.dims = {code % 13, 1 + code % 3, (code * 7) % 11, (code * 5) % 17};
        reshard_pair(sh, FS_BF16, 1 + code % 8, FS_FSDP2_PER_PARAM, 0, 1 + (code / 8) % 8, FS_FSDP1_FLAT, code & 1);
        reshard_pair(sh, FS_FP32, 1 + code % 5, FS_FSDP1_FLAT, 1, 1 + (code / 5) % 6, FS_FSDP2_PER_PARAM, 0);
    }
    // workload shapes: a Llama-7B block and a 70B block (FSDP2 and FSDP1), a
    // padding-stress list of element counts spread over [1, 4M]
    {
        const int64_t d = 4096, f = 11008;
        Shapes blk;
        blk.ndim = {2, 2, 2, 2, 2, 2, 2, 1, 1};
        blk.dims = {d, d, d, d, d, d, d, d, d, f, d, f, f, d, d, d};
        check_case(blk, FS_BF16, 8, 0, FS_FSDP2_PER_PARAM);
        check_case(blk, FS_BF16, 8, 1, FS_FSDP1_FLAT);
        const int64_t D = 8192, F = 28672, KV = 1024;
        Shapes big;
        big.ndim = {2, 2, 2, 2, 2, 2, 2, 1, 1};
        big.dims = {D, D, D, KV, D, KV, D, D, D, F, D, F, F, D, D, D};
        fs_plan_t p = nullptr;
        EXPECT(fs_plan(9, big.ndim.data(), big.dims.data(), FS_BF16, 8, 0, FS_FSDP2_PER_PARAM, 2, &p) == FS_OK, "70B block");
        fs_plan_info_t I;
        if (p) {
            fs_plan_info(p, &I);
            EXPECT(I.shard_numel == 106956800, "70B block shard %lld", (long long)I.shard_numel);
        }
        fs_plan_destroy(p);
        Shapes st;
        uint64_t x = 3;
        for (int i = 0; i < 97; ++i) {
            x = x * 6364136223846793005ull + 1442695040888963407ull;
            st.ndim.push_back(1);
            st.dims.push_back(1 + (int64_t)((x >> 33) % (1u << 22)));
        }
        for (int32_t uo : {0, 1})
            for (fs_dtype dt : {FS_BF16, FS_FP32}) check_case(st, dt, 8, uo, FS_FSDP1_FLAT);
    }
    // error paths return codes and leave nothing behind
    {
        fs_plan_t p = nullptr;
        int32_t nd = 1;
        int64_t dm = 5, neg = -1, huge = INT64_MAX / 2;
        EXPECT(fs_plan(1, &nd, &dm, FS_BF16, 0, 0, FS_FSDP1_FLAT, 1, &p) == FS_E_INVAL && !p, "world 0");
        EXPECT(fs_plan(1, &nd, &neg, FS_BF16, 2, 0, FS_FSDP1_FLAT, 1, &p) == FS_E_INVAL && !p, "negative dim");
        EXPECT(fs_plan(1, &nd, &dm, FS_BF16, 2, 1, FS_FSDP2_PER_PARAM, 1, &p) == FS_E_UNSUPPORTED && !p, "uo fsdp2");
        EXPECT(fs_plan(1, &nd, &dm, (fs_dtype)7, 2, 0, FS_FSDP1_FLAT, 1, &p) == FS_E_DTYPE && !p, "dtype");
        int32_t nd2[2] = {2, 2};
        int64_t dm2[4] = {huge, 4, huge, 4};
        EXPECT(fs_plan(2, nd2, dm2, FS_FP32, 2, 0, FS_FSDP1_FLAT, 1, &p) == FS_E_OVERFLOW && !p, "overflow");
        EXPECT(fs_plan(1, nullptr, &dm, FS_BF16, 2, 0, FS_FSDP1_FLAT, 1, &p) == FS_E_INVAL && !p, "null ndim");
    }
    if (g_fail) {
        fprintf(stderr, "%d failures over %ld checked plans\n", g_fail, g_checked);
        return 1;
    }
    printf("ok: %ld plans checked against the oracle\n", g_checked);
    return 0;
}
