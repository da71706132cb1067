// fs_kernels.hip -- gfx950 (CDNA4) kernels and the C-ABI launchers.
//
// Every kernel here is an HBM-bandwidth-bound stream with no reuse: the
// copies (pack, unpack, cast pack, re-shard, state-dict import) move bytes,
// the reduces do one fp32 add per input element, AdamW a few dozen flops per
// 30 bytes.  None is a contraction, so none uses MFMA; the design goals are
// 16-byte (dwordx4) accesses on every lane, enough loads in flight to cover
// HBM latency but not so many concurrent streams per CU that the DRAM loses
// efficiency (long launches of the reduces, AdamW, the unpack and the
// re-shard cap their resident workgroups), and no divergent control flow at
// layout boundaries.
//
// Sources (page title, section):
//   pack / unpack: "FSDP1 vs FSDP2", section 03 (FlatParameter padding and
//     chunk(N); FSDP2 dim-0 chunks concatenated into one all-gather input).
//   reduce: "Data parallelism, ZeRO and FSDP", sections 2.1 (sum, then divide
//     by N), 1 and 9.2 (fp32 accumulation on the own shard), 5 (1/grad_acc in
//     the loss).
//   AdamW: "Data parallelism, ZeRO and FSDP", sections 1 (moments, then the
//     parameter) and 9.1 (update the fp32 shard, then cast it to bf16).
//   fused reduce + AdamW: the same, section 9.2 (the own averaged fp32
//     gradient feeds the own shard's update).
//   bf16 reduce dtype and the fp32 -> bf16 cast pack: "FSDP1 vs FSDP2",
//     mixed-precision section (reduce_dtype, param_dtype).
//   re-shard and the state-dict import: "FSDP1 vs FSDP2", memory and
//     engineering section (the shards are the sharded state dict).
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "fs_plan_impl.h"
#include "../../include/fs_bench.h"

using fsi::BufInfo;
using fsi::Segment;
using fsi::Tile;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = fsi::kThreads;

__host__ __device__ __forceinline__ int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }
__host__ __device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------- memory --

__device__ __forceinline__ u32x4 ld16(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16(char *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Bytes [sh, sh+16) of the 32-byte window lo:hi (sh in 0..15): a two-level
// word select (by 2 words, then by 1) followed by a byte align.  Written with
// scalars only, so the words stay in registers.
__device__ __forceinline__ u32x4 funnel16(u32x4 lo, u32x4 hi, uint32_t sh) {
    const uint32_t q = sh >> 2, r = sh & 3;
    const bool s2 = (q & 2) != 0, s1 = (q & 1) != 0;
    const uint32_t b0 = s2 ? lo.z : lo.x, b1 = s2 ? lo.w : lo.y, b2 = s2 ? hi.x : lo.z;
    const uint32_t b3 = s2 ? hi.y : lo.w, b4 = s2 ? hi.z : hi.x, b5 = s2 ? hi.w : hi.y;
    const uint32_t a0 = s1 ? b1 : b0, a1 = s1 ? b2 : b1, a2 = s1 ? b3 : b2;
    const uint32_t a3 = s1 ? b4 : b3, a4 = s1 ? b5 : b4;
    u32x4 o;
    o.x = __builtin_amdgcn_alignbyte(a1, a0, r);
    o.y = __builtin_amdgcn_alignbyte(a2, a1, r);
    o.z = __builtin_amdgcn_alignbyte(a3, a2, r);
    o.w = __builtin_amdgcn_alignbyte(a4, a3, r);
    return o;
}

// Select mask of the elements [e_lo, e_hi) of a 16-byte block (W-byte elements).
template <int W>
__device__ __forceinline__ u32x4 elem_mask(int e_lo, int e_hi) {
    uint32_t m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (W == 4) {
            m[i] = (i >= e_lo && i < e_hi) ? 0xFFFFFFFFu : 0u;
        } else {
            uint32_t lo = (2 * i >= e_lo && 2 * i < e_hi) ? 0x0000FFFFu : 0u;
            uint32_t hi = (2 * i + 1 >= e_lo && 2 * i + 1 < e_hi) ? 0xFFFF0000u : 0u;
            m[i] = lo | hi;
        }
    }
    return u32x4{m[0], m[1], m[2], m[3]};
}

template <int W>
__device__ __forceinline__ void store_elems(char *dst, u32x4 v, int e_lo, int e_hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 16 / W; ++e) {
        if (e >= e_lo && e < e_hi) {
            if (W == 4)
                *reinterpret_cast<uint32_t *>(dst + 4 * e) = w[e];
            else
                *reinterpret_cast<uint16_t *>(dst + 2 * e) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// --------------------------------------------------------- pack / unpack --
//
// One workgroup per tile.  The tile's segments are staged in LDS; every lane
// builds 16-byte destination blocks.  For a block, each overlapping segment
// contributes its elements through two aligned 16-byte loads and a byte
// funnel shift (so a source at any element offset is read with aligned
// dwordx4 loads), merged under an element mask; elements no segment covers
// stay zero (pads).  Tiles covered by a single segment -- nearly all of them
// for large parameters -- take a uniform fast path: straight dwordx4 copies,
// or, when source and destination differ in 16-byte phase, one aligned load
// per lane with the next block taken from the neighbouring lane by a
// wavefront shuffle.
//
// Every load is a naturally aligned 16-byte block that overlaps bytes of the
// source run it serves; such a block never crosses a page, so only mapped
// memory is read.  Stores are full 16-byte blocks inside the destination, or
// per-element stores at its edges.

struct TileLds {
    int64_t vx[fsi::kTileSegs];
    int64_t end[fsi::kTileSegs];
    int64_t src[fsi::kTileSegs];
    int32_t buf[fsi::kTileSegs];
};

__device__ __forceinline__ int find_first_ending_after(const TileLds &L, int nseg, int64_t x) {
    int lo = 0, hi = nseg;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (L.end[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Source pointer of a segment: pack reads parameter `buf`, unpack reads the
// gathered buffer.
struct PackSrc {
    const void *const *params;
    __device__ __forceinline__ const char *operator()(int buf) const {
        return reinterpret_cast<const char *>(params[buf]);
    }
};
struct UnpackSrc {
    const char *gathered;
    __device__ __forceinline__ const char *operator()(int) const { return gathered; }
};
// State-dict import: parameter `buf`'s elements come from the rank's local
// piece of it, which starts at the parameter element first[buf].  The base
// is shifted back by that many elements so the segments' parameter offsets
// index the piece; only offsets inside the piece are ever read.
template <int W>
struct LocalSrc {
    const void *const *pieces;
    const int64_t *first;
    __device__ __forceinline__ const char *operator()(int buf) const {
        return reinterpret_cast<const char *>(pieces[buf]) - first[buf] * W;
    }
};

// Assemble the 16-byte block of virtual elements [x0, x0+VEC) from the
// staged segments; pads are zero.  *first receives the first overlapping
// segment (nseg if none).
template <int W, class Src>
__device__ __forceinline__ u32x4 gather_block(const TileLds &L, int nseg, int64_t x0, Src src, int *first) {
    constexpr int VEC = 16 / W;
    u32x4 r = {0u, 0u, 0u, 0u};
    int s = find_first_ending_after(L, nseg, x0);
    *first = s;
    for (; s < nseg && L.vx[s] < x0 + VEC; ++s) {
        const int e_lo = (int)(imax(x0, L.vx[s]) - x0);
        const int e_hi = (int)(imin(x0 + VEC, L.end[s]) - x0);
        // byte address element 0 of this block would have in the source run
        const intptr_t base = reinterpret_cast<intptr_t>(src(L.buf[s])) + (L.src[s] + (x0 - L.vx[s])) * W;
        const intptr_t a0 = base & ~(intptr_t)15;
        const uint32_t sh = (uint32_t)(base & 15);
        const intptr_t valid_lo = base + e_lo * W, valid_hi = base + e_hi * W;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (a0 + 16 > valid_lo) lo = ld16(reinterpret_cast<const char *>(a0));
        if (sh != 0 && a0 + 16 < valid_hi) hi = ld16(reinterpret_cast<const char *>(a0 + 16));
        const u32x4 v = funnel16(lo, hi, sh);
        const u32x4 m = elem_mask<W>(e_lo, e_hi);
        r = (r & ~m) | (v & m);
    }
    return r;
}

template <int W>
__device__ __forceinline__ void stage_tile(TileLds &L, const Segment *segs, const Tile &t) {
    for (int k = threadIdx.x; k < t.nseg; k += kThreads) {
        const Segment sg = segs[t.seg_lo + k];
        L.vx[k] = sg.vx;
        L.end[k] = sg.vx + sg.len;
        L.src[k] = sg.src_off;
        L.buf[k] = sg.buf;
    }
    __syncthreads();
}

// Uniform fast path: the whole tile is one contiguous run src -> dst with a
// 16-byte-aligned destination.  `src` is the byte address of the tile's
// first element in the source.
__device__ __forceinline__ void copy_run(char *dst, const char *src, int nblk) {
    constexpr int U = fsi::kBlocksPerThread;
    const int tid = threadIdx.x;
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(src) & 15);
    if (sh == 0) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = u * kThreads + tid;
            if (b < nblk) v[u] = ld16(src + 16 * (int64_t)b);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = u * kThreads + tid;
            if (b < nblk) st16(dst + 16 * (int64_t)b, v[u]);
        }
        return;
    }
    // Misaligned source: lane l loads aligned block b (containing the start
    // of its 16 bytes); the following aligned block is lane l+1's load,
    // fetched with a wavefront shuffle.  The last lane of each wave (and the
    // lane holding the tile's last block) loads it itself; that block holds
    // needed bytes because sh > 0.
    const char *a = src - sh;
    const int lane = tid & 63;
    u32x4 lo[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int b = u * kThreads + tid;
        lo[u] = b < nblk ? ld16(a + 16 * (int64_t)b) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int b = u * kThreads + tid;
        u32x4 hi;
        hi.x = __shfl_down(lo[u].x, 1);
        hi.y = __shfl_down(lo[u].y, 1);
        hi.z = __shfl_down(lo[u].z, 1);
        hi.w = __shfl_down(lo[u].w, 1);
        if (b < nblk) {
            if (lane == 63 || b + 1 >= nblk) hi = ld16(a + 16 * (int64_t)(b + 1));
            st16(dst + 16 * (int64_t)b, funnel16(lo[u], hi, sh));
        }
    }
}

// Destination-driven copy into one contiguous buffer (`out`, addressed from
// virtual element dst_lo): the gathered buffer for pack (Src = PackSrc, one
// source per parameter), for reshard (Src = UnpackSrc, one source: the
// other plan's gathered buffer) and one rank's shard for the state-dict
// import (Src = LocalSrc, one local piece per parameter).  Elements no
// segment covers are written as zero.
template <int W, class Src>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const Segment *__restrict__ segs,
                                                           const Tile *__restrict__ tiles, Src S,
                                                           char *__restrict__ out, int64_t dst_lo,
                                                           int64_t dst_hi) {
    constexpr int VEC = 16 / W;
    __shared__ TileLds L;
    const Tile t = tiles[blockIdx.x];
    const int64_t x_end = t.x_begin + (int64_t)t.nblk * VEC;
    char *dst0 = out + (t.x_begin - dst_lo) * W;
    const bool dst_full = t.x_begin >= dst_lo && x_end <= dst_hi &&
                          (reinterpret_cast<uintptr_t>(dst0) & 15) == 0;
    if (dst_full && t.run_buf >= 0) {   // the whole tile is one contiguous run
        copy_run(dst0, S(t.run_buf) + t.run_src * W, t.nblk);
        return;
    }
    stage_tile<W>(L, segs, t);
#pragma unroll 2
    for (int u = 0; u < fsi::kBlocksPerThread; ++u) {
        const int b = u * kThreads + threadIdx.x;
        if (b >= t.nblk) break;
        const int64_t x0 = t.x_begin + (int64_t)b * VEC;
        int first;
        const u32x4 v = gather_block<W>(L, t.nseg, x0, S, &first);
        char *dst = dst0 + 16 * (int64_t)b;
        if (dst_full) {
            st16(dst, v);
        } else {
            const int e_lo = (int)imax(0, dst_lo - x0);
            const int e_hi = (int)imin(VEC, dst_hi - x0);
            if (e_lo == 0 && e_hi == VEC && (reinterpret_cast<uintptr_t>(dst) & 15) == 0)
                st16(dst, v);
            else
                store_elems<W>(dst, v, e_lo, e_hi);
        }
    }
}

template <int W>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const Segment *__restrict__ segs,
                                                          const Tile *__restrict__ tiles,
                                                          const BufInfo *__restrict__ bufs,
                                                          const char *__restrict__ gathered,
                                                          void *const *__restrict__ params) {
    constexpr int VEC = 16 / W;
    __shared__ TileLds L;
    const Tile t = tiles[blockIdx.x];
    if (t.run_buf >= 0) {   // the whole tile is one contiguous run of parameter run_buf
        const char *src = gathered + t.run_src * W;
        if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
            // aligned source: the tile's loads go out before the destination
            // pointer is read from the parameter table (1% faster on the 7B
            // groups); a misaligned destination drops them and takes the
            // segment path below
            constexpr int U = fsi::kBlocksPerThread;
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int b = u * kThreads + threadIdx.x;
                if (b < t.nblk) v[u] = ld16(src + 16 * (int64_t)b);
            }
            char *dst0 = reinterpret_cast<char *>(params[t.run_buf]) + t.run_dst * W;
            if ((reinterpret_cast<uintptr_t>(dst0) & 15) == 0) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int b = u * kThreads + threadIdx.x;
                    if (b < t.nblk) st16(dst0 + 16 * (int64_t)b, v[u]);
                }
                return;
            }
        } else {
            char *dst0 = reinterpret_cast<char *>(params[t.run_buf]) + t.run_dst * W;
            if ((reinterpret_cast<uintptr_t>(dst0) & 15) == 0) {
                copy_run(dst0, src, t.nblk);
                return;
            }
        }
    }
    stage_tile<W>(L, segs, t);
    const UnpackSrc S{gathered};
#pragma unroll 2
    for (int u = 0; u < fsi::kBlocksPerThread; ++u) {
        const int b = u * kThreads + threadIdx.x;
        if (b >= t.nblk) break;
        const int64_t x0 = t.x_begin + (int64_t)b * VEC;
        int first;
        const u32x4 v = gather_block<W>(L, t.nseg, x0, S, &first);
        if (first >= t.nseg || L.vx[first] >= x0 + VEC) continue;   // no element of any parameter
        const int j = L.buf[first];
        const BufInfo bi = bufs[j];
        char *dst = reinterpret_cast<char *>(params[j]) + (x0 - bi.vbase) * W;
        const int e_hi = (int)imin(VEC, bi.vbase + bi.numel - x0);
        if (e_hi == VEC && (reinterpret_cast<uintptr_t>(dst) & 15) == 0)
            st16(dst, v);
        else
            store_elems<W>(dst, v, 0, e_hi);
    }
}

// ------------------------------------------------------------ cast pack --
//
// Copy-in with the parameter-dtype cast at the all-gather boundary: fp32
// parameters, bf16 gathered buffer (the plan's dtype), each element rounded
// to nearest even.  Same tiles and segments as the bit-copy pack (they are in
// destination elements); a 16-byte destination block of 8 bf16 needs 32
// source bytes: up to three aligned 16-byte loads and two funnel shifts.
// Single-run tiles with a 16-byte-aligned source (the usual case) go by
// half-blocks instead: a lane loads 16 contiguous source bytes (the wave's
// loads cover 1 KB without gaps) and stores their 8 destination bytes, all of
// the lane's loads issued before any conversion.  With the launch capped at
// six workgroups per CU this measured 3% faster on the 7B groups than whole
// blocks per lane (two 16-byte loads 32 bytes apart, one 16-byte store)
// uncapped, which had been 4% faster than one block at a time.

__device__ __forceinline__ uint16_t bf16_rne_bits(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ u32x4 cvt8_bf16(u32x4 a, u32x4 b) {
    return u32x4{(uint32_t)bf16_rne_bits(a.x) | ((uint32_t)bf16_rne_bits(a.y) << 16),
                 (uint32_t)bf16_rne_bits(a.z) | ((uint32_t)bf16_rne_bits(a.w) << 16),
                 (uint32_t)bf16_rne_bits(b.x) | ((uint32_t)bf16_rne_bits(b.y) << 16),
                 (uint32_t)bf16_rne_bits(b.z) | ((uint32_t)bf16_rne_bits(b.w) << 16)};
}

// 8 fp32 starting at byte address `base` (4-byte aligned), read with aligned
// 16-byte loads of the blocks that overlap [valid_lo, valid_hi).
__device__ __forceinline__ u32x4 load8_f32_as_bf16(intptr_t base, intptr_t valid_lo, intptr_t valid_hi) {
    const intptr_t a0 = base & ~(intptr_t)15;
    const uint32_t sh = (uint32_t)(base & 15);
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 b0 = a0 + 16 > valid_lo ? ld16(reinterpret_cast<const char *>(a0)) : z;
    const u32x4 b1 = (a0 + 16 < valid_hi && a0 + 32 > valid_lo) ? ld16(reinterpret_cast<const char *>(a0 + 16)) : z;
    const u32x4 b2 = (sh != 0 && a0 + 32 < valid_hi) ? ld16(reinterpret_cast<const char *>(a0 + 32)) : z;
    return cvt8_bf16(funnel16(b0, b1, sh), funnel16(b1, b2, sh));
}

__global__ __launch_bounds__(kThreads) void pack_cast_kernel(const Segment *__restrict__ segs,
                                                             const Tile *__restrict__ tiles,
                                                             const void *const *__restrict__ params,
                                                             char *__restrict__ out, int64_t dst_lo,
                                                             int64_t dst_hi) {
    constexpr int VEC = 8;   // bf16 per destination block
    __shared__ TileLds L;
    const Tile t = tiles[blockIdx.x];
    const int64_t x_end = t.x_begin + (int64_t)t.nblk * VEC;
    char *dst0 = out + (t.x_begin - dst_lo) * 2;
    const bool dst_full = t.x_begin >= dst_lo && x_end <= dst_hi &&
                          (reinterpret_cast<uintptr_t>(dst0) & 15) == 0;
    if (dst_full && t.run_buf >= 0) {   // one contiguous run: 32 source bytes per block
        const intptr_t src = reinterpret_cast<intptr_t>(params[t.run_buf]) + t.run_src * 4;
        if ((src & 15) == 0) {   // aligned source: half-blocks, all loads in flight, then convert and store
            constexpr int U = 2 * fsi::kBlocksPerThread;
            const int nh = 2 * t.nblk;   // half-block h: source bytes [16h, 16h+16), destination [8h, 8h+8)
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = u * kThreads + threadIdx.x;
                if (h < nh) x[u] = ld16(reinterpret_cast<const char *>(src + 16 * (intptr_t)h));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = u * kThreads + threadIdx.x;
                if (h < nh) {
                    const u32x2 w = {(uint32_t)bf16_rne_bits(x[u].x) | ((uint32_t)bf16_rne_bits(x[u].y) << 16),
                                     (uint32_t)bf16_rne_bits(x[u].z) | ((uint32_t)bf16_rne_bits(x[u].w) << 16)};
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(dst0 + 8 * (int64_t)h));
                }
            }
            return;
        }
        for (int u = 0; u < fsi::kBlocksPerThread; ++u) {
            const int b = u * kThreads + threadIdx.x;
            if (b < t.nblk) {   // the run covers all 32 source bytes of every block
                const intptr_t a = src + 32 * (intptr_t)b;
                st16(dst0 + 16 * (int64_t)b, load8_f32_as_bf16(a, a, a + 32));
            }
        }
        return;
    }
    stage_tile<2>(L, segs, t);
    for (int u = 0; u < fsi::kBlocksPerThread; ++u) {
        const int b = u * kThreads + threadIdx.x;
        if (b >= t.nblk) break;
        const int64_t x0 = t.x_begin + (int64_t)b * VEC;
        u32x4 r = {0u, 0u, 0u, 0u};
        for (int s = find_first_ending_after(L, t.nseg, x0); s < t.nseg && L.vx[s] < x0 + VEC; ++s) {
            const int e_lo = (int)(imax(x0, L.vx[s]) - x0);
            const int e_hi = (int)(imin(x0 + VEC, L.end[s]) - x0);
            const intptr_t base = reinterpret_cast<intptr_t>(params[L.buf[s]]) + (L.src[s] + (x0 - L.vx[s])) * 4;
            const u32x4 v = load8_f32_as_bf16(base, base + 4 * e_lo, base + 4 * e_hi);
            const u32x4 m = elem_mask<2>(e_lo, e_hi);
            r = (r & ~m) | (v & m);
        }
        char *dst = dst0 + 16 * (int64_t)b;
        const int e_lo = (int)imax(0, dst_lo - x0);
        const int e_hi = (int)imin(VEC, dst_hi - x0);
        if (e_lo == 0 && e_hi == VEC && (reinterpret_cast<uintptr_t>(dst) & 15) == 0)
            st16(dst, r);
        else
            store_elems<2>(dst, r, e_lo, e_hi);
    }
}

// ---------------------------------------------------------------- reduce --
//
// Every output element is the sum of its A*N terms added in fp32 in slice
// order, then one division by N.  Each lane owns whole elements, so the order
// is exactly the sequential one with no cross-lane traffic.
//
// Main kernel (16-byte-aligned slices and output): a workgroup owns a chunk
// of kThreads*4*G elements and walks the slices one after another, reading G
// groups of 4 bf16 (8 bytes) per lane from the current slice -- 2*G KB
// contiguous per slice per workgroup.  The 4*G fp32 accumulators live in
// registers; the chunk is written once, 16 bytes per lane, every store
// instruction covering 1 KB contiguous.  Reading each slice in long
// contiguous runs keeps the HBM row buffers busy on one stream at a time,
// which measured faster than interleaving all slices per element.  Passes of
// more than 16 terms use G = 16 (32 KB per slice) with two slices in flight,
// at one workgroup per CU: run in the launch spans below, it measured 0.7-1.5%
// faster than G = 32 with one slice in flight (the same 64 KB in flight) on
// all of three placements, and faster than G = 16 at two per CU (-3 to -4%
// for those), with three slices in flight (-0.3%) or G = 8 with four at two
// per CU (-2 to -10%).  (In single whole-shard launches G = 32 had measured
// 3% ahead on two of three placements.)
// Fewer terms give each workgroup little work, and G = 4 (more, shorter
// workgroups) measured 6-10% faster there (8 terms) and no slower at 16;
// at G = 4 one slice in flight beat two by 1-3% at 8 terms and 1% at 16
// (three or four: slower).
//
// General kernel (misaligned slices or output): lane i owns 8 consecutive
// elements, one 16-byte (funnel-shifted when misaligned) load per term, plus
// an element-wise tail.  The main kernel covers a partial last chunk itself
// (see the chunk dispatch below).
//
// More than kTermsPerPass terms run as chained passes that carry the fp32
// partial sum through `out` -- the same arithmetic as one pass.

constexpr int kTermsPerPass = 32;

struct SliceArgs {
    const uint16_t *p[kTermsPerPass];
};

__device__ __forceinline__ void add_bf16x8(float acc[8], u32x4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + __uint_as_float(w[i] << 16);
        acc[2 * i + 1] = acc[2 * i + 1] + __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void set_bf16x8(float acc[8], u32x4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __uint_as_float(w[i] << 16);
        acc[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Load 16 bytes of slice `p` starting at byte offset `off` (even); aligned
// loads plus a funnel shift when the slice is not 16-byte aligned.  Both
// loads overlap bytes [p+off, p+off+16), which lie inside the slice.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 ld_slice16(const uint16_t *p, int64_t off) {
    const char *c = reinterpret_cast<const char *>(p) + off;
    if (ALIGNED) return ld16(c);
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(c) & 15);
    const char *a = c - sh;
    const u32x4 lo = ld16(a);
    const u32x4 hi = sh ? ld16(a + 16) : u32x4{0u, 0u, 0u, 0u};
    return funnel16(lo, hi, sh);
}

// Misaligned slices or output: lane i owns 8 consecutive elements, one
// funnel-shifted 16-byte load per term, element stores; the last n % 8
// elements go one per lane of the first wave.
__global__ __launch_bounds__(kThreads) void reduce_general_kernel(SliceArgs sa, int nterms, int first_pass,
                                                                  int last_pass, float world, int64_t n,
                                                                  float *__restrict__ out) {
    const int64_t nvec = n >> 3;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < nvec) {
        const int64_t off = i * 16;
        float acc[8];
        int t = 0;
        if (first_pass) {
            set_bf16x8(acc, ld_slice16<false>(sa.p[0], off));
            t = 1;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = out[8 * i + e];
        }
        for (; t + 8 <= nterms; t += 8) {
            u32x4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = ld_slice16<false>(sa.p[t + k], off);
#pragma unroll
            for (int k = 0; k < 8; ++k) add_bf16x8(acc, v[k]);
        }
        for (; t < nterms; ++t) add_bf16x8(acc, ld_slice16<false>(sa.p[t], off));
        if (last_pass) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] / world;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) out[8 * i + e] = acc[e];
    }
    const int64_t tail = n - nvec * 8;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < tail) {
        const int64_t e = nvec * 8 + threadIdx.x;
        float acc;
        int t = 0;
        if (first_pass) {
            acc = __uint_as_float((uint32_t)sa.p[0][e] << 16);
            t = 1;
        } else {
            acc = out[e];
        }
        for (; t < nterms; ++t) acc = acc + __uint_as_float((uint32_t)sa.p[t][e] << 16);
        out[e] = last_pass ? acc / world : acc;
    }
}

constexpr int kRedGroupsMany = 16;                                      // passes of > kRedFewTerms terms
constexpr int kRedGroupsFew = 4;                                        // passes of <= kRedFewTerms terms
constexpr int kRedFewTerms = 16;
constexpr int64_t kWgRow = (int64_t)kThreads * 4;                       // elements of one group index across a workgroup
constexpr int64_t kRedChunk = kWgRow * kRedGroupsMany;                  // 16384 elements
constexpr int64_t kRedChunkFew = kWgRow * kRedGroupsFew;                // 4096 elements

__device__ __forceinline__ void f4(u32x4 v, float o[4]) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ u32x4 u4(const float o[4]) {
    return u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
}

__device__ __forceinline__ void add_bf16x4(float *acc, u32x2 v) {
    acc[0] = acc[0] + __uint_as_float(v.x << 16);
    acc[1] = acc[1] + __uint_as_float(v.x & 0xFFFF0000u);
    acc[2] = acc[2] + __uint_as_float(v.y << 16);
    acc[3] = acc[3] + __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void set_bf16x4(float *acc, u32x2 v) {
    acc[0] = __uint_as_float(v.x << 16);
    acc[1] = __uint_as_float(v.x & 0xFFFF0000u);
    acc[2] = __uint_as_float(v.y << 16);
    acc[3] = __uint_as_float(v.y & 0xFFFF0000u);
}

// Chunked kernels: a workgroup owns kWgRow*G consecutive elements and lane i
// the groups of 4 starting at base + u*kWgRow (base = chunk start + 4i), so
// every wave-wide access of one group index is contiguous.  A launch covers n
// with ceil(n / chunk) workgroups.  The last one, when its chunk runs past n,
// walks it in sub-chunks of kTailGroups groups with bounds (TAIL): a group is
// live when its first element lies below n, and full when all four do.  A
// live group's aligned 8- or 16-byte block still holds its first element, so
// the block lies inside a page of the buffer and is read whole; only the
// elements below n are stored.  The tail code is instantiated at the small
// group count, so it never needs more registers than the main path.
constexpr int kTailGroups = 4;

template <int G, bool TAIL>
struct Bounds {
    int nlive = G, nfull = G;   // groups of the lane with e < n, with e + 4 <= n
    int64_t n = 0;
    __device__ __forceinline__ Bounds(int64_t base, int64_t n_) : n(n_) {
        if (TAIL) {
            const int64_t rem = n_ - base;
            nlive = rem <= 0 ? 0 : (int)imin(G, (rem + kWgRow - 1) / kWgRow);
            nfull = rem < 4 ? 0 : (int)imin(G, (rem - 4) / kWgRow + 1);
        }
    }
    __device__ __forceinline__ bool live(int u) const { return !TAIL || u < nlive; }
    __device__ __forceinline__ bool full(int u) const { return !TAIL || u < nfull; }
};

template <int G, bool TAIL>
__device__ __forceinline__ void load_groups(u32x2 (&x)[G], const uint16_t *p, int64_t base, const Bounds<G, TAIL> &B) {
#pragma unroll
    for (int u = 0; u < G; ++u)
        x[u] = B.live(u) ? __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p + base + u * kWgRow))
                         : u32x2{0u, 0u};
}

template <int G, int GB, bool TAIL>
__device__ __forceinline__ void load_f32_groups(float *o, const float *p, int64_t base, const Bounds<GB, TAIL> &B,
                                                int u0 = 0) {
#pragma unroll
    for (int u = 0; u < G; ++u)
        f4(B.live(u0 + u) ? ld16(reinterpret_cast<const char *>(p + base + (u0 + u) * kWgRow)) : u32x4{0u, 0u, 0u, 0u},
           o + 4 * u);
}

// Store group u's four values (those below n, in a straddling group).
template <int G, bool TAIL>
__device__ __forceinline__ void store_f32_group(float *p, int64_t base, int u, const float *v, const Bounds<G, TAIL> &B) {
    const int64_t e = base + u * kWgRow;
    if (B.full(u)) {
        st16(reinterpret_cast<char *>(p + e), u4(v));
    } else if (B.live(u)) {
        for (int k = 0; k < 4; ++k)
            if (e + k < B.n) p[e + k] = v[k];
    }
}

// Sum the lane's G groups over slices 0..nterms-1 in slice order, into acc
// (init: acc starts as slice 0 itself, so -0 survives; else slice 0 is added
// to acc).  SL slices are in flight: slot k % SL holds slice k, refilled with
// slice k + SL once added.  Reading one slice at a time per workgroup keeps
// each HBM stream in long contiguous runs.
template <int G, int SL, bool TAIL>
__device__ __forceinline__ void sum_slices(const SliceArgs &sa, int nterms, bool init, float *acc, int64_t base,
                                           const Bounds<G, TAIL> &B) {
    u32x2 x[SL][G];
#pragma unroll
    for (int s = 0; s < SL; ++s)
        if (s < nterms) load_groups<G, TAIL>(x[s], sa.p[s], base, B);
#pragma unroll
    for (int u = 0; u < G; ++u) {
        if (init) set_bf16x4(acc + 4 * u, x[0][u]);
        else add_bf16x4(acc + 4 * u, x[0][u]);
    }
    if (SL < nterms) load_groups<G, TAIL>(x[0], sa.p[SL], base, B);
    for (int r = 0;; ++r) {
#pragma unroll
        for (int k = 1; k <= SL; ++k) {
            const int t = r * SL + k;
            if (t >= nterms) return;
#pragma unroll
            for (int u = 0; u < G; ++u) add_bf16x4(acc + 4 * u, x[k % SL][u]);
            if (t + SL < nterms) load_groups<G, TAIL>(x[k % SL], sa.p[t + SL], base, B);
        }
    }
}

template <int G, bool TAIL>
__device__ __forceinline__ void reduce_chunk(const SliceArgs &sa, int nterms, int first_pass, int last_pass,
                                             float world, float *__restrict__ out, int64_t base, int64_t n) {
    const Bounds<G, TAIL> B(base, n);
    float acc[4 * G];
    if (!first_pass) load_f32_groups<G, G, TAIL>(acc, out, base, B);   // partial sums of the earlier passes
    sum_slices<G, (G >= 16 ? 2 : 1), TAIL>(sa, nterms, first_pass, acc, base, B);   // slices in flight
    if (last_pass) {
#pragma unroll
        for (int e = 0; e < 4 * G; ++e) acc[e] = acc[e] / world;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) store_f32_group<G, TAIL>(out, base, u, acc + 4 * u, B);
}

// The chunk of workgroup blockIdx.x: whole, or the last one cut by n (walked
// in sub-chunks of kTailGroups groups).  `body(groups_tag, base, tail)` runs
// one (sub-)chunk.
#define FS_CHUNK_DISPATCH(G, FULL_CALL, TAIL_CALL)                                               \
    do {                                                                                        \
        const int64_t chunk_lo = (int64_t)blockIdx.x * (kWgRow * (G));                         \
        if (chunk_lo + kWgRow * (G) <= n) {                                                     \
            const int64_t base = chunk_lo + 4 * threadIdx.x;                                    \
            FULL_CALL;                                                                          \
        } else {                                                                                \
            for (int64_t sub = chunk_lo; sub < n; sub += kWgRow * kTailGroups) {                \
                const int64_t base = sub + 4 * threadIdx.x;                                     \
                TAIL_CALL;                                                                      \
            }                                                                                   \
        }                                                                                       \
    } while (0)

template <int G>
__global__ __launch_bounds__(kThreads) void reduce_chunk_kernel(SliceArgs sa, int nterms, int first_pass,
                                                                int last_pass, float world,
                                                                float *__restrict__ out, int64_t n) {
    static_assert(G % kTailGroups == 0, "the tail walks whole sub-chunks");
    FS_CHUNK_DISPATCH(G, (reduce_chunk<G, false>(sa, nterms, first_pass, last_pass, world, out, base, n)),
                      (reduce_chunk<kTailGroups, true>(sa, nterms, first_pass, last_pass, world, out, base, n)));
}

// ------------------------------------------------- bf16 reduce dtype --
//
// The reduce-scatter delivers each micro-step's N-way average in bf16, and
// the own shard accumulates those in fp32: per element and micro-step j, the
// N terms are added in fp32 in rank order and divided once by N, the
// quotient is rounded to bf16 (nearest even) and widened, and the micro-step
// values are accumulated in fp32 starting from the first.  Same slice-major
// chunk layout as the fp32 reduce, with a second register block for the
// running micro-step sum.  A pass holds whole micro-steps (floor(32/N) of
// them); passes carry the fp32 accumulator through `out`.

constexpr int kRsGroupsMany = 8;   // passes of more than kRedFewTerms terms: 8192-element chunks
constexpr int kRsGroupsFew = 4;    // up to kRedFewTerms terms: 4096-element chunks (5% faster at 8 terms)

__device__ __forceinline__ float bf16_round_f32(float f) {
    return __uint_as_float((uint32_t)bf16_rne_bits(__float_as_uint(f)) << 16);
}

template <int G, bool TAIL>
__device__ __forceinline__ void reduce_rs_chunk(const SliceArgs &sa, int nsteps, int world, int first_pass,
                                                float worldf, float *__restrict__ out, int64_t base, int64_t n) {
    const Bounds<G, TAIL> B(base, n);
    float acc[4 * G], sum[4 * G];
    u32x2 xa[G], xb[G];
    if (!first_pass) load_f32_groups<G, G, TAIL>(acc, out, base, B);
    const int total = nsteps * world;
    // add term t (held in x) into the micro-step sum; fold the finished micro-step into acc
    auto consume = [&](const u32x2 (&x)[G], int t) {
        const int k = t % world, j = t / world;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const float w[4] = {__uint_as_float(x[u].x << 16), __uint_as_float(x[u].x & 0xFFFF0000u),
                                __uint_as_float(x[u].y << 16), __uint_as_float(x[u].y & 0xFFFF0000u)};
#pragma unroll
            for (int q = 0; q < 4; ++q) sum[4 * u + q] = k == 0 ? w[q] : sum[4 * u + q] + w[q];
        }
        if (k == world - 1) {
#pragma unroll
            for (int e = 0; e < 4 * G; ++e) {
                const float d = bf16_round_f32(sum[e] / worldf);
                acc[e] = (first_pass && j == 0) ? d : acc[e] + d;
            }
        }
    };
    if constexpr (G <= 4) {   // short chunks: one slice in flight (1% faster at 8 terms than two)
        (void)xb;
        for (int t = 0; t < total; ++t) {
            load_groups<G, TAIL>(xa, sa.p[t], base, B);
            consume(xa, t);
        }
    } else {            // two slices in flight (one: 3-5% slower at 32 terms)
        int t = 0;
        if (t < total) load_groups<G, TAIL>(xa, sa.p[t], base, B);
        while (t < total) {
            if (t + 1 < total) load_groups<G, TAIL>(xb, sa.p[t + 1], base, B);
            consume(xa, t);
            if (++t >= total) break;
            if (t + 1 < total) load_groups<G, TAIL>(xa, sa.p[t + 1], base, B);
            consume(xb, t);
            ++t;
        }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) store_f32_group<G, TAIL>(out, base, u, acc + 4 * u, B);
}

template <int G>
__global__ __launch_bounds__(kThreads) void reduce_rs_chunk_kernel(SliceArgs sa, int nsteps, int world,
                                                                   int first_pass, float worldf,
                                                                   float *__restrict__ out, int64_t n) {
    static_assert(G % kTailGroups == 0, "the tail walks whole sub-chunks");
    FS_CHUNK_DISPATCH(G, (reduce_rs_chunk<G, false>(sa, nsteps, world, first_pass, worldf, out, base, n)),
                      (reduce_rs_chunk<kTailGroups, true>(sa, nsteps, world, first_pass, worldf, out, base, n)));
}

// Misaligned variant: 8 elements per lane, element tail.
__global__ __launch_bounds__(kThreads) void reduce_rs_general_kernel(SliceArgs sa, int nsteps, int world,
                                                                     int first_pass, float worldf, int64_t n,
                                                                     float *__restrict__ out) {
    const int64_t nvec = n >> 3;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < nvec) {
        const int64_t off = i * 16;
        float acc[8], sum[8];
        if (!first_pass) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = out[8 * i + e];
        }
        for (int j = 0; j < nsteps; ++j) {
            set_bf16x8(sum, ld_slice16<false>(sa.p[j * world], off));
            for (int k = 1; k < world; ++k) add_bf16x8(sum, ld_slice16<false>(sa.p[j * world + k], off));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = bf16_round_f32(sum[e] / worldf);
                acc[e] = (first_pass && j == 0) ? d : acc[e] + d;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) out[8 * i + e] = acc[e];
    }
    const int64_t tail = n - nvec * 8;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < tail) {
        const int64_t e = nvec * 8 + threadIdx.x;
        float acc = first_pass ? 0.0f : out[e];
        for (int j = 0; j < nsteps; ++j) {
            float sum = __uint_as_float((uint32_t)sa.p[j * world][e] << 16);
            for (int k = 1; k < world; ++k) sum = sum + __uint_as_float((uint32_t)sa.p[j * world + k][e] << 16);
            const float d = bf16_round_f32(sum / worldf);
            acc = (first_pass && j == 0) ? d : acc + d;
        }
        out[e] = acc;
    }
}

// ----------------------------------------------------------------- AdamW --
//
// One fused read-modify-write pass: read g, theta, m, v; write theta, m, v
// and the bf16 parameter.  The update is evaluated in double from the fp32
// inputs and rounded to fp32 once per stored value; the bias corrections
// 1 - beta^t are per-step scalars computed on the host.

struct AdamConsts {
    double b1, b2, omb1, omb2, bc1, bc2, lr, eps, decay;
};

__device__ __forceinline__ uint16_t bf16_rne(float f) { return bf16_rne_bits(__float_as_uint(f)); }

__device__ __forceinline__ void adam_elem(const AdamConsts &c, float g32, float &th32, float &m32,
                                          float &v32) {
    const double g = g32, th = th32, m = m32, v = v32;
    const double m_new = c.b1 * m + c.omb1 * g;
    const double v_new = c.b2 * v + c.omb2 * g * g;
    const double m_hat = m_new / c.bc1;
    const double v_hat = v_new / c.bc2;
    const double th_new = th * c.decay - c.lr * m_hat / (sqrt(v_hat) + c.eps);
    th32 = (float)th_new;
    m32 = (float)m_new;
    v32 = (float)v_new;
}

template <int G, bool TAIL>
__device__ __forceinline__ void store_bf16_group(uint16_t *p, int64_t base, int u, const float *v,
                                                 const Bounds<G, TAIL> &B) {
    const int64_t e = base + u * kWgRow;
    if (B.full(u)) {
        const u32x2 w = {(uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                         (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p + e));
    } else if (B.live(u)) {
        for (int k = 0; k < 4; ++k)
            if (e + k < B.n) p[e + k] = bf16_rne(v[k]);
    }
}

// Main AdamW kernel (all buffers 16-byte aligned): one group of 4 elements per
// lane and one wave per workgroup (256 elements), so each load or store of an
// array covers 1 KB (fp32) or 512 B (bf16) contiguous.  The kernel needs about
// 50 registers; its launch caps residency at twelve workgroups (waves) per CU.
// Small workgroups keep the last round of a launch short (one Llama-7B
// block's shard, 25.3M elements: 117 us for 1024-element workgroups against
// 143 us for 8192-element ones with a separate remainder launch); single-wave
// workgroups at twelve per CU measured 2-4% faster than 1024-element ones at
// three per CU on two of three placements and equal on the third.
constexpr int kAdamThreads = 64;
constexpr int64_t kAdamRow = (int64_t)kAdamThreads * 4;   // elements per workgroup
template <bool GRAD_BF16, bool HAS_P16, bool TAIL>
__device__ __forceinline__ void adamw_group(float *__restrict__ th, float *__restrict__ m, float *__restrict__ v,
                                            const void *__restrict__ grad, uint16_t *__restrict__ p16,
                                            const AdamConsts &c, int64_t e, int64_t n) {
    const Bounds<1, TAIL> B(e, n);
    if (!B.live(0)) return;
    float G[4], T[4], M[4], V[4];
    if (GRAD_BF16) {
        const u32x2 gb = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(
            reinterpret_cast<const uint16_t *>(grad) + e));
        set_bf16x4(G, gb);
    } else {
        f4(ld16(reinterpret_cast<const char *>(reinterpret_cast<const float *>(grad) + e)), G);
    }
    f4(ld16(reinterpret_cast<const char *>(th + e)), T);
    f4(ld16(reinterpret_cast<const char *>(m + e)), M);
    f4(ld16(reinterpret_cast<const char *>(v + e)), V);
#pragma unroll
    for (int k = 0; k < 4; ++k) adam_elem(c, G[k], T[k], M[k], V[k]);
    store_f32_group<1, TAIL>(th, e, 0, T, B);
    store_f32_group<1, TAIL>(m, e, 0, M, B);
    store_f32_group<1, TAIL>(v, e, 0, V, B);
    if (HAS_P16) store_bf16_group<1, TAIL>(p16, e, 0, T, B);
}

template <bool GRAD_BF16, bool HAS_P16>
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(float *__restrict__ th, float *__restrict__ m,
                                                             float *__restrict__ v, const void *__restrict__ grad,
                                                             uint16_t *__restrict__ p16, AdamConsts c, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * kAdamRow + 4 * threadIdx.x;
    if ((int64_t)(blockIdx.x + 1) * kAdamRow <= n)
        adamw_group<GRAD_BF16, HAS_P16, false>(th, m, v, grad, p16, c, e, n);
    else
        adamw_group<GRAD_BF16, HAS_P16, true>(th, m, v, grad, p16, c, e, n);
}

// Element-wise variant for misaligned buffers.
__global__ __launch_bounds__(kThreads) void adamw_scalar_kernel(int64_t n, float *th, float *m, float *v,
                                                                const void *grad, int grad_bf16,
                                                                uint16_t *p16, AdamConsts c) {
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= n) return;
    const float g = grad_bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(grad)[e] << 16)
                              : reinterpret_cast<const float *>(grad)[e];
    float T = th[e], M = m[e], V = v[e];
    adam_elem(c, g, T, M, V);
    th[e] = T;
    m[e] = M;
    v[e] = V;
    if (p16) p16[e] = bf16_rne(T);
}

// ------------------------------------------------------- fused reduce+AdamW --
//
// The reduce's fp32 gradient feeds AdamW directly: per element, the A*N terms
// are summed in slice order and divided by N exactly as in fs_reduce_shard,
// and that fp32 value is the gradient of the same double-precision update as
// fs_adamw_step -- so theta, m, v and the bf16 copy are bit-identical to the
// two-kernel path, while the gradient shard is never written and re-read
// (unless the caller asks for it).  Traffic per element: 2*A*N + 26 bytes
// instead of 2*A*N + 4 + 30.
//
// A workgroup sums its chunk over the slices (the reduce's loop), then loads
// theta, m, v after the slice loop -- not before it, where they would hold
// registers through the whole loop -- and updates them in batches of KB
// groups, the next batch's loads in flight during the current batch's
// arithmetic, storing array by array (all of theta, then m, v, the bf16 copy).
// With 16 groups per lane (the chunk of passes of more than kRedFewTerms
// terms) that measured 5% faster than loading the first batch before the
// slice loop and storing group by group.  The kernel is bound by HBM's mixed
// read/write rate, not by its double-precision arithmetic: a cheaper update
// formula and variants at two to four waves per SIMD measured no faster.
// Slices in flight (SL): two at 16 groups; at 4 groups (passes of at most
// kRedFewTerms terms) four when the pass has at most kFusedDeepTerms terms
// (3% faster than two at 8 terms, 2% slower at 16) and one above that (1%
// faster than two at 16 terms, up to 1% slower at 8).
constexpr int kFusedGroupsMany = 16;
constexpr int kFusedGroupsFew = 4;
constexpr int kFusedBatch = 8;
constexpr int kFusedDeepTerms = 8;

template <int G, int SL, bool HAS_P16, bool HAS_G, bool TAIL>
__device__ __forceinline__ void reduce_adamw_chunk(const SliceArgs &sa, int nterms, int first_pass, float world,
                                                   float *__restrict__ th, float *__restrict__ m,
                                                   float *__restrict__ v, uint16_t *__restrict__ p16,
                                                   const float *part, float *gout, const AdamConsts &c,
                                                   int64_t base, int64_t n) {
    constexpr int KB = kFusedBatch < G ? kFusedBatch : G;
    constexpr int NB = G / KB;
    const Bounds<G, TAIL> B(base, n);
    float acc[4 * G];
    if (!first_pass) load_f32_groups<G, G, TAIL>(acc, part, base, B);   // partial sums left by the reduce passes
    sum_slices<G, SL, TAIL>(sa, nterms, first_pass, acc, base, B);
#pragma unroll
    for (int e = 0; e < 4 * G; ++e) acc[e] = acc[e] / world;
    float T[2][4 * KB], M[2][4 * KB], V[2][4 * KB];
    auto load_state = [&](int slot, int u0) {
        load_f32_groups<KB, G, TAIL>(T[slot], th, base, B, u0);
        load_f32_groups<KB, G, TAIL>(M[slot], m, base, B, u0);
        load_f32_groups<KB, G, TAIL>(V[slot], v, base, B, u0);
    };
    load_state(0, 0);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
        const int slot = bi & 1, u0 = bi * KB;
        if (bi + 1 < NB) load_state(slot ^ 1, u0 + KB);
#pragma unroll
        for (int k = 0; k < 4 * KB; ++k) adam_elem(c, acc[4 * u0 + k], T[slot][k], M[slot][k], V[slot][k]);
#pragma unroll
        for (int q = 0; q < KB; ++q) store_f32_group<G, TAIL>(th, base, u0 + q, T[slot] + 4 * q, B);
#pragma unroll
        for (int q = 0; q < KB; ++q) store_f32_group<G, TAIL>(m, base, u0 + q, M[slot] + 4 * q, B);
#pragma unroll
        for (int q = 0; q < KB; ++q) store_f32_group<G, TAIL>(v, base, u0 + q, V[slot] + 4 * q, B);
        if (HAS_P16) {
#pragma unroll
            for (int q = 0; q < KB; ++q) store_bf16_group<G, TAIL>(p16, base, u0 + q, T[slot] + 4 * q, B);
        }
        if (HAS_G) {
#pragma unroll
            for (int q = 0; q < KB; ++q) store_f32_group<G, TAIL>(gout, base, u0 + q, acc + 4 * (u0 + q), B);
        }
    }
}

template <int G, int SL, bool HAS_P16, bool HAS_G>
__global__ __launch_bounds__(kThreads) void reduce_adamw_chunk_kernel(SliceArgs sa, int nterms, int first_pass,
                                                                      float world, float *__restrict__ th,
                                                                      float *__restrict__ m,
                                                                      float *__restrict__ v,
                                                                      uint16_t *__restrict__ p16,
                                                                      const float *part, float *gout, AdamConsts c,
                                                                      int64_t n) {
    static_assert(G % kTailGroups == 0, "the tail walks whole sub-chunks");
    FS_CHUNK_DISPATCH(G,
                      (reduce_adamw_chunk<G, SL, HAS_P16, HAS_G, false>(sa, nterms, first_pass, world, th, m, v,
                                                                        p16, part, gout, c, base, n)),
                      (reduce_adamw_chunk<kTailGroups, SL, HAS_P16, HAS_G, true>(sa, nterms, first_pass, world, th,
                                                                                 m, v, p16, part, gout, c, base, n)));
}

// Misaligned variant: lane i owns 8 consecutive elements (the general
// reduce's loads), then updates them element by element; the last n % 8
// elements go one per lane of the first wave.
__global__ __launch_bounds__(kThreads) void reduce_adamw_general_kernel(SliceArgs sa, int nterms, int first_pass,
                                                                        float world, int64_t n, float *th,
                                                                        float *m, float *v, uint16_t *p16,
                                                                        const float *part, float *gout,
                                                                        AdamConsts c) {
    const int64_t nvec = n >> 3;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < nvec) {
        const int64_t off = i * 16;
        float acc[8];
        int t = 0;
        if (first_pass) {
            set_bf16x8(acc, ld_slice16<false>(sa.p[0], off));
            t = 1;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = part[8 * i + e];
        }
        for (; t < nterms; ++t) add_bf16x8(acc, ld_slice16<false>(sa.p[t], off));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = 8 * i + e;
            const float g = acc[e] / world;
            float T = th[k], M = m[k], V = v[k];
            adam_elem(c, g, T, M, V);
            th[k] = T;
            m[k] = M;
            v[k] = V;
            if (p16) p16[k] = bf16_rne(T);
            if (gout) gout[k] = g;
        }
    }
    const int64_t tail = n - nvec * 8;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < tail) {
        const int64_t k = nvec * 8 + threadIdx.x;
        float acc;
        int t = 0;
        if (first_pass) {
            acc = __uint_as_float((uint32_t)sa.p[0][k] << 16);
            t = 1;
        } else {
            acc = part[k];
        }
        for (; t < nterms; ++t) acc = acc + __uint_as_float((uint32_t)sa.p[t][k] << 16);
        const float g = acc / world;
        float T = th[k], M = m[k], V = v[k];
        adam_elem(c, g, T, M, V);
        th[k] = T;
        m[k] = M;
        v[k] = V;
        if (p16) p16[k] = bf16_rne(T);
        if (gout) gout[k] = g;
    }
}

// ------------------------------------------------------------------ copy --

// Streaming ceilings (measurement aids): read-only, write-only and copy
// kernels, dwordx4 accesses, every instruction covering 4 KB of the
// workgroup's contiguous range, each in the shape that measured fastest on
// MI355X.  Reads want many loads in flight: two per lane at full occupancy
// (7.2 TB/s; 16 per lane 7.1).  Writes want few stores outstanding per CU:
// two per lane at one workgroup per CU (7.2 TB/s), against 5.8 for four per
// lane at full occupancy.  A copy mixes both: one block per lane in
// single-wave workgroups at full occupancy copies 6.7 TB/s (256-thread
// workgroups: 6.6 at two blocks per lane and three per CU, 6.5 at one block
// uncapped).  Read and write streams do not take single-wave workgroups of
// one block per lane: at 1 KB per workgroup the dispatcher's rate of about
// two workgroups per clock caps them near 4.8 TB/s.
constexpr int kStreamVecs = 2;         // 16-byte blocks per lane (read, fill)
constexpr int kFillWgsPerCu = 1;
constexpr int kCopyThreads = 64;       // one wave per workgroup, one block per lane

__global__ __launch_bounds__(kThreads) void read_kernel(const char *__restrict__ src, int64_t nvec,
                                                        uint32_t *__restrict__ sink) {
    const int64_t i0 = (int64_t)blockIdx.x * kThreads * kStreamVecs + threadIdx.x;
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kStreamVecs; ++u) {
        const int64_t i = i0 + u * kThreads;
        if (i < nvec) {
            const u32x4 v = ld16(src + 16 * i);
            x ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (x == 0x9E3779B9u) sink[0] = x;   // data-dependent, so the loads stay; rarely taken
}

__global__ __launch_bounds__(kThreads) void fill_kernel(char *__restrict__ dst, int64_t nvec, uint32_t value) {
    const int64_t i0 = (int64_t)blockIdx.x * kThreads * kStreamVecs + threadIdx.x;
    const u32x4 v = {value, value, value, value};
#pragma unroll
    for (int u = 0; u < kStreamVecs; ++u) {
        const int64_t i = i0 + u * kThreads;
        if (i < nvec) st16(dst + 16 * i, v);
    }
}

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(char *__restrict__ dst,
                                                            const char *__restrict__ src, int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (i < nvec) st16(dst + 16 * i, ld16(src + 16 * i));
}

// -------------------------------------------------------------- launchers --

// Per-step AdamW scalars, in double from the fp32 hyperparameters: the bias
// corrections 1 - beta^t and the decoupled decay factor 1 - lr*wd.
AdamConsts adam_consts(const fs_adamw_hparams_t &hp) {
    AdamConsts c;
    c.b1 = hp.beta1;
    c.b2 = hp.beta2;
    c.omb1 = 1.0 - c.b1;
    c.omb2 = 1.0 - c.b2;
    c.bc1 = 1.0 - pow(c.b1, (double)hp.step);
    c.bc2 = 1.0 - pow(c.b2, (double)hp.step);
    c.lr = hp.lr;
    c.eps = hp.eps;
    c.decay = 1.0 - (double)hp.lr * (double)hp.weight_decay;
    return c;
}

// Workgroups resident per CU.  The reduce and AdamW kernels stream HBM best
// with about 48-64 KB of loads in flight per CU; where their register use
// alone would let more workgroups share a CU, the extra concurrent streams
// cost DRAM efficiency.  Measured side by side on one MI355X, same buffers,
// three placements: the 32-term reduce on the 7B shard ran 4-8% faster at
// one workgroup per CU than at three (16 groups per lane; in launch spans
// one per CU still beats two by 3-4%), AdamW's single-wave workgroups 4-11% faster at
// twelve per CU (registers allow 32) than 256-thread workgroups uncapped; on
// a 70B group's shard the 16-term reduce gained 6% at three, the
// bf16-reduce-dtype kernels 3% at two (8 groups per lane) and three (4
// groups).  Of the copy kernels the unpack and the re-shard, whose loads do
// not wait for a pointer-table read, run capped at six per CU (1.6% and 2.6%
// faster); the pack, which reads the parameter pointer table before its
// loads, measured slower capped; the cast pack, whose loads are twice its
// stores, runs capped at six (3% faster with its half-block loads; five and
// seven 1% slower than six, four 7%).  A cap of k is set
// by reserving dynamic LDS that the kernel never touches: with L bytes of
// LDS per CU, L / (k + 1) + 1 bytes per workgroup let k workgroups fit but
// not k + 1.  Grids shorter than kCapMinRounds rounds of resident
// workgroups keep full occupancy: the last round of a short grid weighs
// more than the DRAM gain (one block's 8-term reduce measured 2% slower
// capped).
constexpr int kRedManyWgsPerCu = 1;    // reduce_chunk_kernel<kRedGroupsMany>
constexpr int kRedFewWgsPerCu = 3;     // reduce_chunk_kernel<kRedGroupsFew>
constexpr int kRsManyWgsPerCu = 2;     // reduce_rs_chunk_kernel<kRsGroupsMany>
constexpr int kRsFewWgsPerCu = 3;      // reduce_rs_chunk_kernel<kRsGroupsFew>
constexpr int kAdamWgsPerCu = 12;      // adamw_kernel (one wave per workgroup)
constexpr int kUnpackWgsPerCu = 6;     // unpack_kernel (registers allow 7-8)
constexpr int kReshardWgsPerCu = 6;    // scatter_kernel<W, UnpackSrc> (registers allow 8)
constexpr int kCastWgsPerCu = 6;       // pack_cast_kernel (registers allow 8)
constexpr int64_t kCapMinRounds = 16;

// Long calls run as consecutive launches over sub-ranges of at most kSpan
// elements (kRsSpan for the bf16 reduce dtype, kAdamSpan for AdamW), one
// after the other on the caller's stream.  Within one long launch the
// workgroups drift apart -- workgroups are handed to the XCDs in turn, so an
// XCD that falls behind keeps its share of the grid, and the launch ends
// with part of the chip idle -- and each launch boundary lines them up
// again.  Measured side by side on the 7B shard (842M elements), three
// separately allocated state pools: the 32-term reduce 3-8% faster in
// 32M-element launches than in one, the fused reduce + AdamW 7-13%, the
// bf16 reduce dtype 4-14% in 16M-element launches, AdamW 0.4-2% in
// 64M-element ones; the slow placements gain the most.  Spans are multiples
// of every chunk size, so each sub-range keeps the buffers' 16-byte
// alignment, and the residency caps are decided on the whole call's length.
constexpr int64_t kSpan = 32ll << 20;
constexpr int64_t kRsSpan = 16ll << 20;
constexpr int64_t kAdamSpan = 64ll << 20;

struct CuLimits {
    int lds_per_cu = 0, lds_per_wg = 0, cus = 0;   // 0: unknown, no cap
};

CuLimits cu_limits() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> lds_cu[kMaxDev], lds_wg[kMaxDev], ncu[kMaxDev];   // 0: not read yet, -1: failed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return {};
    if (lds_cu[dev].load(std::memory_order_acquire) == 0) {
        int a = 0, b = 0, c = 0;
        const bool ok = hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
                            hipSuccess &&
                        hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
                        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                        a > 0 && b > 0 && c > 0;
        lds_wg[dev].store(ok ? b : -1, std::memory_order_relaxed);
        ncu[dev].store(ok ? c : -1, std::memory_order_relaxed);
        lds_cu[dev].store(ok ? a : -1, std::memory_order_release);
    }
    CuLimits L;
    if (lds_cu[dev].load(std::memory_order_acquire) < 0) return L;
    L.lds_per_cu = lds_cu[dev].load(std::memory_order_relaxed);
    L.lds_per_wg = lds_wg[dev].load(std::memory_order_relaxed);
    L.cus = ncu[dev].load(std::memory_order_relaxed);
    return L;
}

// Dynamic LDS bytes for a grid of `grid` workgroups capped at k per CU, for a
// kernel that already uses `static_bytes` of LDS (0: no cap).
uint32_t lds_cap(int k, int64_t grid, int64_t static_bytes = 0) {
    const CuLimits L = cu_limits();
    if (L.lds_per_cu <= 0 || k < 1) return 0;
    if (grid < kCapMinRounds * k * (int64_t)L.cus) return 0;
    const int64_t per_wg = L.lds_per_cu / (k + 1) + 1;   // k of these fit in a CU, k + 1 do not
    if (per_wg > L.lds_per_wg || per_wg * k > L.lds_per_cu || per_wg <= static_bytes) return 0;
    return (uint32_t)(per_wg - static_bytes);
}

int check_hparams(const char *what, const fs_adamw_hparams_t *hp) {
    if (!hp) return fsi::fail(FS_E_INVAL, "%s: hp is NULL", what);
    if (hp->step < 1) return fsi::fail(FS_E_INVAL, "%s: step must be >= 1", what);
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f && hp->beta2 >= 0.f && hp->beta2 < 1.f))
        return fsi::fail(FS_E_INVAL, "%s: betas must lie in [0, 1)", what);
    return FS_OK;
}

// The tables live on the device they were uploaded to: launching from
// another device would hand its kernels a foreign address.
int check_device(const char *what, int dev_id) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fsi::fail(FS_E_HIP, "%s: no current device", what);
    if (dev != dev_id)
        return fsi::fail(FS_E_INVAL, "%s: the plan was uploaded on device %d, current device is %d", what, dev_id, dev);
    return FS_OK;
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// A plan's workspace holds the tables its kernels read, so it must be
// device memory of the current device; *dev receives that device.
int check_workspace(const char *what, const void *ws, int *dev) {
    if (hipGetDevice(dev) != hipSuccess) return fsi::fail(FS_E_HIP, "%s: no current device", what);
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof a);
    if (hipPointerGetAttributes(&a, ws) != hipSuccess) {
        (void)hipGetLastError();   // the query's error is not a launch error: do not leave it behind
        return fsi::fail(FS_E_INVAL, "%s: workspace is not device memory", what);
    }
    if (a.type != hipMemoryTypeDevice || a.device != *dev)
        return fsi::fail(FS_E_INVAL, "%s: workspace must be device memory of the current device (%d)", what, *dev);
    return FS_OK;
}

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fsi::fail(FS_E_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return FS_OK;
}

// Call f(std::integral_constant<bool, a>, std::integral_constant<bool, b>):
// picks the kernel instantiation for two run-time flags.
template <class F>
void with_flags(bool a, bool b, F &&f) {
    using T = std::true_type;
    using U = std::false_type;
    if (a) {
        if (b) f(T{}, T{}); else f(T{}, U{});
    } else {
        if (b) f(U{}, T{}); else f(U{}, U{});
    }
}

template <int G, int SL>
void launch_fused(int64_t n, hipStream_t stream, const SliceArgs &sa, int cnt, int first, float world, float *th,
                  float *m, float *v, uint16_t *p16, const float *part, float *gout, const AdamConsts &c) {
    const dim3 g((uint32_t)((n + kWgRow * G - 1) / (kWgRow * G))), b(kThreads);
    with_flags(p16 != nullptr, gout != nullptr, [&](auto has_p16, auto has_g) {
        hipLaunchKernelGGL((reduce_adamw_chunk_kernel<G, SL, decltype(has_p16)::value, decltype(has_g)::value>), g, b,
                           0, stream, sa, cnt, first, world, th, m, v, p16, part, gout, c, n);
    });
}

// One pass of the fp32 reduce over terms [t0, t0 + cnt) and the sub-range
// [off, off + len) of a call over n elements: chunked when every pointer is
// 16-byte aligned (one launch, its last chunk partial; the residency cap is
// decided on n), else the general kernel.
void launch_reduce_pass(int64_t n, int64_t off, int64_t len, hipStream_t stream, const uint16_t *const *slices,
                        int t0, int cnt, int first, int last, float world, bool aligned, float *out) {
    SliceArgs sa;
    memset(&sa, 0, sizeof sa);
    for (int k = 0; k < cnt; ++k) sa.p[k] = slices[t0 + k] + off;
    float *o = out + off;
    if (aligned) {
        const bool few = cnt <= kRedFewTerms;
        const int64_t chunk = few ? kRedChunkFew : kRedChunk;
        const dim3 g((uint32_t)((len + chunk - 1) / chunk));
        const uint32_t lds = lds_cap(few ? kRedFewWgsPerCu : kRedManyWgsPerCu, (n + chunk - 1) / chunk);
        if (few)
            hipLaunchKernelGGL(reduce_chunk_kernel<kRedGroupsFew>, g, dim3(kThreads), lds, stream, sa, cnt, first,
                               last, world, o, len);
        else
            hipLaunchKernelGGL(reduce_chunk_kernel<kRedGroupsMany>, g, dim3(kThreads), lds, stream, sa, cnt, first,
                               last, world, o, len);
    } else {
        const int64_t grid = std::max<int64_t>(1, ((len >> 3) + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(reduce_general_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, sa, cnt, first,
                           last, world, len, o);
    }
}

// Largest grid any launch over n elements needs: one workgroup per kAdamRow
// elements (AdamW) bounds every chunked kernel; the general kernels use one
// lane per 8 elements.
bool grid_fits(int64_t n) {
    return (n + kAdamRow - 1) / kAdamRow <= INT32_MAX && ((n >> 3) + kThreads - 1) / kThreads <= INT32_MAX;
}

bool ranges_overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return abytes > 0 && bbytes > 0 && x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

// Index of the first of `cnt` buffers that overlaps an earlier one, or -1.
// AdamW reads element k of every array and writes element k of its outputs,
// so two arrays sharing memory would mix one element's state into another's.
int first_overlap(const void *const *ptr, const int64_t *bytes, int cnt) {
    for (int i = 1; i < cnt; ++i)
        for (int j = 0; j < i; ++j)
            if (ranges_overlap(ptr[i], bytes[i], ptr[j], bytes[j])) return i;
    return -1;
}

}  // namespace

extern "C" int fs_plan_upload(fs_plan_t plan, void *workspace, size_t bytes, hipStream_t stream) {
    fsi::clear_error();
    if (!plan || !workspace) return fsi::fail(FS_E_INVAL, "fs_plan_upload: NULL argument");
    if (misaligned(workspace, 16)) return fsi::fail(FS_E_ALIGN, "fs_plan_upload: workspace must be 16-byte aligned");
    const fsi::WorkspaceLayout &w = plan->ws;
    if ((int64_t)bytes < w.total_bytes)
        return fsi::fail(FS_E_INVAL, "fs_plan_upload: workspace too small (%zu < %lld bytes)", bytes,
                         (long long)w.total_bytes);
    int dev = -1;
    if (int rc = check_workspace("fs_plan_upload", workspace, &dev)) return rc;
    char *ws = static_cast<char *>(workspace);
    struct Part { int64_t off; const void *src; int64_t bytes; };
    const Part parts[] = {
        {w.pack_segs, plan->pack_segs.data(), w.n_pack_segs * (int64_t)sizeof(Segment)},
        {w.unpack_segs, plan->unpack_segs.data(), w.n_unpack_segs * (int64_t)sizeof(Segment)},
        // (empty when the all-ranks launch shares the per-rank table)
        {w.pack_tiles_all, plan->pack_tiles_all.data(), (int64_t)plan->pack_tiles_all.size() * (int64_t)sizeof(Tile)},
        {w.pack_tiles_rank, plan->pack_tiles_rank.data(), w.n_pack_tiles_rank * (int64_t)sizeof(Tile)},
        {w.unpack_tiles, plan->unpack_tiles.data(), w.n_unpack_tiles * (int64_t)sizeof(Tile)},
        {w.bufinfo, plan->bufinfo.data(), w.n_bufinfo * (int64_t)sizeof(BufInfo)},
        {w.local_first, plan->local_first.data(), w.n_local_first * (int64_t)sizeof(int64_t)},
    };
    for (const Part &p : parts) {
        if (p.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(ws + p.off, p.src, (size_t)p.bytes, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return fsi::fail(FS_E_HIP, "fs_plan_upload: copy failed: %s", hipGetErrorString(e));
    }
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fsi::fail(FS_E_HIP, "fs_plan_upload: sync failed: %s", hipGetErrorString(e));
    plan->dev_ws = workspace;
    plan->dev_id = dev;
    return FS_OK;
}

extern "C" int fs_pack(fs_plan_t plan, const void *const *params, void *out, int32_t rank,
                       hipStream_t stream) {
    fsi::clear_error();
    if (!plan) return fsi::fail(FS_E_INVAL, "fs_pack: plan is NULL");
    const fs_plan_info_t &I = plan->info;
    if (!plan->dev_ws) return fsi::fail(FS_E_INVAL, "fs_pack: plan has no uploaded workspace (call fs_plan_upload)");
    if (int rc = check_device("fs_pack", plan->dev_id)) return rc;
    if (rank < -1 || rank >= I.world) return fsi::fail(FS_E_INVAL, "fs_pack: rank %d out of range [-1, %d)", rank, I.world);
    const int64_t lo = rank < 0 ? 0 : (int64_t)rank * I.shard_numel;
    const int64_t hi = rank < 0 ? I.gathered_numel : lo + I.shard_numel;
    if (hi == lo) return FS_OK;
    if (!out) return fsi::fail(FS_E_INVAL, "fs_pack: out is NULL");
    if (I.n_params > 0 && !params) return fsi::fail(FS_E_INVAL, "fs_pack: params is NULL");
    if (misaligned(out, I.elem_bytes)) return fsi::fail(FS_E_ALIGN, "fs_pack: out not aligned to %d bytes", I.elem_bytes);
    const char *ws = static_cast<const char *>(plan->dev_ws);
    const Segment *segs = reinterpret_cast<const Segment *>(ws + plan->ws.pack_segs);
    const Tile *tiles;
    int64_t ntiles;
    if (rank < 0) {
        tiles = reinterpret_cast<const Tile *>(ws + plan->ws.pack_tiles_all);
        ntiles = plan->ws.n_pack_tiles_all;
    } else {
        tiles = reinterpret_cast<const Tile *>(ws + plan->ws.pack_tiles_rank) + plan->rank_tile_off[rank];
        ntiles = plan->rank_tile_off[rank + 1] - plan->rank_tile_off[rank];
    }
    if (ntiles == 0) return FS_OK;
    if (ntiles > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_pack: too many tiles for one launch");
    (void)hipGetLastError();
    // `out` is addressed from the virtual element `lo` on
    char *base = static_cast<char *>(out);
    const PackSrc src{params};
    if (I.elem_bytes == 2)
        hipLaunchKernelGGL((scatter_kernel<2, PackSrc>), dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, segs,
                           tiles, src, base, lo, hi);
    else
        hipLaunchKernelGGL((scatter_kernel<4, PackSrc>), dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, segs,
                           tiles, src, base, lo, hi);
    return check_launch("fs_pack");
}

extern "C" int fs_load_local(fs_plan_t plan, int32_t rank, const void *const *pieces, void *shard,
                             hipStream_t stream) {
    fsi::clear_error();
    if (!plan) return fsi::fail(FS_E_INVAL, "fs_load_local: plan is NULL");
    const fs_plan_info_t &I = plan->info;
    if (!plan->dev_ws) return fsi::fail(FS_E_INVAL, "fs_load_local: plan has no uploaded workspace (call fs_plan_upload)");
    if (int rc = check_device("fs_load_local", plan->dev_id)) return rc;
    if (rank < 0 || rank >= I.world) return fsi::fail(FS_E_INVAL, "fs_load_local: rank %d out of range [0, %d)", rank, I.world);
    if (I.shard_numel == 0) return FS_OK;
    if (!shard) return fsi::fail(FS_E_INVAL, "fs_load_local: shard is NULL");
    if (I.n_params > 0 && !pieces) return fsi::fail(FS_E_INVAL, "fs_load_local: pieces is NULL");
    if (misaligned(shard, I.elem_bytes))
        return fsi::fail(FS_E_ALIGN, "fs_load_local: shard not aligned to %d bytes", I.elem_bytes);
    const char *ws = static_cast<const char *>(plan->dev_ws);
    const Segment *segs = reinterpret_cast<const Segment *>(ws + plan->ws.pack_segs);
    const Tile *tiles = reinterpret_cast<const Tile *>(ws + plan->ws.pack_tiles_rank) + plan->rank_tile_off[rank];
    const int64_t ntiles = plan->rank_tile_off[rank + 1] - plan->rank_tile_off[rank];
    if (ntiles == 0) return FS_OK;
    if (ntiles > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_load_local: too many tiles for one launch");
    const int64_t *first = reinterpret_cast<const int64_t *>(ws + plan->ws.local_first) + (int64_t)rank * I.n_params;
    const int64_t lo = (int64_t)rank * I.shard_numel, hi = lo + I.shard_numel;
    (void)hipGetLastError();
    char *out = static_cast<char *>(shard);   // addressed from the virtual element lo
    if (I.elem_bytes == 2)
        hipLaunchKernelGGL((scatter_kernel<2, LocalSrc<2>>), dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, segs,
                           tiles, LocalSrc<2>{pieces, first}, out, lo, hi);
    else
        hipLaunchKernelGGL((scatter_kernel<4, LocalSrc<4>>), dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, segs,
                           tiles, LocalSrc<4>{pieces, first}, out, lo, hi);
    return check_launch("fs_load_local");
}

extern "C" int fs_reshard_upload(fs_reshard_t r, void *workspace, size_t bytes, hipStream_t stream) {
    fsi::clear_error();
    if (!r || !workspace) return fsi::fail(FS_E_INVAL, "fs_reshard_upload: NULL argument");
    if (misaligned(workspace, 16)) return fsi::fail(FS_E_ALIGN, "fs_reshard_upload: workspace must be 16-byte aligned");
    if ((int64_t)bytes < r->ws_bytes)
        return fsi::fail(FS_E_INVAL, "fs_reshard_upload: workspace too small (%zu < %lld bytes)", bytes,
                         (long long)r->ws_bytes);
    int dev = -1;
    if (int rc = check_workspace("fs_reshard_upload", workspace, &dev)) return rc;
    char *ws = static_cast<char *>(workspace);
    if (!r->segs.empty()) {
        hipError_t e = hipMemcpyAsync(ws + r->ws_segs, r->segs.data(), r->segs.size() * sizeof(Segment),
                                      hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return fsi::fail(FS_E_HIP, "fs_reshard_upload: copy failed: %s", hipGetErrorString(e));
    }
    if (!r->tiles.empty()) {
        hipError_t e = hipMemcpyAsync(ws + r->ws_tiles, r->tiles.data(), r->tiles.size() * sizeof(Tile),
                                      hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return fsi::fail(FS_E_HIP, "fs_reshard_upload: copy failed: %s", hipGetErrorString(e));
    }
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fsi::fail(FS_E_HIP, "fs_reshard_upload: sync failed: %s", hipGetErrorString(e));
    r->dev_ws = workspace;
    r->dev_id = dev;
    return FS_OK;
}

extern "C" int fs_reshard(fs_reshard_t r, const void *src_gathered, void *dst_gathered, hipStream_t stream) {
    fsi::clear_error();
    if (!r) return fsi::fail(FS_E_INVAL, "fs_reshard: plan is NULL");
    if (!r->dev_ws) return fsi::fail(FS_E_INVAL, "fs_reshard: no uploaded workspace (call fs_reshard_upload)");
    if (int rc = check_device("fs_reshard", r->dev_id)) return rc;
    if (r->dst_gathered == 0) return FS_OK;
    if (!dst_gathered || (r->src_gathered > 0 && !src_gathered)) return fsi::fail(FS_E_INVAL, "fs_reshard: NULL buffer");
    if (misaligned(dst_gathered, r->elem_bytes) || (src_gathered && misaligned(src_gathered, r->elem_bytes)))
        return fsi::fail(FS_E_ALIGN, "fs_reshard: buffers must be aligned to %d bytes", r->elem_bytes);
    if (ranges_overlap(src_gathered, r->src_gathered * r->elem_bytes, dst_gathered, r->dst_gathered * r->elem_bytes))
        return fsi::fail(FS_E_INVAL, "fs_reshard: source and destination overlap");
    const char *ws = static_cast<const char *>(r->dev_ws);
    const Segment *segs = reinterpret_cast<const Segment *>(ws + r->ws_segs);
    const Tile *tiles = reinterpret_cast<const Tile *>(ws + r->ws_tiles);
    const int64_t ntiles = (int64_t)r->tiles.size();
    if (ntiles == 0) return FS_OK;
    if (ntiles > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_reshard: too many tiles for one launch");
    (void)hipGetLastError();
    const UnpackSrc src{static_cast<const char *>(src_gathered)};
    char *dst = static_cast<char *>(dst_gathered);
    const uint32_t lds = lds_cap(kReshardWgsPerCu, ntiles, (int64_t)sizeof(TileLds));
    if (r->elem_bytes == 2)
        hipLaunchKernelGGL((scatter_kernel<2, UnpackSrc>), dim3((uint32_t)ntiles), dim3(kThreads), lds, stream, segs,
                           tiles, src, dst, (int64_t)0, r->dst_gathered);
    else
        hipLaunchKernelGGL((scatter_kernel<4, UnpackSrc>), dim3((uint32_t)ntiles), dim3(kThreads), lds, stream, segs,
                           tiles, src, dst, (int64_t)0, r->dst_gathered);
    return check_launch("fs_reshard");
}

extern "C" int fs_unpack(fs_plan_t plan, const void *gathered, void *const *params, hipStream_t stream) {
    fsi::clear_error();
    if (!plan) return fsi::fail(FS_E_INVAL, "fs_unpack: plan is NULL");
    const fs_plan_info_t &I = plan->info;
    if (!plan->dev_ws) return fsi::fail(FS_E_INVAL, "fs_unpack: plan has no uploaded workspace (call fs_plan_upload)");
    if (int rc = check_device("fs_unpack", plan->dev_id)) return rc;
    const int64_t ntiles = plan->ws.n_unpack_tiles;
    if (ntiles == 0 || I.total_numel == 0) return FS_OK;
    if (ntiles > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_unpack: too many tiles for one launch");
    if (!gathered || !params) return fsi::fail(FS_E_INVAL, "fs_unpack: NULL pointer");
    if (misaligned(gathered, I.elem_bytes))
        return fsi::fail(FS_E_ALIGN, "fs_unpack: gathered not aligned to %d bytes", I.elem_bytes);
    const char *ws = static_cast<const char *>(plan->dev_ws);
    const Segment *segs = reinterpret_cast<const Segment *>(ws + plan->ws.unpack_segs);
    const Tile *tiles = reinterpret_cast<const Tile *>(ws + plan->ws.unpack_tiles);
    const BufInfo *bufs = reinterpret_cast<const BufInfo *>(ws + plan->ws.bufinfo);
    (void)hipGetLastError();
    const char *g = static_cast<const char *>(gathered);
    const uint32_t lds = lds_cap(kUnpackWgsPerCu, ntiles, (int64_t)sizeof(TileLds));
    if (I.elem_bytes == 2)
        hipLaunchKernelGGL(unpack_kernel<2>, dim3((uint32_t)ntiles), dim3(kThreads), lds, stream, segs, tiles,
                           bufs, g, params);
    else
        hipLaunchKernelGGL(unpack_kernel<4>, dim3((uint32_t)ntiles), dim3(kThreads), lds, stream, segs, tiles,
                           bufs, g, params);
    return check_launch("fs_unpack");
}

namespace {

// Shared argument checks of the reduce entry points.  Sets *terms and
// *aligned (every slice and `out` 16-byte aligned).  Returns FS_OK, or the
// error; *skip is set when n == 0 (nothing to launch).
int check_reduce(const char *what, int64_t n, int32_t world, int32_t grad_acc, const uint16_t *const *slices,
                 const float *out, int *terms, bool *aligned, bool *skip) {
    *skip = false;
    if (n < 0) return fsi::fail(FS_E_INVAL, "%s: n < 0", what);
    if (world < 1 || grad_acc < 1) return fsi::fail(FS_E_INVAL, "%s: world and grad_acc must be >= 1", what);
    int64_t terms64;
    if (__builtin_mul_overflow((int64_t)world, (int64_t)grad_acc, &terms64) || terms64 > (1 << 20))
        return fsi::fail(FS_E_OVERFLOW, "%s: too many terms", what);
    int64_t bytes_in, bytes_out;
    if (__builtin_mul_overflow(n, (int64_t)2, &bytes_in) || __builtin_mul_overflow(n, (int64_t)4, &bytes_out))
        return fsi::fail(FS_E_OVERFLOW, "%s: n too large", what);
    if (n == 0) {
        *skip = true;
        return FS_OK;
    }
    if (!slices || !out) return fsi::fail(FS_E_INVAL, "%s: NULL pointer", what);
    *terms = (int)terms64;
    *aligned = !misaligned(out, 16);
    if (misaligned(out, 4)) return fsi::fail(FS_E_ALIGN, "%s: out not 4-byte aligned", what);
    for (int t = 0; t < *terms; ++t) {
        if (!slices[t]) return fsi::fail(FS_E_INVAL, "%s: slice %d is NULL", what, t);
        if (misaligned(slices[t], 2)) return fsi::fail(FS_E_ALIGN, "%s: slice %d not 2-byte aligned", what, t);
        if (misaligned(slices[t], 16)) *aligned = false;
        if (ranges_overlap(slices[t], bytes_in, out, bytes_out))
            return fsi::fail(FS_E_INVAL, "%s: out overlaps slice %d", what, t);
    }
    return FS_OK;
}

}  // namespace

extern "C" int fs_reduce_shard(int64_t n, int32_t world, int32_t grad_acc, const uint16_t *const *slices,
                               float *out, hipStream_t stream) {
    fsi::clear_error();
    int terms = 0;
    bool aligned = false, skip = false;
    if (int rc = check_reduce("fs_reduce_shard", n, world, grad_acc, slices, out, &terms, &aligned, &skip)) return rc;
    if (skip) return FS_OK;
    if (!grid_fits(n)) return fsi::fail(FS_E_OVERFLOW, "fs_reduce_shard: n too large for one launch");
    (void)hipGetLastError();
    for (int64_t off = 0; off < n; off += kSpan) {
        const int64_t len = std::min(kSpan, n - off);
        for (int t0 = 0; t0 < terms; t0 += kTermsPerPass) {
            const int cnt = std::min(kTermsPerPass, terms - t0);
            launch_reduce_pass(n, off, len, stream, slices, t0, cnt, t0 == 0, t0 + cnt == terms, (float)world,
                               aligned, out);
            int rc = check_launch("fs_reduce_shard");
            if (rc != FS_OK) return rc;
        }
    }
    return FS_OK;
}

extern "C" int fs_reduce_shard_ex(int64_t n, int32_t world, int32_t grad_acc, fs_dtype reduce_dtype,
                                  const uint16_t *const *slices, float *out, hipStream_t stream) {
    fsi::clear_error();
    if (reduce_dtype == FS_FP32) return fs_reduce_shard(n, world, grad_acc, slices, out, stream);
    if (reduce_dtype != FS_BF16) return fsi::fail(FS_E_DTYPE, "fs_reduce_shard_ex: unknown reduce dtype");
    int terms = 0;
    bool aligned = false, skip = false;
    if (int rc = check_reduce("fs_reduce_shard_ex", n, world, grad_acc, slices, out, &terms, &aligned, &skip))
        return rc;
    if (skip) return FS_OK;
    if (world > kTermsPerPass)
        return fsi::fail(FS_E_UNSUPPORTED, "fs_reduce_shard_ex: bf16 reduce dtype supports world <= %d", kTermsPerPass);
    const int steps_per_pass = kTermsPerPass / world;
    if (!grid_fits(n)) return fsi::fail(FS_E_OVERFLOW, "fs_reduce_shard_ex: n too large for one launch");
    (void)hipGetLastError();
    for (int64_t off = 0; off < n; off += kRsSpan) {
        const int64_t len = std::min(kRsSpan, n - off);
        float *o = out + off;
        for (int j0 = 0; j0 < grad_acc; j0 += steps_per_pass) {
            const int steps = std::min(steps_per_pass, grad_acc - j0);
            const int first = j0 == 0;
            SliceArgs sa;
            memset(&sa, 0, sizeof sa);
            for (int k = 0; k < steps * world; ++k) sa.p[k] = slices[j0 * world + k] + off;
            if (aligned) {
                const bool few = steps * world <= kRedFewTerms;
                const int64_t chunk = kWgRow * (few ? kRsGroupsFew : kRsGroupsMany);
                const dim3 g((uint32_t)((len + chunk - 1) / chunk));
                const uint32_t lds = lds_cap(few ? kRsFewWgsPerCu : kRsManyWgsPerCu, (n + chunk - 1) / chunk);
                if (few)
                    hipLaunchKernelGGL(reduce_rs_chunk_kernel<kRsGroupsFew>, g, dim3(kThreads), lds, stream, sa,
                                       steps, (int)world, first, (float)world, o, len);
                else
                    hipLaunchKernelGGL(reduce_rs_chunk_kernel<kRsGroupsMany>, g, dim3(kThreads), lds, stream, sa,
                                       steps, (int)world, first, (float)world, o, len);
            } else {
                const int64_t grid = std::max<int64_t>(1, ((len >> 3) + kThreads - 1) / kThreads);
                hipLaunchKernelGGL(reduce_rs_general_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, sa,
                                   steps, (int)world, first, (float)world, len, o);
            }
            int rc = check_launch("fs_reduce_shard_ex");
            if (rc != FS_OK) return rc;
        }
    }
    return FS_OK;
}

extern "C" int fs_pack_cast(fs_plan_t plan, const void *const *params, fs_dtype param_dtype, void *out,
                            int32_t rank, hipStream_t stream) {
    fsi::clear_error();
    if (!plan) return fsi::fail(FS_E_INVAL, "fs_pack_cast: plan is NULL");
    const fs_plan_info_t &I = plan->info;
    if (param_dtype != FS_BF16 && param_dtype != FS_FP32) return fsi::fail(FS_E_DTYPE, "fs_pack_cast: unknown dtype");
    if ((int)param_dtype == I.dtype) return fs_pack(plan, params, out, rank, stream);
    if (!(param_dtype == FS_FP32 && I.dtype == FS_BF16))
        return fsi::fail(FS_E_UNSUPPORTED, "fs_pack_cast: only fp32 parameters into a bf16 layout are defined");
    if (!plan->dev_ws) return fsi::fail(FS_E_INVAL, "fs_pack_cast: plan has no uploaded workspace (call fs_plan_upload)");
    if (int rc = check_device("fs_pack_cast", plan->dev_id)) return rc;
    if (rank < -1 || rank >= I.world)
        return fsi::fail(FS_E_INVAL, "fs_pack_cast: rank %d out of range [-1, %d)", rank, I.world);
    const int64_t lo = rank < 0 ? 0 : (int64_t)rank * I.shard_numel;
    const int64_t hi = rank < 0 ? I.gathered_numel : lo + I.shard_numel;
    if (hi == lo) return FS_OK;
    if (!out) return fsi::fail(FS_E_INVAL, "fs_pack_cast: out is NULL");
    if (I.n_params > 0 && !params) return fsi::fail(FS_E_INVAL, "fs_pack_cast: params is NULL");
    if (misaligned(out, 2)) return fsi::fail(FS_E_ALIGN, "fs_pack_cast: out not aligned to 2 bytes");
    const char *ws = static_cast<const char *>(plan->dev_ws);
    const Segment *segs = reinterpret_cast<const Segment *>(ws + plan->ws.pack_segs);
    const Tile *tiles;
    int64_t ntiles;
    if (rank < 0) {
        tiles = reinterpret_cast<const Tile *>(ws + plan->ws.pack_tiles_all);
        ntiles = plan->ws.n_pack_tiles_all;
    } else {
        tiles = reinterpret_cast<const Tile *>(ws + plan->ws.pack_tiles_rank) + plan->rank_tile_off[rank];
        ntiles = plan->rank_tile_off[rank + 1] - plan->rank_tile_off[rank];
    }
    if (ntiles == 0) return FS_OK;
    if (ntiles > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_pack_cast: too many tiles for one launch");
    (void)hipGetLastError();
    const uint32_t lds = lds_cap(kCastWgsPerCu, ntiles, (int64_t)sizeof(TileLds));
    hipLaunchKernelGGL(pack_cast_kernel, dim3((uint32_t)ntiles), dim3(kThreads), lds, stream, segs, tiles, params,
                       static_cast<char *>(out), lo, hi);
    return check_launch("fs_pack_cast");
}

extern "C" int fs_adamw_step(int64_t n, float *master, float *exp_avg, float *exp_avg_sq, const void *grad,
                             fs_dtype grad_dtype, uint16_t *param_bf16, const fs_adamw_hparams_t *hp,
                             hipStream_t stream) {
    fsi::clear_error();
    if (n < 0) return fsi::fail(FS_E_INVAL, "fs_adamw_step: n < 0");
    if (int rc = check_hparams("fs_adamw_step", hp)) return rc;
    if (grad_dtype != FS_BF16 && grad_dtype != FS_FP32) return fsi::fail(FS_E_DTYPE, "fs_adamw_step: unknown grad dtype");
    int64_t nb;
    if (__builtin_mul_overflow(n, (int64_t)4, &nb)) return fsi::fail(FS_E_OVERFLOW, "fs_adamw_step: n too large");
    if (n == 0) return FS_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad) return fsi::fail(FS_E_INVAL, "fs_adamw_step: NULL pointer");
    const int gb = grad_dtype == FS_BF16 ? 2 : 4;
    if (misaligned(master, 4) || misaligned(exp_avg, 4) || misaligned(exp_avg_sq, 4) || misaligned(grad, gb) ||
        (param_bf16 && misaligned(param_bf16, 2)))
        return fsi::fail(FS_E_ALIGN, "fs_adamw_step: pointer not aligned to its element size");
    {
        const void *arr[5] = {master, exp_avg, exp_avg_sq, grad, param_bf16};
        const int64_t len[5] = {nb, nb, nb, n * gb, param_bf16 ? 2 * n : 0};
        static const char *const name[5] = {"master", "exp_avg", "exp_avg_sq", "grad", "param_bf16"};
        const int i = first_overlap(arr, len, 5);
        if (i >= 0) return fsi::fail(FS_E_INVAL, "fs_adamw_step: %s overlaps another array", name[i]);
    }
    const AdamConsts c = adam_consts(*hp);
    const bool aligned = !misaligned(master, 16) && !misaligned(exp_avg, 16) && !misaligned(exp_avg_sq, 16) &&
                         !misaligned(grad, 16) && !(param_bf16 && misaligned(param_bf16, 16));
    if (!grid_fits(n)) return fsi::fail(FS_E_OVERFLOW, "fs_adamw_step: n too large for one launch");
    (void)hipGetLastError();
    const uint32_t lds = aligned ? lds_cap(kAdamWgsPerCu, (n + kAdamRow - 1) / kAdamRow) : 0;
    for (int64_t off = 0; off < n; off += kAdamSpan) {
        const int64_t len = std::min(kAdamSpan, n - off);
        float *th = master + off, *m = exp_avg + off, *v = exp_avg_sq + off;
        const void *g = static_cast<const char *>(grad) + off * gb;
        uint16_t *p16 = param_bf16 ? param_bf16 + off : nullptr;
        if (aligned) {
            const dim3 grid((uint32_t)((len + kAdamRow - 1) / kAdamRow)), b(kAdamThreads);
            with_flags(grad_dtype == FS_BF16, p16 != nullptr, [&](auto grad_bf16, auto has_p16) {
                hipLaunchKernelGGL((adamw_kernel<decltype(grad_bf16)::value, decltype(has_p16)::value>), grid, b, lds,
                                   stream, th, m, v, g, p16, c, len);
            });
        } else {
            hipLaunchKernelGGL(adamw_scalar_kernel, dim3((uint32_t)((len + kThreads - 1) / kThreads)), dim3(kThreads),
                               0, stream, len, th, m, v, g, (int)(grad_dtype == FS_BF16), p16, c);
        }
        if (int rc = check_launch("fs_adamw_step")) return rc;
    }
    return FS_OK;
}

namespace {

// ------------------------------------------------------ no-allocation scratch --
//
// fs_reduce_adamw_step_noalloc keeps the partial sums of a step with more
// than kTermsPerPass terms in this file-scope device array instead of a
// caller-supplied buffer, so it allocates nothing.  Every GPU the library
// runs on holds its own copy (64 MiB) until the process ends, and every call
// on that GPU shares it: the first reduce pass writes all n partial sums
// before any is read, so nothing needs clearing, and calls that overlap on
// one GPU (two streams at once) race.  In host code the array's name is not
// a device address: its per-device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr int64_t kScratchBytes = 64ll << 20;
constexpr int64_t kScratchFloats = kScratchBytes / (int64_t)sizeof(float);
static __device__ __align__(256) float scratch[kScratchFloats];
static_assert(kScratchFloats == FS_NOALLOC_MAX_NUMEL, "the header states the scratch capacity");

int scratch_on_current_device(const char *what, float **out) {
    static std::mutex mu;
    static std::vector<float *> by_device;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fsi::fail(FS_E_HIP, "%s: no current device", what);
    std::lock_guard<std::mutex> lock(mu);
    if ((int)by_device.size() <= dev) by_device.resize((size_t)dev + 1, nullptr);
    if (!by_device[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fsi::fail(FS_E_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", what, dev,
                             hipGetErrorString(e));
        by_device[dev] = static_cast<float *>(ptr);
    }
    *out = by_device[dev];
    return FS_OK;
}

// The fused step behind both entry points.  More than kTermsPerPass terms
// run as plain reduce passes that leave partial sums in `partial`
// (fs_reduce_adamw_step: the caller's grad_out; the no-allocation variant:
// the library's scratch array, obtained only when it is needed).
int reduce_adamw_impl(const char *what, int64_t n, int32_t world, int32_t grad_acc, const uint16_t *const *slices,
                      float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_bf16, float *grad_out,
                      bool static_partial, const fs_adamw_hparams_t *hp, hipStream_t stream) {
    if (n < 0) return fsi::fail(FS_E_INVAL, "%s: n < 0", what);
    if (world < 1 || grad_acc < 1)
        return fsi::fail(FS_E_INVAL, "%s: world and grad_acc must be >= 1", what);
    if (int rc = check_hparams(what, hp)) return rc;
    int64_t terms64, bytes_in, bytes_out;
    if (__builtin_mul_overflow((int64_t)world, (int64_t)grad_acc, &terms64) || terms64 > (1 << 20))
        return fsi::fail(FS_E_OVERFLOW, "%s: too many terms", what);
    if (__builtin_mul_overflow(n, (int64_t)2, &bytes_in) || __builtin_mul_overflow(n, (int64_t)4, &bytes_out))
        return fsi::fail(FS_E_OVERFLOW, "%s: n too large", what);
    if (n == 0) return FS_OK;
    const int terms = (int)terms64;
    if (!slices || !master || !exp_avg || !exp_avg_sq)
        return fsi::fail(FS_E_INVAL, "%s: NULL pointer", what);
    const bool multi_pass = terms > kTermsPerPass;
    if (multi_pass && static_partial && n > kScratchFloats)
        return fsi::fail(FS_E_OVERFLOW, "%s: more than %d terms keep partial sums in the library's scratch "
                         "array, which holds %lld elements (n = %lld)", what, kTermsPerPass,
                         (long long)kScratchFloats, (long long)n);
    if (multi_pass && !static_partial && !grad_out)
        return fsi::fail(FS_E_INVAL, "%s: more than %d terms need grad_out for the partial sums", what,
                         kTermsPerPass);
    if (misaligned(master, 4) || misaligned(exp_avg, 4) || misaligned(exp_avg_sq, 4) ||
        (grad_out && misaligned(grad_out, 4)) || (param_bf16 && misaligned(param_bf16, 2)))
        return fsi::fail(FS_E_ALIGN, "%s: pointer not aligned to its element size", what);
    bool aligned = !misaligned(master, 16) && !misaligned(exp_avg, 16) && !misaligned(exp_avg_sq, 16) &&
                   !(grad_out && misaligned(grad_out, 16)) && !(param_bf16 && misaligned(param_bf16, 16));
    const void *outs[5] = {master, exp_avg, exp_avg_sq, grad_out, param_bf16};
    const int64_t out_bytes[5] = {bytes_out, bytes_out, bytes_out, grad_out ? bytes_out : 0,
                                  param_bf16 ? bytes_in : 0};
    {
        static const char *const name[5] = {"master", "exp_avg", "exp_avg_sq", "grad_out", "param_bf16"};
        const int i = first_overlap(outs, out_bytes, 5);
        if (i >= 0) return fsi::fail(FS_E_INVAL, "%s: %s overlaps another output", what, name[i]);
    }
    for (int t = 0; t < terms; ++t) {
        if (!slices[t]) return fsi::fail(FS_E_INVAL, "%s: slice %d is NULL", what, t);
        if (misaligned(slices[t], 2))
            return fsi::fail(FS_E_ALIGN, "%s: slice %d not 2-byte aligned", what, t);
        if (misaligned(slices[t], 16)) aligned = false;
        for (int o = 0; o < 5; ++o)
            if (ranges_overlap(slices[t], bytes_in, outs[o], out_bytes[o]))
                return fsi::fail(FS_E_INVAL, "%s: an output overlaps slice %d", what, t);
    }
    const AdamConsts c = adam_consts(*hp);
    if (!grid_fits(n)) return fsi::fail(FS_E_OVERFLOW, "%s: n too large for one launch", what);
    float *partial = grad_out;
    if (multi_pass && static_partial)
        if (int rc = scratch_on_current_device(what, &partial)) return rc;
    // terms before the last kTermsPerPass: plain reduce passes leave partial sums in `partial`
    const int last_cnt = terms - (terms - 1) / kTermsPerPass * kTermsPerPass;
    const int t_last = terms - last_cnt;
    (void)hipGetLastError();
    const int first = t_last == 0;
    for (int64_t off = 0; off < n; off += kSpan) {
        const int64_t len = std::min(kSpan, n - off);
        for (int t0 = 0; t0 < t_last; t0 += kTermsPerPass)
            launch_reduce_pass(n, off, len, stream, slices, t0, kTermsPerPass, t0 == 0, 0, (float)world, aligned,
                               partial);
        SliceArgs sa;
        memset(&sa, 0, sizeof sa);
        for (int k = 0; k < last_cnt; ++k) sa.p[k] = slices[t_last + k] + off;
        float *th = master + off, *m = exp_avg + off, *v = exp_avg_sq + off;
        uint16_t *p16 = param_bf16 ? param_bf16 + off : nullptr;
        const float *part = partial ? partial + off : nullptr;
        float *gout = grad_out ? grad_out + off : nullptr;
        if (aligned) {
            if (last_cnt <= kFusedDeepTerms)
                launch_fused<kFusedGroupsFew, 4>(len, stream, sa, last_cnt, first, (float)world, th, m, v, p16, part,
                                                 gout, c);
            else if (last_cnt <= kRedFewTerms)
                launch_fused<kFusedGroupsFew, 1>(len, stream, sa, last_cnt, first, (float)world, th, m, v, p16, part,
                                                 gout, c);
            else
                launch_fused<kFusedGroupsMany, 2>(len, stream, sa, last_cnt, first, (float)world, th, m, v, p16, part,
                                                  gout, c);
        } else {
            const int64_t grid = std::max<int64_t>(1, ((len >> 3) + kThreads - 1) / kThreads);
            hipLaunchKernelGGL(reduce_adamw_general_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, sa,
                               last_cnt, first, (float)world, len, th, m, v, p16, part, gout, c);
        }
        if (int rc = check_launch(what)) return rc;
    }
    return FS_OK;
}

}  // namespace

extern "C" int fs_reduce_adamw_step(int64_t n, int32_t world, int32_t grad_acc, const uint16_t *const *slices,
                                    float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_bf16,
                                    float *grad_out, const fs_adamw_hparams_t *hp, hipStream_t stream) {
    fsi::clear_error();
    return reduce_adamw_impl("fs_reduce_adamw_step", n, world, grad_acc, slices, master, exp_avg, exp_avg_sq,
                             param_bf16, grad_out, false, hp, stream);
}

extern "C" int fs_reduce_adamw_step_noalloc(int64_t n, int32_t world, int32_t grad_acc,
                                            const uint16_t *const *slices, float *master, float *exp_avg,
                                            float *exp_avg_sq, uint16_t *param_bf16, const fs_adamw_hparams_t *hp,
                                            hipStream_t stream) {
    fsi::clear_error();
    return reduce_adamw_impl("fs_reduce_adamw_step_noalloc", n, world, grad_acc, slices, master, exp_avg,
                             exp_avg_sq, param_bf16, nullptr, true, hp, stream);
}

extern "C" int fs_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    fsi::clear_error();
    if (bytes < 0 || (bytes & 15)) return fsi::fail(FS_E_INVAL, "fs_stream_read: bytes must be a multiple of 16");
    if (bytes == 0) return FS_OK;
    if (!src || !sink) return fsi::fail(FS_E_INVAL, "fs_stream_read: NULL pointer");
    if (misaligned(src, 16) || misaligned(sink, 4)) return fsi::fail(FS_E_ALIGN, "fs_stream_read: misaligned pointer");
    const int64_t nvec = bytes / 16;
    const int64_t grid = (nvec + kStreamVecs * kThreads - 1) / (kStreamVecs * kThreads);
    if (grid > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_stream_read: too large for one launch");
    (void)hipGetLastError();
    hipLaunchKernelGGL(read_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream, static_cast<const char *>(src),
                       nvec, sink);
    return check_launch("fs_stream_read");
}

extern "C" int fs_stream_fill(void *dst, int64_t bytes, uint32_t value, hipStream_t stream) {
    fsi::clear_error();
    if (bytes < 0 || (bytes & 15)) return fsi::fail(FS_E_INVAL, "fs_stream_fill: bytes must be a multiple of 16");
    if (bytes == 0) return FS_OK;
    if (!dst) return fsi::fail(FS_E_INVAL, "fs_stream_fill: NULL pointer");
    if (misaligned(dst, 16)) return fsi::fail(FS_E_ALIGN, "fs_stream_fill: dst must be 16-byte aligned");
    const int64_t nvec = bytes / 16;
    const int64_t grid = (nvec + kStreamVecs * kThreads - 1) / (kStreamVecs * kThreads);
    if (grid > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_stream_fill: too large for one launch");
    (void)hipGetLastError();
    hipLaunchKernelGGL(fill_kernel, dim3((uint32_t)grid), dim3(kThreads), lds_cap(kFillWgsPerCu, grid), stream,
                       static_cast<char *>(dst), nvec, value);
    return check_launch("fs_stream_fill");
}

extern "C" int fs_copy_bytes(void *dst, const void *src, int64_t bytes, hipStream_t stream) {
    fsi::clear_error();
    if (bytes < 0 || (bytes & 15)) return fsi::fail(FS_E_INVAL, "fs_copy_bytes: bytes must be a multiple of 16");
    if (bytes == 0) return FS_OK;
    if (!dst || !src) return fsi::fail(FS_E_INVAL, "fs_copy_bytes: NULL pointer");
    if (misaligned(dst, 16) || misaligned(src, 16)) return fsi::fail(FS_E_ALIGN, "fs_copy_bytes: pointers must be 16-byte aligned");
    if (ranges_overlap(dst, bytes, src, bytes)) return fsi::fail(FS_E_INVAL, "fs_copy_bytes: ranges overlap");
    const int64_t nvec = bytes / 16;
    const int64_t grid = (nvec + kCopyThreads - 1) / kCopyThreads;
    if (grid > INT32_MAX) return fsi::fail(FS_E_OVERFLOW, "fs_copy_bytes: too large for one launch");
    (void)hipGetLastError();
    hipLaunchKernelGGL(copy_kernel, dim3((uint32_t)grid), dim3(kCopyThreads), 0, stream, static_cast<char *>(dst),
                       static_cast<const char *>(src), nvec);
    return check_launch("fs_copy_bytes");
}
