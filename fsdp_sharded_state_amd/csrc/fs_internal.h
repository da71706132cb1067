// fs_internal.h -- structures shared by the host planner (fs_plan.cpp) and
// the HIP kernels (fs_kernels.hip).  Not part of the public ABI.
//
// The planner lowers a layout into "copy segments" over a virtual element
// space and cuts that space into tiles:
//
//   * Pack (copy-in): the virtual space is the gathered buffer itself,
//     [0, N*shard).  A segment says: virtual elements [vx, vx+len) come from
//     parameter `buf`, elements [src_off, src_off+len).  Virtual elements not
//     covered by any segment are pads (written as zero).
//   * Unpack (copy-out): the virtual space concatenates the parameters, each
//     starting on a multiple of VEC elements (parameter j occupies
//     [vbase_j, vbase_j + numel_j)).  A segment says: virtual elements
//     [vx, vx+len) of parameter `buf` come from gathered elements
//     [src_off, src_off+len).
//
// Work unit: a "block" is VEC consecutive virtual elements (16 bytes of the
// destination).  A tile is a run of at most kTileBlocks blocks that overlaps
// at most kTileSegs segments; a workgroup stages its tile's segments in LDS.
#pragma once
#include <stdint.h>

namespace fsi {

// Tile sizes measured on the 7B model's 33 groups: every copy kernel (pack,
// unpack, reshard, local import) builds tiles of 8 KB of destination per
// workgroup (pack 16 KB: -4%, 4 KB: -3%; unpack 16 KB: -3%, 4 KB: -1%).  The
// kernels' per-thread loop has room for twice that: the same 8 KB tiles with
// a loop of two blocks per thread measured 3% slower on the unpack.
constexpr int kThreads = 256;                 // threads per workgroup (4 waves of 64)
constexpr int kBlocksPerThread = 4;           // loop capacity: 16-byte blocks per thread
constexpr int kTileBlocks = kThreads * kBlocksPerThread;      // largest tile a kernel accepts (16 KB)
constexpr int kCopyTileBlocks = kTileBlocks / 2;              // tiles the planner builds (8 KB of destination)
static_assert(kCopyTileBlocks <= kTileBlocks, "a tile must fit the kernel's per-thread loop");
constexpr int kTileSegs = 256;                // max segments staged in LDS per tile

struct Segment {        // 32 bytes, sorted by vx, non-overlapping, len > 0
    int64_t vx;         // first virtual (destination) element
    int64_t src_off;    // first source element
    int64_t len;        // elements
    int32_t buf;        // parameter index (pack: source; unpack: destination)
    int32_t rank;       // shard the gathered side lies in
};
static_assert(sizeof(Segment) == 32, "segment layout");

struct Tile {           // 40 bytes
    int64_t x_begin;    // virtual element of the tile's first block (multiple of VEC from its grid anchor)
    int64_t run_src;    // single-run tiles: source element of the tile's first element
    int64_t run_dst;    // single-run unpack tiles: destination element within parameter run_buf
    int32_t nblk;       // blocks in the tile (1..kTileBlocks)
    int32_t seg_lo;     // first overlapping segment
    int32_t nseg;       // overlapping segments (0..kTileSegs)
    int32_t run_buf;    // >= 0: every block of the tile lies inside one segment (of this buffer)
};
static_assert(sizeof(Tile) == 40, "tile layout");

struct BufInfo {        // unpack destinations: 16 bytes per parameter
    int64_t vbase;      // virtual element of the parameter's element 0 (multiple of VEC)
    int64_t numel;
};

// Offsets (bytes) of the tables inside the device workspace.
struct WorkspaceLayout {
    int64_t pack_segs, n_pack_segs;
    int64_t unpack_segs, n_unpack_segs;
    int64_t pack_tiles_all, n_pack_tiles_all;      // grid over [0, N*shard), anchored at 0 (may alias pack_tiles_rank)
    int64_t pack_tiles_rank, n_pack_tiles_rank;    // N grids over [r*shard, (r+1)*shard), anchored at r*shard
    int64_t unpack_tiles, n_unpack_tiles;
    int64_t bufinfo, n_bufinfo;
    int64_t local_first, n_local_first;            // [N][n_params]: first parameter element of each rank's run
    int64_t total_bytes;
};

}  // namespace fsi
