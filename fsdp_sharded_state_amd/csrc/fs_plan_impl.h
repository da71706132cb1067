// fs_plan_impl.h -- the plan object behind the opaque fs_plan_t, shared by
// the host planner (fs_plan.cpp) and the launchers (fs_kernels.hip).
#pragma once
#include <stdarg.h>
#include <stdint.h>

#include <vector>

#include "../../include/fs.h"
#include "fs_internal.h"

struct fs_plan_s {
    fs_plan_info_t info;
    int vec;                                   // elements per 16-byte block: 8 (bf16) or 4 (fp32)
    std::vector<fs_param_layout_t> params;
    std::vector<fsi::Segment> pack_segs;       // gathered order
    std::vector<fsi::Segment> unpack_segs;     // parameter order
    std::vector<fsi::Tile> pack_tiles_all;
    std::vector<fsi::Tile> pack_tiles_rank;
    std::vector<int64_t> rank_tile_off;        // N+1 offsets into pack_tiles_rank
    std::vector<fsi::Tile> unpack_tiles;
    std::vector<fsi::BufInfo> bufinfo;
    std::vector<int64_t> local_first;          // [N][n_params]: src_off of parameter i's run on rank r (0 if none)
    fsi::WorkspaceLayout ws;
    void *dev_ws = nullptr;                    // bound by fs_plan_upload
    int dev_id = -1;                           // device of dev_ws
};

// Relayout of one group's gathered buffer from one plan to another (other N,
// other mode): segments in destination-gathered order whose source offsets
// index the source plan's gathered buffer, and a tile index over the
// destination.
struct fs_reshard_s {
    int32_t elem_bytes = 0;
    int vec = 0;
    int64_t src_gathered = 0, dst_gathered = 0;
    std::vector<fsi::Segment> segs;
    std::vector<fsi::Tile> tiles;
    int64_t ws_segs = 0, ws_tiles = 0, ws_bytes = 0;
    void *dev_ws = nullptr;                    // bound by fs_reshard_upload
    int dev_id = -1;
};

namespace fsi {
// Record a message for fs_last_error() and return `code`.
int fail(int code, const char *fmt, ...);
void clear_error();
// Tile a sorted, non-overlapping segment list (see fs_plan.cpp).
void build_tiles(const std::vector<Segment> &segs, int64_t lo, int64_t hi, int vec, int tile_blocks,
                 std::vector<Tile> &out);
}  // namespace fsi
