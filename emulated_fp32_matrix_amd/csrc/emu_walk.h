// A workgroup's walk over its static list of (output tile, k-step)
// positions, shared by the persistent GEMM kernels whose two wave groups take
// turns (gfx950 only).
#pragma once

#include "emu_tile.h"

namespace emu {

// A position (item, k-step) in a workgroup's static sequence.  An item is a
// whole output tile or, in a launch with a split K, one K segment of a split
// tile; the workgroup's items are i0, i0 + G, i0 + 2G, ...  Without a split
// each advance adds G tiles (n fastest) as G / tiles_n tile rows and
// G % tiles_n columns, without divisions.  Past the last step it stays put
// (prefetches re-read valid data).
struct Walk {
    int kt;          // k-step (of the whole K)
    int kt_end;      // one past the item's last k-step
    int seg;         // K segment
    int tn;          // tile column
    int left;        // items after this one
    int64_t m0;      // first row
    int64_t arow;    // m0 * lda (element offset of the tile's first A row)
    int rows;        // rows of the tile inside op(A): min(M - m0, th)
    int kvalid;      // k of this step inside op(A): min(K - 32 kt, 32)
    int item;        // (split launch) the item's number in the launch's list
    int part;        // (split launch) the item is one K segment of a split tile
    int widx;        // (split launch, part) its slot in the workspace of partial results
};

// The item a finished step belonged to (what the epilogue needs of a Walk).
struct TilePos {
    int64_t m0;
    int tn, rows, seg, part, widx;
};

struct WalkConst {
    int nk, nk_item, tiles_n, gtn, tail_k;   // tail_k: valid k of the last step
    int th;                      // rows of an output tile
    int G;                       // workgroups of the launch (items added per advance)
    // (split launch) items [0, split_from) are whole tiles 0 .. split_from-1;
    // item split_from + j is segment j / nsplit of tile split_from + j % nsplit
    int split_from, nsplit;
    int64_t gm, M, lda;          // gm: rows added per advance
};

__device__ __forceinline__ void walk_set_tile(Walk& w, const WalkConst& c)
{
    w.arow = w.m0 * c.lda;
    const int64_t r = c.M - w.m0;
    w.rows = r < c.th ? (int)r : c.th;
}

// (split launch) w at item number it of the launch's list: a whole tile
// (k-steps 0 .. nk-1) or one K segment of a split tile.  Divisions: once per
// item.
__device__ __forceinline__ void walk_set_item(Walk& w, const WalkConst& c, int it)
{
    w.item = it;
    int tile;
    if (it < c.split_from) {
        tile = it;
        w.seg = 0;
        w.part = 0;
        w.widx = 0;
        w.kt = 0;
        w.kt_end = c.nk;
    } else {
        const int j = it - c.split_from;
        w.seg = j / c.nsplit;
        tile = c.split_from + (j - w.seg * c.nsplit);
        w.part = 1;
        w.widx = j;
        w.kt = w.seg * c.nk_item;
        w.kt_end = w.kt + c.nk_item;
    }
    const int tm = tile / c.tiles_n;
    w.tn = tile - tm * c.tiles_n;
    w.m0 = (int64_t)tm * c.th;
    walk_set_tile(w, c);
}

// SPLIT: the launch's items include K segments of split tiles (otherwise
// every item is a whole tile and the walk advances without divisions).
template <bool SPLIT>
__device__ __forceinline__ void walk_next(Walk& w, const WalkConst& c)
{
    if (w.kt + 1 < (SPLIT ? w.kt_end : c.nk)) {
        ++w.kt;
    } else if (w.left > 0) {
        --w.left;
        if constexpr (SPLIT) {
            walk_set_item(w, c, w.item + c.G);
        } else {
            w.tn += c.gtn;
            w.m0 += c.gm;
            if (w.tn >= c.tiles_n) {
                w.tn -= c.tiles_n;
                w.m0 += c.th;
            }
            w.kt = 0;
            walk_set_tile(w, c);
        }
    }
    w.kvalid = w.kt + 1 < c.nk ? BK : c.tail_k;
}

}  // namespace emu
