// A workgroup's walk over its static list of (output tile, k-step)
// positions, shared by the persistent GEMM kernels whose two wave groups take
// turns (gfx950 only).
#pragma once

#include "emu_tile.h"

namespace emu {

// A position (item, k-step) in a workgroup's static sequence, advanced
// without divisions.  An item is one K segment of one output tile; items
// are numbered seg * ntiles + tile (tiles n fastest), and the workgroup's
// items are i0, i0 + G, i0 + 2G, ..., so each advance adds G / ntiles
// segments and G % ntiles tiles, the latter as tile rows and columns.  Past
// the last step it stays put (prefetches re-read valid data).
struct Walk {
    int kt;          // k-step (of the whole K)
    int kt_end;      // one past the segment's last k-step
    int seg;         // K segment
    int tn;          // tile column
    int left;        // items after this one
    int64_t m0;      // first row
    int64_t arow;    // m0 * lda (element offset of the tile's first A row)
    int rows;        // rows of the tile inside op(A): min(M - m0, th)
    int kvalid;      // k of this step inside op(A): min(K - 32 kt, 32)
};

// The item a finished step belonged to (what the epilogue needs of a Walk).
struct TilePos {
    int64_t m0;
    int tn, rows, seg;
};

struct WalkConst {
    int nk, nk_item, tiles_n, gtn, gseg, tail_k;   // tail_k: valid k of the last step
    int th;                      // rows of an output tile
    int64_t gm, mrows, M, lda;   // gm: rows added per advance; mrows: tiles_m * th
};

__device__ __forceinline__ void walk_set_tile(Walk& w, const WalkConst& c)
{
    w.arow = w.m0 * c.lda;
    const int64_t r = c.M - w.m0;
    w.rows = r < c.th ? (int)r : c.th;
}

__device__ __forceinline__ void walk_start_segment(Walk& w, const WalkConst& c)
{
    w.kt = w.seg * c.nk_item;
    w.kt_end = w.kt + c.nk_item;
}

// SPLIT: K is split into segments (otherwise seg stays 0, kt_end = nk and
// the segment bookkeeping compiles away).
template <bool SPLIT>
__device__ __forceinline__ void walk_next(Walk& w, const WalkConst& c)
{
    if (w.kt + 1 < (SPLIT ? w.kt_end : c.nk)) {
        ++w.kt;
    } else if (w.left > 0) {
        --w.left;
        w.tn += c.gtn;
        w.m0 += c.gm;
        if (w.tn >= c.tiles_n) {
            w.tn -= c.tiles_n;
            w.m0 += c.th;
        }
        if constexpr (SPLIT) {
            w.seg += c.gseg;
            if (w.m0 >= c.mrows) {
                w.m0 -= c.mrows;
                ++w.seg;
            }
            walk_start_segment(w, c);
        } else {
            w.kt = 0;
        }
        walk_set_tile(w, c);
    }
    w.kvalid = w.kt + 1 < c.nk ? BK : c.tail_k;
}

}  // namespace emu
