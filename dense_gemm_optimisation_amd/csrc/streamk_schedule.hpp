// The stream-K partition of a tile grid: which (tile, k step) iterations each
// workgroup computes, where it leaves a partial tile and which pieces the
// fix-up adds.  One copy of this arithmetic serves the three stream-K
// kernels, their fix-up kernels, the host code that sizes their workspace and
// the CPU test of the partition.
//
// Persistent kernels and Stream-K are named in section 12.5 of "CUDA GEMM
// 矩阵乘法优化指南" (blog.zhenwei.site) without fixing how partial tiles are
// combined; the reading taken here is a static split with a separate fix-up:
//   * G workgroups run; the first dp_tiles = floor(T / G) * G tiles fill
//     whole waves and are computed whole, tile w + n*G by workgroup w;
//   * the W = (T - dp_tiles) * S iterations of the remaining tiles (S k steps
//     each) are split over Gs workgroups, workgroup w taking the contiguous
//     range [w*W/Gs, (w+1)*W/Gs);
//   * a piece that covers a whole tile goes through the normal epilogue; any
//     other is a partial tile, written to slot 2w (the piece that holds the
//     range's last iteration) or 2w + 1 (its first): only those two pieces
//     of a range can be partial;
//   * the fix-up of a cut tile adds the pieces of workgroups owner(first
//     iteration) .. owner(last iteration), lowest first, so the result does
//     not depend on the order the workgroups ran in.
#pragma once

#include <cstdint>

#if !defined(__HIPCC__)
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace libgemm {

struct StreamKSplit {
    int64_t steps;     // k steps per tile (S)
    int64_t dp_tiles;  // tiles computed whole (a multiple of the grid)
    int64_t iters;     // W = (tiles - dp_tiles) * S
    int64_t groups;    // Gs = workgroups sharing the W iterations (0 when W = 0)
};

// Workgroups that share the k steps of `cut` tiles of `steps` k steps each,
// out of G: cutting each tile into s pieces costs steps/s k steps of time and
// cut*s partial tiles written and read back; with one k step worth `ratio`
// partial tiles (the kernel's step time over the time to move one partial
// tile through HBM twice), s = sqrt(steps*ratio/cut) balances the two.
inline int64_t streamk_groups(int64_t G, int64_t cut, int64_t steps, double ratio) {
    const int64_t W = cut * steps;
    int64_t s = static_cast<int64_t>(__builtin_sqrt(double(steps) * ratio / double(cut)) + 0.5);
    s = s < 1 ? 1 : (s > steps ? steps : s);
    int64_t g = cut * s;
    g = g < G ? g : G;
    return g < W ? g : W;
}

// The split of `tiles` tiles of `steps` k steps each over G workgroups.
inline StreamKSplit streamk_split(int64_t tiles, int64_t steps, int64_t G, double ratio) {
    StreamKSplit s{};
    s.steps = steps;
    s.dp_tiles = tiles / G * G;
    s.iters = (tiles - s.dp_tiles) * steps;
    s.groups = s.iters == 0 ? 0 : streamk_groups(G, tiles - s.dp_tiles, steps, ratio);
    return s;
}

// Workgroups the main kernel launches (G when some tiles are whole, else Gs).
inline int64_t streamk_grid(const StreamKSplit &s, int64_t G) {
    return s.dp_tiles > 0 ? G : s.groups;
}

// Whole tiles workgroup w computes (w, w + G, ...).
__host__ __device__ inline int64_t sk_whole_tiles(const StreamKSplit &s, int64_t w, int64_t G) {
    return w < s.dp_tiles ? (s.dp_tiles - w + G - 1) / G : 0;
}

// Workgroup w's range of cut-tile iterations [sk_begin, sk_end).
__host__ __device__ inline int64_t sk_begin(const StreamKSplit &s, int64_t w) {
    return w < s.groups ? w * s.iters / s.groups : 0;
}
__host__ __device__ inline int64_t sk_end(const StreamKSplit &s, int64_t w) {
    return w < s.groups ? (w + 1) * s.iters / s.groups : 0;
}

// The piece a workgroup computes from iteration `it` of its range ending at
// `end`: k steps [kb, ke) of cut tile `local` (tile dp_tiles + local); the
// workgroup then continues from local*S + ke.
struct StreamKPiece {
    int64_t local, kb, ke;
};
__host__ __device__ inline StreamKPiece sk_piece(const StreamKSplit &s, int64_t local,
                                                 int64_t it, int64_t end) {
    StreamKPiece p;
    p.local = local;  // it / S, computed by the caller (kernels keep it in a scalar register)
    p.kb = it - local * s.steps;
    p.ke = end - local * s.steps < s.steps ? end - local * s.steps : s.steps;
    return p;
}

// Slot of the partial tile that workgroup w (range ending at `end`) leaves
// for cut tile `local`: 2w when its last iteration lies in that tile, else
// 2w + 1.
__host__ __device__ inline int64_t sk_slot(const StreamKSplit &s, int64_t w, int64_t local,
                                           int64_t end) {
    return 2 * w + (end - 1 < (local + 1) * s.steps ? 0 : 1);
}

// The workgroup whose range holds iteration x: the largest g with
// g*W/Gs <= x.
__host__ __device__ inline int64_t sk_owner(const StreamKSplit &s, int64_t x) {
    return ((x + 1) * s.groups - 1) / s.iters;
}

}  // namespace libgemm
