// Dispatch size limit shared by the launchers and the C ABI front end.
#pragma once

#include <stdint.h>

namespace mxg {

// One dispatch runs fewer than 2^32 work-items: the dispatch packet holds the
// grid size in 32 bits.  Each launcher has a *_grid_items function giving the
// work-items of the dispatch it would make, by the formula the launcher itself
// uses; the C ABI rejects a request above the limit before any HIP call, so a
// grid is never cut short, and the launchers check it again.
constexpr int64_t kMaxGridItems = ((int64_t)1 << 32) - 1;

// layout: kLayoutRows (one lane per 32-element block) or kLayoutTiled (the
// resident workgroups walk the chunks)
int64_t quantize_grid_items(int64_t rows, int64_t k, int layout);
// one workgroup of 64 * waves lanes per output tile
inline int64_t gemm_grid_items(int64_t tiles_m, int64_t tiles_n, int waves) { return tiles_m * tiles_n * 64 * waves; }
// one workgroup per two 32-feature weight groups
int64_t splitk_grid_items(int64_t n);
// src_type: kSrcBf16 or kSrcF32 (they take different kernels)
int64_t rmsnorm_quantize_grid_items(int64_t rows, int64_t d, int src_type);

}  // namespace mxg
