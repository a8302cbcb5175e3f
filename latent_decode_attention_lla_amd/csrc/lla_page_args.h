// Paged latent cache: launch arguments shared by the C ABI and the kernels that read or
// write a cache stored in pages.
#pragma once

#include <stdint.h>

namespace lla {

constexpr int kPage = 16;  // tokens per page (one 16-token tile of the decode kernels)
// Pages of one context split that the wide fold kernel keeps in LDS; the planner keeps
// paged splits of that kernel within it.
constexpr int kMaxSplitPages = 256;

// A layer's pool is [num_pages][Hc][kPage][r]; logical token j of sequence b lives in row
// j % kPage of page table[b * max_blocks + j / kPage]. A null table means the dense layout.
struct PageArgs {
  const int32_t* table;
  int max_blocks;
  int num_pages;  // page indices are clamped into [0, num_pages) before use
};

__device__ __forceinline__ int page_of(const PageArgs& pg, int b, int logical_page) {
  const int p = pg.table[static_cast<size_t>(b) * pg.max_blocks + logical_page];
  return min(max(p, 0), pg.num_pages - 1);
}

}  // namespace lla
