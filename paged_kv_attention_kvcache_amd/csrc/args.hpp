// Constants and launch-argument types shared by the host code and the gfx950
// kernels. Plain C++ (no device code), so host-only translation units can
// include it with any C++ compiler.
#pragma once
#include <stdint.h>

namespace pkv {

constexpr int kPage = 16;              // tokens per page

// Early-exit decode ("latest bank"): position pos of request r is read from
// plane min(plane, depth[r * stride + pos]) of the query's layer instead of
// the query's own plane. Bank byte offsets relative to the query's bank:
// d0 for plane 0, d1 + (p - 1) * step for plane p >= 1 (the per-plane maps
// put a recurrent layer's banks of planes 1, 2, ... at a fixed distance).
struct LatestArgs {
  const uint8_t *depth;  // [batch][stride] exit depths, or null (ordinary decode)
  int32_t stride;        // a multiple of 16; rows are 16-byte aligned
  int32_t plane;         // the query's plane
  int64_t d0, d1, step;
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pkv
