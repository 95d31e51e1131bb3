// Host-visible launch interface of the gfx950 kernels.
#pragma once

#include "qg_device.hpp"

namespace qg {

// The similarity GEMM C = P~_new^T P~_old (r x r), split over the m rows.
struct CosArgs {
  const uint8_t* qa;
  const float* sa;
  const uint8_t* qb;
  const float* sb;
  int64_t m;
  int r;
  int tiles;     // output tiles per side (128 wide)
  int split;     // K splits
  int kslab;     // rows per split
  float* Cpart;  // split x r x r partial sums
};

// Scratch of the Newton-Schulz polar iteration on C.
struct CosWork {
  float* C;
  float* X;
  float* Xn;
  float* A;
  float* blocks;   // per-block partial sums
  int iters;
};

hipError_t launch_project(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_adam(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_backproject(const StepArgs& a, int grid, hipStream_t s);
hipError_t launch_quantize_int4(const float* P, int64_t numel, uint8_t* Pq, float* Ps,
                                hipStream_t s);
hipError_t launch_cossim(const CosArgs& c, const CosWork& w, float* out, hipStream_t s);

}  // namespace qg
