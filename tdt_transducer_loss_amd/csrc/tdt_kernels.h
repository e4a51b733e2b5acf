// Kernel launchers of the gfx950 TDT loss, shared by the host entry points.
#pragma once

#include "tdt_common.h"

namespace tdt {

// Duration logit at element offset `off` of the duration view, widened exactly to float.
__device__ __forceinline__ float load_dur(const Params& p, int64_t off) {
  if (p.dtype == 0) return F32::load(p.dur, off);
  if (p.dtype == 1) return F16::load(p.dur, off);
  return BF16::load(p.dur, off);
}

// Token logit at element offset `off` of the token view, widened exactly to float.
__device__ __forceinline__ float load_tok(const Params& p, int64_t off) {
  if (p.dtype == 0) return F32::load(p.tok, off);
  if (p.dtype == 1) return F16::load(p.tok, off);
  return BF16::load(p.tok, off);
}

// which: 0 row statistics, 1 gradient pass
hipError_t launch_rows_f32(const Params& p, bool aligned, hipStream_t st, int which);
hipError_t launch_rows_f16(const Params& p, bool aligned, hipStream_t st, int which);
hipError_t launch_rows_bf16(const Params& p, bool aligned, hipStream_t st, int which);
// which: 0 node weights, 1 lattice, 2 coefficients + loss (long rows), 3 loss only
hipError_t launch_lattice_side(const Params& p, int which, hipStream_t st);

}  // namespace tdt
