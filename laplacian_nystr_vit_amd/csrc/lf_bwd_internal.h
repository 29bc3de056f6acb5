// Host-side interface of the backward-pass kernels (lf_bwd.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#include "lf_internal.h"

namespace lf {

// Pointers into the buffer the forward pass filled (layout: lf_saved_layout).
struct SavedPtrs {
  const float *L, *CQ, *CK, *We, *xs, *mu, *rstd, *S, *P, *alpha;
};

// Backward workspace in bytes; 0 when the shape is outside what the backward kernels support (m or d > 64).
size_t bwd_ws_bytes(const Shape& s);

// Optional outputs of the training op beyond dQ, dK, dV.
struct BwdExtras {
  float* d_dwc_w = nullptr;   // [heads * d][3][3], summed over the batch
  float* d_lambda = nullptr;  // one float, summed over every slice
  bool exact_alpha = false;   // gradient through alpha instead of holding it constant
};

// aux: NULL keeps every launch on st; otherwise the independent parts run on aux->s (see lf_bwd.hip).
hipError_t launch_backward(const Shape& s, bool whiten, const void* Q, const void* K, const void* V, const float* w,
                           const SavedPtrs& sp, const void* dY, void* dQ, void* dK, void* dV, void* ws,
                           hipStream_t st, const BwdExtras& ex, const AuxStream* aux);

}  // namespace lf
