// Optional check of the selected-block indices handed to bsattn_forward (enabled by the
// environment variable BSATTN_VALIDATE=1): every row must hold topk values in [0, nkb) (the key
// blocks: nb, or more when key blocks overlap), strictly ascending. The attention kernels themselves only guard against out-of-range values (such a
// row's output becomes NaN); duplicates or a wrong order would silently change the result.
// The failing-row counter lives in memory the caller hands in (the first four bytes of the
// attention's output, which the attention launch overwrites afterwards): the library keeps no
// device state between calls.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

__global__ void reset_kernel(unsigned int* counter) { *counter = 0u; }

// one thread per row; causal rows (query block i = row index mod nb) use min(topk, i+1)
// places with values in [0, i] and hold -1 in the others
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ idx,
                                                       int64_t rows, int topk, int nb,
                                                       int nkb, bool causal,
                                                       unsigned int* counter) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int i = (int)(r % nb);
  const int used = causal && i + 1 < topk ? i + 1 : topk;
  const int lim = causal ? i + 1 : nkb;
  const int32_t* row = idx + r * topk;
  bool ok = true;
  int prev = -1;
  for (int j = 0; j < used; ++j) {
    const int x = row[j];
    ok &= x > prev && x < lim;
    prev = x;
  }
  for (int j = used; j < topk; ++j) ok &= row[j] == -1;
  if (!ok) atomicAdd(counter, 1u);
}

}  // namespace

hipError_t validate_idx(int64_t rows, int topk, int nb, int nkb, const int32_t* idx,
                        bool causal, unsigned int* counter, hipStream_t stream,
                        unsigned int* bad_rows) {
  *bad_rows = 0;
  if (rows == 0) return hipSuccess;
  reset_kernel<<<1, 1, 0, stream>>>(counter);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  validate_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, stream>>>(idx, rows, topk, nb,
                                                                      nkb, causal, counter);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(bad_rows, counter, sizeof(unsigned int), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace bsattn
