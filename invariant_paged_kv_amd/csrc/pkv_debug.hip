// pkv_debug.hip -- the debug-mode check kernel: the device-data preconditions
// of pkv_checks.h evaluated on the device, before the kernels of the call
// that reads that data (each of which returns at once when a violation was
// recorded).
#include "pkv_checks.h"
#include "pkv_internal.h"

namespace pkv {

// One thread per sequence.  word[0] collects the violation flags; word[1] the
// largest 0x7fffffff - b over bad sequences b (0: none), i.e. the lowest bad b.
// Vector (global) atomics: the word is read back by later kernels and the host.
__global__ __launch_bounds__(256) void check_kernel(CheckLimits l, const int32_t* cu, const int32_t* sk,
                                                    const int32_t* block_table, const int32_t* cu_k, int32_t* word) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= l.batch) return;
  const int32_t f = check_sequence(l, b, cu, sk, block_table, cu_k);
  if (f != 0) {
    atomicOr(&word[0], f);
    atomicMax(&word[1], 0x7fffffff - b);
  }
}

hipError_t launch_check(const CheckLimits& l, const int32_t* cu, const int32_t* sk, const int32_t* block_table,
                        const int32_t* cu_k, int32_t* word, hipStream_t stream) {
  (void)hipGetLastError();
  if (l.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_kernel, dim3((l.batch + 255) / 256), dim3(256), 0, stream, l, cu, sk, block_table, cu_k,
                     word);
  return hipGetLastError();
}

}  // namespace pkv
