/*
 * copy_ceiling.hip -- libzscopy: the plain device copy that the benchmark
 * times beside the shard step, as the practical HBM ceiling of the part it
 * runs on. Measurement only: no step of the method runs here, and the
 * shard-step library does not use it.
 *
 * Shape: every lane moves one 16-byte vector (a non-temporal load, then a
 * plain store), so each 64-lane wave reads 1 KB and writes 1 KB. On MI355X
 * copies with 1-2 KB per wave streamed fastest (about 6.45 TB/s for read
 * plus write); wider bursts per wave and persistent grids were slower, and
 * the runtime's device-to-device memcpy reaches 4.6-5.2 TB/s.
 */
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kCopyBlock = 256;

thread_local const char *g_copy_err = "";

using f4 = float __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kCopyBlock)
copy_kernel(const f4 *__restrict__ src, f4 *__restrict__ dst, uint64_t nvec) {
  const uint64_t i = (uint64_t)blockIdx.x * kCopyBlock + threadIdx.x;
  if (i < nvec) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace

extern "C" {

/* Copies `bytes` bytes from device buffer src to device buffer dst on HIP
 * stream `stream` (NULL = the default stream); asynchronous, nothing is
 * allocated. Returns 0 when the launch was enqueued; 1 (nothing enqueued)
 * for a null pointer, a base that is not 16-byte aligned, a size that is
 * not a multiple of 16 or too large for one grid, or buffers that overlap;
 * 4 when the launch fails (zs_copy_last_error() has HIP's message).
 * bytes == 0 returns 0 and does nothing. */
int zs_copy_ceiling(const void *src, void *dst, uint64_t bytes, void *stream) {
  if (!src || !dst || (uintptr_t)src % 16 || (uintptr_t)dst % 16 || bytes % 16) return 1;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (bytes && s0 < d0 + bytes && d0 < s0 + bytes) return 1;
  const uint64_t nvec = bytes / 16;
  const uint64_t blocks = (nvec + kCopyBlock - 1) / kCopyBlock;
  if (blocks > 0x7fffffffull) return 1;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const f4 *>(src),
                     static_cast<f4 *>(dst), nvec);
  const hipError_t e = hipGetLastError();
  g_copy_err = e == hipSuccess ? "" : hipGetErrorString(e);
  return e == hipSuccess ? 0 : 4;
}

/* HIP's message for the last launch failure on this thread ("" after a
 * successful launch). */
const char *zs_copy_last_error(void) { return g_copy_err; }

}  // extern "C"
