/* Device side of the synthetic-input generator (definitions in synth_core.h):
 * fills device buffers with the same bits the host side produces, so that
 * multi-GiB weight sets need not cross PCIe. */
#include <hip/hip_runtime.h>
#include "synth_core.h"

__global__ void synth_normal_kernel(uint16_t* out, int64_t n, uint64_t key, int64_t offset,
                                    double mean, double std) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = synth_normal_elem(key, (uint64_t)(offset + i), mean, std);
}

__global__ void synth_tokens_kernel(int32_t* out, int64_t n, uint64_t key, int64_t offset,
                                    int32_t vocab) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = synth_token_elem(key, (uint64_t)(offset + i), vocab);
}

__global__ void synth_uniform_kernel(float* out, int64_t n, uint64_t key, int64_t offset) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = synth_uniform_elem(key, (uint64_t)(offset + i));
}

#include <stdio.h>

// A launch failure is reported as -2 with its reason on stderr.  Errors left
// behind by unrelated earlier runtime calls are cleared first.
static int launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return -2;
}

static int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" int synth_normal_bf16_dev(void* out, int64_t n, uint64_t seed, uint64_t tensor_id,
                                     int64_t offset, double mean, double std, void* stream) {
  if (n <= 0) return 0;
  if (!out) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(synth_normal_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)out, n, synth_key(seed, tensor_id), offset, mean, std);
  return launched("synth_normal_bf16_dev");
}

extern "C" int synth_tokens_dev(void* out, int64_t n, uint64_t seed, uint64_t tensor_id,
                                int64_t offset, int32_t vocab, void* stream) {
  if (n <= 0) return 0;
  if (!out || vocab <= 0) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(synth_tokens_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (int32_t*)out, n, synth_key(seed, tensor_id), offset, vocab);
  return launched("synth_tokens_dev");
}

extern "C" int synth_uniform_f32_dev(void* out, int64_t n, uint64_t seed, uint64_t tensor_id,
                                     int64_t offset, void* stream) {
  if (n <= 0) return 0;
  if (!out) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(synth_uniform_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (float*)out, n, synth_key(seed, tensor_id), offset);
  return launched("synth_uniform_f32_dev");
}
