// Device side of the seeded synthetic input generator: fills device buffers
// with the same bits as the host generator (same header, same definition).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "philox4x32.h"

template <bool BF16>
__global__ void __launch_bounds__(256) moegen_fill_kernel(void* out, uint64_t start, int64_t count,
                                                         uint32_t seed, uint32_t stream, double scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    float v = moegen_value_f32(start + (uint64_t)i, seed, stream, scale);
    if (BF16) static_cast<uint16_t*>(out)[i] = moegen_f32_to_bf16_rne(v);
    else static_cast<float*>(out)[i] = v;
  }
}

static int launch(bool bf16, void* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream,
                  double scale, void* hip_stream) {
  if (count < 0 || (count > 0 && out == nullptr)) return 1;
  if (count == 0) return 0;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (bf16) moegen_fill_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(out, start, count, seed, stream, scale);
  else moegen_fill_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(out, start, count, seed, stream, scale);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moegen_dev_fill_f32(float* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream,
                                   double scale, void* hip_stream) {
  return launch(false, out, start, count, seed, stream, scale, hip_stream);
}
extern "C" int moegen_dev_fill_bf16(uint16_t* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream,
                                    double scale, void* hip_stream) {
  return launch(true, out, start, count, seed, stream, scale, hip_stream);
}
