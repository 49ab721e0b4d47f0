// GPU check of the hardware fp32 -> e4m3 conversion (test infrastructure).
//
// The cache-append kernel rounds with v_cvt_pk_fp8_f32 after clamping every
// value to [-448, 448].  This kernel converts every fp32 value in [0, 448]
// and its negation with that instruction and compares the codes with a plain
// encoder written from the OCP e4m3 ("fn") definition: round to nearest,
// ties to the even code, k * 2^-9 steps below 2^-6.  Mismatches are counted;
// the first 16 inputs that mismatch are recorded.  Reads nothing, writes only
// the two result buffers (the record index is bounds-checked).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ uint32_t plain_e4m3(float a) {   // a in [0, 448]
  if (a < 0.015625f) return uint32_t(__builtin_rintf(a * 512.f));
  const uint32_t v = __float_as_uint(a), m = v & 0x7FFFFFu;
  uint32_t code = (((v >> 23) - 120u) << 3) | (m >> 20);
  const uint32_t rest = m & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ++code;
  return code;
}

__global__ void e4m3_convert_check_kernel(uint32_t n, unsigned long long* bad, uint32_t* first) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < n; u += stride) {
    const float f = __uint_as_float(u);
    const uint32_t hw = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(f, -f, 0, false));
    const uint32_t want = plain_e4m3(f);
    if ((hw & 0xFFu) != want || ((hw >> 8) & 0xFFu) != (want | 0x80u)) {
      const unsigned long long k = atomicAdd(bad, 1ull);
      if (k < 16ull) first[k] = u;
    }
  }
}

}  // namespace

// Counts into bad[0] (zeroed by the caller) the fp32 values in [0, 448]
// whose conversion (or that of their negation) differs; first[16] receives
// the first mismatching inputs.  Returns 0, or the HIP error of the launch.
extern "C" int e4m3_convert_check(unsigned long long* bad, uint32_t* first, void* stream) {
  const uint32_t n = 0x43E00001u;   // bit patterns of +0 .. 448
  hipLaunchKernelGGL(e4m3_convert_check_kernel, dim3(4096), dim3(256), 0,
                     static_cast<hipStream_t>(stream), n, bad, first);
  return int(hipGetLastError());
}
