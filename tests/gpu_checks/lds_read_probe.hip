// LDS read throughput per CU (test infrastructure, a measurement aid).
//
// The decode kernels feed their matrix instructions from LDS with two read
// forms: 16-byte ds_read_b128 (key fragments) and ds_read_b64_tr_b16
// (transposed value fragments, 8 bytes per lane).  How many bytes per clock
// one CU's LDS delivers to them, with four or with eight waves reading at
// once, bounds how busy a kernel with two waves per SIMD can keep its matrix
// units.  This kernel measures it: one workgroup per CU fills a 64 KB LDS
// buffer, then every wave issues `iters` x 8 reads of one form back to back,
// in lane patterns without bank conflicts (contiguous 16-byte pieces; the
// decode kernels' transposed-read pattern).
//
// Bounds: every LDS address is below 40 KB of the 64 KB buffer and aligned to
// the read's width; the output holds exactly one word per thread of the grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_PTR(T) T __attribute__((address_space(3)))*

namespace {

constexpr int kBufBytes = 65536;

__device__ __forceinline__ uint32_t opaque_u(uint32_t x) {
  asm volatile("" : "=v"(x) : "0"(x));
  return x;
}

template <int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES, 1) void lds_read_probe_kernel(int iters, uint32_t* out) {
  __shared__ __attribute__((aligned(1024))) char buf[kBufBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kBufBytes / 4; i += 64 * WAVES)
    ((LDS_PTR(uint32_t))buf)[i] = uint32_t(i) * 2654435761u;
  __syncthreads();

  // A step's eight results are handed together to an empty asm statement,
  // which keeps the reads (eight in flight per wave) without any arithmetic
  // on them, so the loop is bound by the reads alone; the base alternates between two 32 KB halves, so every offset of
  // a step is an immediate and every address stays below 40 KB.
  uint32_t off = 0;
  if constexpr (MODE == 0) {
    // ds_read_b128: lane l reads bytes 16 l .. of a 1 KB run; 8 runs per step
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t base = uint32_t(lane * 16);
    for (int it = 0; it < iters; ++it) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const LDS_PTR(u32x4))(buf + base + off + u * 1024);
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
                   "v"(v[6]), "v"(v[7]));
      off = opaque_u(off ^ 32768u);
    }
  } else {
    // ds_read_b64_tr_b16 in the decode kernels' value-fragment pattern: lane
    // (g4 = l / 16, l16 = l % 16) names row 4 g4 + l16 / 4 of a 16-row tile
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const int l16 = lane & 15, g4 = lane >> 4;
    const int vr = 4 * g4 + (l16 >> 2), vrh = vr >> 3, vr8 = vr & 7, vx = (l16 & 3) >> 1;
    const uint32_t base = uint32_t(vrh * 1024 + 16 * (8 * (vx ^ vrh) + vr8) + 8 * (l16 & 1));
    for (int it = 0; it < iters; ++it) {
      bf16x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_PTR(bf16x4))(buf + base + off + 2048 * (u >> 2) + 256 * (u & 3)));
      asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
                   "v"(v[6]), "v"(v[7]));
      off = opaque_u(off ^ 32768u);
    }
  }
  const uint32_t acc = off;
  out[blockIdx.x * blockDim.x + tid] = acc;
}

template <int MODE>
int launch(int waves, int iters, int grid, uint32_t* out, hipStream_t s) {
  if (waves == 4)
    hipLaunchKernelGGL((lds_read_probe_kernel<4, MODE>), dim3(grid), dim3(256), 0, s, iters, out);
  else if (waves == 8)
    hipLaunchKernelGGL((lds_read_probe_kernel<8, MODE>), dim3(grid), dim3(512), 0, s, iters, out);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace

// One launch of `grid` workgroups of `waves` (4 or 8) waves, each wave
// issuing iters x 8 reads of form `mode` (0: ds_read_b128, 1 KB per read per
// wave; 1: ds_read_b64_tr_b16, 512 bytes).  `out` holds grid * waves * 64
// words.  Returns 0, or the HIP error of the launch (bad arguments: the
// invalid-value error, nothing launched).
extern "C" int lds_read_probe(int waves, int mode, int iters, int grid, uint32_t* out,
                              void* stream) {
  if (iters < 1 || grid < 1 || !out) return int(hipErrorInvalidValue);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return mode == 0 ? launch<0>(waves, iters, grid, out, s)
                   : mode == 1 ? launch<1>(waves, iters, grid, out, s) : int(hipErrorInvalidValue);
}
