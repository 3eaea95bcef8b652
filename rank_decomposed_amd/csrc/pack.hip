// Fragment-packed layout of a bf16 factor.
//
// A row-major W[N, K] becomes 16-row blocks, each a run of 32-column steps,
// each step the 1 KiB that one wave feeds to an MFMA 16x16x32 as its weight
// operand: lane l holds row 16b + l%16, columns 32s + 8(l/16) .. +8.  Element
// (n, k) goes to ((b*pitch + s)*64 + lane)*8 + e with b = n/16, s = k/32,
// lane = n%16 + 16((k%32)/8), e = k%8; rows past N and columns past K are
// zero.  The decode kernels then stream each step as contiguous memory.
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

// one thread per 16-byte output chunk (block, step, lane)
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W, int64_t N,
                                                   int64_t K, int64_t ld,
                                                   uint16_t* __restrict__ out, int64_t pitch,
                                                   int64_t nsteps, int64_t total) {
  for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
    const int lane = (int)(c & 63);
    const int64_t bs = c >> 6;
    const int64_t b = bs / nsteps, s = bs % nsteps;
    const int64_t n = b * 16 + (lane & 15), k0 = s * 32 + (lane >> 4) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N) {
      const uint16_t* row = W + n * ld + k0;
      if (k0 + 8 <= K) {
        v = ldg16(row);  // rows are 16-byte aligned (ld % 8 == 0)
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8 && k0 + e < K; ++e) w[e >> 1] |= (uint32_t)row[e] << (16 * (e & 1));
        v = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    *reinterpret_cast<u32x4*>(out + ((b * pitch + s) * 64 + lane) * 8) = v;
  }
}

}  // namespace

hipError_t pack_factor_bf16(const void* W, int64_t N, int64_t K, int64_t ld, void* packed,
                            int64_t pitch, hipStream_t st) {
  const int64_t nsteps = (K + 31) / 32, total = (N + 15) / 16 * nsteps * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(W), N, K, ld, static_cast<uint16_t*>(packed),
                     pitch, nsteps, total);
  return hipGetLastError();
}

}  // namespace lr
