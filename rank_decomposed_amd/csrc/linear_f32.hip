// fp32 path of the decomposed linear: t = x U_r, y = t V_r (DeInfer/en §2.A)
// with fp32 operands and fp32 accumulation, for callers that need full
// single precision.  Both stages are C[M, N] = A[M, K] . B[N, K]^T on a
// 64 x 64 SIMT tile (16 x 16 threads, 4 x 4 outputs each, K staged through
// LDS 16 at a time).  Arbitrary shapes and leading dimensions.
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int fT = 64, fK = 16;

__global__ __launch_bounds__(256) void f32_nt_kernel(const float* __restrict__ A, int64_t lda,
                                                     const float* __restrict__ B, int64_t ldb,
                                                     float* __restrict__ C, int64_t ldc, int M,
                                                     int N, int K) {
  __shared__ float As[fK][fT + 1];
  __shared__ float Bs[fK][fT + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * fT, n0 = blockIdx.x * fT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += fK) {
    // 64 x 16 of A and of B: 1024 elements, 4 per thread
    for (int e = threadIdx.x; e < fT * fK; e += 256) {
      const int row = e / fK, kk = e % fK;
      const int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      As[kk][row] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.f;
      Bs[kk][row] = (gn < N && gk < K) ? B[(int64_t)gn * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < fK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty + 16 * i];
        b[i] = Bs[kk][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * j;
      if (gm < M && gn < N) C[(int64_t)gm * ldc + gn] = acc[i][j];
    }
}

hipError_t launch(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                  int64_t ldc, int M, int N, int K, hipStream_t st) {
  dim3 grid((N + fT - 1) / fT, (M + fT - 1) / fT);
  hipLaunchKernelGGL(f32_nt_kernel, grid, dim3(256), 0, st, A, lda, B, ldb, C, ldc, M, N, K);
  return hipGetLastError();
}

}  // namespace

// t [T, r] past the decode path's control area
size_t f32_workspace_bytes(int64_t T, int64_t r) {
  return kCtlAreaBytes + (size_t)((T * r * 4 + 255) / 256 * 256);
}

hipError_t linear_f32(const DecodeLinear& d, hipStream_t st) {
  float* t = d.t_io;
  int64_t ldt = d.ldt;
  if (!t) {
    t = reinterpret_cast<float*>(static_cast<uint8_t*>(d.workspace) + kCtlAreaBytes);
    ldt = d.r;
  }
  if (d.flags != 2) {
    hipError_t e = launch(static_cast<const float*>(d.x), d.ldx, static_cast<const float*>(d.Ut),
                          d.ldu, t, ldt, (int)d.T, (int)d.r, (int)d.d_in, st);
    if (e != hipSuccess || d.flags == 1) return e;
  }
  return launch(t, ldt, static_cast<const float*>(d.Vt), d.ldv, static_cast<float*>(d.y), d.ldy,
                (int)d.T, (int)d.d_out, (int)d.r, st);
}

}  // namespace lr
