// Remap gather: the graph-replay copy of DeInfer/en §2.C (DeInfer/es §2,
// "Etapa de Reproducción del Gráfico"): rows of the paged latent pool are
// copied into a compact buffer at a fixed address following the remapping
// index list of the preparation stage.
//
// The grid is sized from the fixed capacity, never from the live row count,
// so a captured graph replays unchanged while lengths vary: each wave walks
// rows j = wave_id, wave_id + n_waves, ... and stops at *n_valid (read on the
// device).  Pure data movement: one 16-byte load and store per lane, a row of
// 409..1024 bf16 elements is one or two wave-wide transactions.  Invalid
// source indices produce zero rows; nothing is read out of bounds.
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

// VEC = bytes moved per lane per access (16, 4 or 2)
template <int VEC>
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ src,
                                                     int64_t src_rows, int64_t src_pitch,
                                                     const int32_t* __restrict__ remap,
                                                     int64_t cap, const int32_t* n_valid,
                                                     int64_t row_bytes, char* __restrict__ dst,
                                                     int64_t dst_pitch) {
  int64_t nv = cap;
  if (n_valid) {
    const int64_t v = *n_valid;
    nv = v < 0 ? 0 : (v < cap ? v : cap);
  }
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t nvec = row_bytes / VEC;
  for (int64_t j = wid; j < nv; j += nw) {
    const int64_t s = remap[j];
    const bool ok = s >= 0 && s < src_rows;
    const char* srow = src + (ok ? s : 0) * src_pitch;
    char* drow = dst + j * dst_pitch;
    for (int64_t c = lane; c < nvec; c += 64) {
      if (VEC == 16) {
        u32x4 v = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(srow + c * 16))
                     : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(drow + c * 16) = v;
      } else if (VEC == 4) {
        uint32_t v = ok ? *reinterpret_cast<const uint32_t*>(srow + c * 4) : 0u;
        *reinterpret_cast<uint32_t*>(drow + c * 4) = v;
      } else {
        uint16_t v = ok ? *reinterpret_cast<const uint16_t*>(srow + c * 2) : (uint16_t)0;
        *reinterpret_cast<uint16_t*>(drow + c * 2) = v;
      }
    }
    // tail bytes not covered by VEC-wide accesses (2-byte granularity)
    for (int64_t b = nvec * VEC + 2 * lane; b < row_bytes; b += 128) {
      uint16_t v = ok ? *reinterpret_cast<const uint16_t*>(srow + b) : (uint16_t)0;
      *reinterpret_cast<uint16_t*>(drow + b) = v;
    }
  }
}

}  // namespace

hipError_t remap_gather(int elem_bytes, const void* src, int64_t src_rows, int64_t src_ld,
                        const int32_t* remap, int64_t cap, const int32_t* n_valid,
                        int64_t row_elems, void* dst, int64_t dst_ld, hipStream_t st) {
  const int64_t row_bytes = row_elems * elem_bytes;
  const int64_t sp = src_ld * elem_bytes, dp = dst_ld * elem_bytes;
  const uintptr_t sa = reinterpret_cast<uintptr_t>(src), da = reinterpret_cast<uintptr_t>(dst);
  // one wave per row; cap the grid at 8 waves per CU-equivalent
  int64_t waves = cap < 8192 ? cap : 8192;
  if (waves < 1) waves = 1;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (sp % 16 == 0 && dp % 16 == 0 && sa % 16 == 0 && da % 16 == 0) {
    hipLaunchKernelGGL(gather_kernel<16>, grid, dim3(256), 0, st, (const char*)src, src_rows, sp,
                       remap, cap, n_valid, row_bytes, (char*)dst, dp);
  } else if (sp % 4 == 0 && dp % 4 == 0 && sa % 4 == 0 && da % 4 == 0) {
    hipLaunchKernelGGL(gather_kernel<4>, grid, dim3(256), 0, st, (const char*)src, src_rows, sp,
                       remap, cap, n_valid, row_bytes, (char*)dst, dp);
  } else {
    hipLaunchKernelGGL(gather_kernel<2>, grid, dim3(256), 0, st, (const char*)src, src_rows, sp,
                       remap, cap, n_valid, row_bytes, (char*)dst, dp);
  }
  return hipGetLastError();
}

}  // namespace lr
