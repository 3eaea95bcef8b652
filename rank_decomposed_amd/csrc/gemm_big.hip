// Large-tile NT GEMM on MFMA 32x32x16: C[M, N] = A[M, K] . B[N, K]^T with
// bf16 operands (both K-contiguous), fp32 accumulation, bf16 or fp32 output.
// Used for the many-token (prefill) decomposed linear: both stages, x U_r and
// t V_r, have this form with the factors stored transposed.
//
// Tile 256 x BN x 64 (BN = 256 or 128), one workgroup of 4 waves, each wave
// 128 x BN/2.  Operand tiles move global -> LDS with direct-to-LDS buffer
// loads (no registers in between), double-buffered: the loads of k-tile t+1
// are in flight while tile t multiplies.  LDS rows are 128 B with the 16-B
// chunk index XOR-swizzled by (row / 2) % 8, so the fragment reads (32 rows
// at one chunk) hit distinct banks.  The MFMA takes the B fragment as its
// first operand, so each lane ends with 4 consecutive output columns of one
// row: 8- or 16-byte stores.  Tiles go to the 8 XCDs in contiguous runs
// (workgroups are dealt to XCDs round robin), so an XCD's tiles share A rows
// in its L2.  The last, partial k-tile is masked in registers; rows past M or
// N and k-chunks past K read zero from outside the buffers.
#include <mutex>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int gBM = 256, gBK = 64;
constexpr int gTileA = gBM * gBK * 2;  // bytes of one A tile

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int VM>
__device__ __forceinline__ void wait_vm() {
  // vmcnt(VM); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS loads of a ROWS x 64 operand tile: instruction i moves rows
// 8i .. 8i+7 (lane l: row 8i + l/8, LDS slot l%8, global chunk swizzled), and
// wave w issues instructions w, w + 4, ...; chunks past the K range (kt
// elements left) go outside the buffer and read zero.
template <int ROWS>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kt,
                                          uint8_t* lds, int wave, int lane) {
  const int rr = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int i = 0; i < ROWS / 32; ++i) {
    const int inst = wave + 4 * i;
    const int row = inst * 8 + rr;
    const int chunk = swz(row, slot);
    const int off =
        chunk * 8 < kt ? (int)(((int64_t)row * ld + k0 + chunk * 8) * 2) : (int)0x80000000;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + inst * 1024), 16, off, 0, 0, 0);
  }
}

template <int NBW, bool MASK>
__device__ __forceinline__ void load_frags(u32x4 (&af)[4], u32x4 (&bfr)[NBW], const uint8_t* ta,
                                           const uint8_t* tb, int wm, int wn, int lane, int ks,
                                           int kt) {
  const int chunk = 2 * ks + (lane >> 5);
  const int r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm + i * 32 + r32;
    af[i] = *reinterpret_cast<const u32x4*>(ta + row * 128 + swz(row, chunk) * 16);
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int row = wn + i * 32 + r32;
    bfr[i] = *reinterpret_cast<const u32x4*>(tb + row * 128 + swz(row, chunk) * 16);
  }
  if (MASK) {
    const int kk = chunk * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = mask_tail_nb(af[i], kk, kt);
#pragma unroll
    for (int i = 0; i < NBW; ++i) bfr[i] = mask_tail_nb(bfr[i], kk, kt);
  }
}

// One 64-deep k-tile from LDS: 4 steps of 16 (fragments of step ks + 1 read
// while step ks multiplies).
template <int NBW, bool MASK>
__device__ __forceinline__ void tile_mma(f32x16 (&acc)[NBW][4], const uint8_t* ta,
                                         const uint8_t* tb, int wm, int wn, int lane, int kt) {
  u32x4 af[2][4], bfr[2][NBW];
  load_frags<NBW, MASK>(af[0], bfr[0], ta, tb, wm, wn, lane, 0, kt);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks + 1 < 4)
      load_frags<NBW, MASK>(af[(ks + 1) & 1], bfr[(ks + 1) & 1], ta, tb, wm, wn, lane, ks + 1, kt);
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(bfr[ks & 1][i], af[ks & 1][j], acc[i][j]);
  }
}

struct BigArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  void* c;        // bf16 or fp32 [M, ldc]
  int64_t ldc;
  uint16_t* c2;   // optional bf16 copy of an fp32 output [M, ldc2], 8-byte aligned rows
  int64_t ldc2;
  int M, N, K;
  int vec;        // C rows allow 4-element vector stores (else element stores)
};

template <int BN, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_big_kernel(BigArgs p) {
  constexpr int NBW = BN / 64;              // 32-column blocks per wave
  constexpr int kTileB = BN * gBK * 2;
  constexpr int kStage = gTileA + kTileB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntn = (p.N + BN - 1) / BN, ntiles = ntn * ((p.M + gBM - 1) / gBM);
  const int per_xcd = (ntiles + 7) / 8;
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= ntiles) return;
  const int m0 = (tile / ntn) * gBM, n0 = (tile % ntn) * BN;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.a + (int64_t)m0 * p.lda, view_bytes(min(p.M - m0, gBM), p.K, p.lda));
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(p.b + (int64_t)n0 * p.ldb, view_bytes(min(p.N - n0, BN), p.K, p.ldb));
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * (BN / 2);
  const int nk = (p.K + gBK - 1) / gBK;

  f32x16 acc[NBW][4];  // [n block][m block]; lane: one m row, 4 consecutive n per 4 regs
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  load_tile<gBM>(ra, p.lda, 0, p.K, smem, wave, lane);
  load_tile<BN>(rb, p.ldb, 0, p.K, smem + gTileA, wave, lane);
  for (int t = 0; t + 1 < nk; ++t) {
    uint8_t* cur = smem + (t & 1) * kStage;
    uint8_t* nxt = smem + ((t + 1) & 1) * kStage;
    load_tile<gBM>(ra, p.lda, (t + 1) * gBK, p.K - (t + 1) * gBK, nxt, wave, lane);
    load_tile<BN>(rb, p.ldb, (t + 1) * gBK, p.K - (t + 1) * gBK, nxt + gTileA, wave, lane);
    wait_vm<(gBM + BN) / 32>();  // this tile's loads are done; the next tile's stay in flight
    lds_barrier();
    tile_mma<NBW, false>(acc, cur, cur + gTileA, wm, wn, lane, gBK);
    lds_barrier();
  }
  wait_vm<0>();
  lds_barrier();
  {
    const uint8_t* cur = smem + ((nk - 1) & 1) * kStage;
    const int kt = p.K - (nk - 1) * gBK;
    if (kt < gBK)
      tile_mma<NBW, true>(acc, cur, cur + gTileA, wm, wn, lane, kt);
    else
      tile_mma<NBW, false>(acc, cur, cur + gTileA, wm, wn, lane, gBK);
  }

  // acc[i][j] reg r -> n = wn + 32i + 8(r/4) + 4(lane/32) + r%4, m = wm + 32j + lane%32
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm + 32 * j + (lane & 31);
      if (m >= p.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn + 32 * i + 8 * q + 4 * (lane >> 5);
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (OUT_F32) {
          float* c = static_cast<float*>(p.c) + (int64_t)m * p.ldc + n;
          uint16_t* c2 = p.c2 ? p.c2 + (int64_t)m * p.ldc2 + n : nullptr;
          if (p.vec && n + 3 < p.N) {
            *reinterpret_cast<f32x4*>(c) = f32x4{v0, v1, v2, v3};
            if (c2) *reinterpret_cast<u32x2*>(c2) = u32x2{pack_bf2(v0, v1), pack_bf2(v2, v3)};
          } else {
            const float v[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4 && n + e < p.N; ++e) {
              c[e] = v[e];
              if (c2) c2[e] = (uint16_t)f2bf(v[e]);
            }
          }
        } else {
          uint16_t* c = static_cast<uint16_t*>(p.c) + (int64_t)m * p.ldc + n;
          if (p.vec && n + 3 < p.N) {
            *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf2(v0, v1), pack_bf2(v2, v3)};
          } else {
            const float v[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4 && n + e < p.N; ++e) c[e] = (uint16_t)f2bf(v[e]);
          }
        }
      }
    }
}

template <int BN, bool OUT_F32>
hipError_t launch_big(const BigArgs& a, hipStream_t st) {
  constexpr size_t lds = 2 * (size_t)(gTileA + BN * gBK * 2);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_big_kernel<BN, OUT_F32>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + gBM - 1) / gBM);
  hipLaunchKernelGGL((gemm_big_kernel<BN, OUT_F32>), dim3((unsigned)((tiles + 7) / 8 * 8)),
                     dim3(256), lds, st, a);
  return hipGetLastError();
}

// Fraction of the launch's CU-rounds doing useful columns, for a tile width.
double tile_efficiency(int M, int N, int BN) {
  const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + gBM - 1) / gBM);
  const int64_t rounds = (tiles + 255) / 256;
  return (double)tiles / (rounds * 256) * ((double)N / (((N + BN - 1) / BN) * BN));
}

}  // namespace

bool gemm_big_supported(int64_t lda, int64_t ldb) {
  // 32-bit offsets within a 256-row tile
  return lda < (int64_t(1) << 22) && ldb < (int64_t(1) << 22);
}

hipError_t gemm_nt_big(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                       int64_t ldc, bool c_f32, uint16_t* C2, int64_t ldc2, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
  const uintptr_t cal = c_f32 ? 16 : 8;
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
            C2, ldc2, (int)M, (int)N, (int)K,
            (reinterpret_cast<uintptr_t>(C) % cal == 0 && ldc % 4 == 0) ? 1 : 0};
  const bool narrow = tile_efficiency((int)M, (int)N, 128) > tile_efficiency((int)M, (int)N, 256) + 0.05;
  if (c_f32) return narrow ? launch_big<128, true>(a, st) : launch_big<256, true>(a, st);
  return narrow ? launch_big<128, false>(a, st) : launch_big<256, false>(a, st);
}

}  // namespace lr
