// Decode path of the decomposed linear (few token rows, HBM-bound).
//
// DeInfer/en §2.A: the downward projection forms the rank-r intermediate,
// the upward projection maps it back.  With T <= 64 tokens every weight byte
// is used by at most 64 rows, so both stages are bound by streaming U_r and
// V_r from HBM once.  Each stage is a "skinny" product
//
//     C[T, N] = A[T, K] . B[N, K]^T        (B = weight rows, K contiguous)
//
// run on bf16 MFMA 16x16x32 with the token dimension padded to 16/32/64:
// MFMA issue is nearly free next to the HBM stream, and it removes the VALU
// ceiling that a dot-product GEMV hits once T grows past ~16.
//
// Work split: a workgroup (4 waves) owns 16 weight rows and a K range; the
// waves interleave over its 32-wide k-steps and are reduced through LDS.
// Stage 1 splits K across workgroups (S splits) to put >= ~512 workgroups in
// flight; the S fp32 partials are summed in a fixed order (deterministic) by
// a small reduce kernel that also emits the intermediate as a bf16 hi/lo
// pair, so stage 2 sees t at ~16 mantissa bits (two MFMAs per fragment,
// still far below the memory time).
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

enum { EPI_PARTIAL = 0, EPI_T = 1, EPI_Y = 2 };

struct SkinnyArgs {
  const uint16_t* a_hi;   // [T, lda] bf16 (x, or t hi part)
  const uint16_t* a_lo;   // [T, lda] bf16 (t lo part) or nullptr
  int64_t lda;
  const uint16_t* b;      // [N, ldb] bf16 weight rows
  int64_t ldb;
  int T, N, K;
  int kchunk;             // K range per blockIdx.y (multiple of 32)
  // epilogues
  float* part;            // EPI_PARTIAL: [S][T][N]
  float* t32;             // EPI_T: optional fp32 [T, ldt32]
  int64_t ldt32;
  uint16_t* thi;          // EPI_T: bf16 hi [T, ldtb]
  uint16_t* tlo;          // EPI_T: bf16 lo [T, ldtb]
  int64_t ldtb;
  uint16_t* y;            // EPI_Y: bf16 [T, ldy]
  int64_t ldy;
};

template <int TB, bool SPLIT, int EPI>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int kbeg = blockIdx.y * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int col = lane & 15;       // weight row within the tile / A row
  const int kg = (lane >> 4) * 8;  // k offset of this lane's 8-element group

  const int nrow = n0 + col;
  const bool brow_ok = nrow < p.N;
  const uint16_t* bptr = p.b + (int64_t)(brow_ok ? nrow : 0) * p.ldb;

  const uint16_t* aptr[TB];
  const uint16_t* alop[TB];
  bool arow_ok[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    int tok = tb * 16 + col;
    arow_ok[tb] = tok < p.T;
    aptr[tb] = p.a_hi + (int64_t)(arow_ok[tb] ? tok : 0) * p.lda;
    alop[tb] = SPLIT ? p.a_lo + (int64_t)(arow_ok[tb] ? tok : 0) * p.lda : nullptr;
  }

  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (kend - kbeg + 31) / 32;
  // wave w takes k-steps w, w + 4, w + 8, ...
  for (int s0 = wave; s0 < nsteps; s0 += kWaves * kUnroll) {
    u32x4 bv[kUnroll];
    u32x4 av[kUnroll][TB];
    u32x4 alv[kUnroll][TB];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u * kWaves;
      const int k = kbeg + s * 32 + kg;
      const bool kin = (s < nsteps) && (k < kend);
      bv[u] = (kin && brow_ok) ? ldg16_stream(bptr + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        av[u][tb] = (kin && arow_ok[tb]) ? ldg16(aptr[tb] + k) : u32x4{0, 0, 0, 0};
        if (SPLIT) alv[u][tb] = (kin && arow_ok[tb]) ? ldg16(alop[tb] + k) : u32x4{0, 0, 0, 0};
      }
      if (kin && k + 8 > kend) {
        bv[u] = mask_tail(bv[u], k, kend);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          av[u][tb] = mask_tail(av[u][tb], k, kend);
          if (SPLIT) alv[u][tb] = mask_tail(alv[u][tb], k, kend);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        acc[tb] = mfma16x16x32(av[u][tb], bv[u], acc[tb]);
        if (SPLIT) acc[tb] = mfma16x16x32(alv[u][tb], bv[u], acc[tb]);
      }
    }
  }

  // reduce the 4 waves through LDS: red[wave][tb*4 + v][lane]
  __shared__ float red[kWaves][TB * 4][64];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    red[wave][tb * 4 + 0][lane] = acc[tb].x;
    red[wave][tb * 4 + 1][lane] = acc[tb].y;
    red[wave][tb * 4 + 2][lane] = acc[tb].z;
    red[wave][tb * 4 + 3][lane] = acc[tb].w;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TB * 4 * 64; e += 256) {
    const int j = e / 64, l = e % 64;
    const float v = red[0][j][l] + red[1][j][l] + red[2][j][l] + red[3][j][l];
    const int tok = (j / 4) * 16 + 4 * (l >> 4) + (j % 4);
    const int n = n0 + (l & 15);
    if (tok >= p.T || n >= p.N) continue;
    if (EPI == EPI_PARTIAL) {
      p.part[((int64_t)blockIdx.y * p.T + tok) * p.N + n] = v;
    } else if (EPI == EPI_T) {
      if (p.t32) p.t32[(int64_t)tok * p.ldt32 + n] = v;
      const uint32_t hi = f2bf(v);
      p.thi[(int64_t)tok * p.ldtb + n] = (uint16_t)hi;
      p.tlo[(int64_t)tok * p.ldtb + n] = (uint16_t)f2bf(v - bf2f(hi));
    } else {
      p.y[(int64_t)tok * p.ldy + n] = (uint16_t)f2bf(v);
    }
  }
}

// Sum the S stage-1 partials in split order and emit t (fp32, optional) and
// its bf16 hi/lo pair (row pitch ldtb >= N; the pitch padding is never read
// unmasked).
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int S, int T, int N, float* t32,
                                                              int64_t ldt32, uint16_t* thi,
                                                              uint16_t* tlo, int64_t ldtb) {
  const int64_t total = (int64_t)T * ldtb;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int tok = (int)(e / ldtb), n = (int)(e % ldtb);
    if (n >= N) continue;
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part[((int64_t)s * T + tok) * N + n];
    if (t32) t32[(int64_t)tok * ldt32 + n] = v;
    const uint32_t hi = f2bf(v);
    thi[e] = (uint16_t)hi;
    tlo[e] = (uint16_t)f2bf(v - bf2f(hi));
  }
}

// t (fp32, caller's layout) -> bf16 hi/lo pair for a stage-2-only call.
__global__ __launch_bounds__(256) void split_t_kernel(const float* __restrict__ t, int64_t ldt,
                                                      int T, int N, uint16_t* thi, uint16_t* tlo,
                                                      int64_t ldtb) {
  const int64_t total = (int64_t)T * ldtb;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int tok = (int)(e / ldtb), n = (int)(e % ldtb);
    if (n >= N) continue;
    const float v = t[(int64_t)tok * ldt + n];
    const uint32_t hi = f2bf(v);
    thi[e] = (uint16_t)hi;
    if (tlo) tlo[e] = (uint16_t)f2bf(v - bf2f(hi));
  }
}

template <int TB, bool SPLIT, int EPI>
hipError_t launch_skinny(const SkinnyArgs& a, int S, hipStream_t st) {
  dim3 grid((a.N + 15) / 16, S);
  hipLaunchKernelGGL((skinny_kernel<TB, SPLIT, EPI>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool SPLIT, int EPI>
hipError_t dispatch_tb(int T, const SkinnyArgs& a, int S, hipStream_t st) {
  if (T <= 16) return launch_skinny<1, SPLIT, EPI>(a, S, st);
  if (T <= 32) return launch_skinny<2, SPLIT, EPI>(a, S, st);
  return launch_skinny<4, SPLIT, EPI>(a, S, st);
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

// Stage-1 K split: enough workgroups to cover the chip, each K range a
// multiple of 4 waves x 32.
static void stage1_split(int N, int K, int* S_out, int* kchunk_out) {
  const int tiles = (N + 15) / 16;
  int S = (512 + tiles - 1) / tiles;
  const int max_s = (K + 127) / 128;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  int kchunk = (int)round_up((K + S - 1) / S, 128);
  S = (K + kchunk - 1) / kchunk;
  *S_out = S;
  *kchunk_out = kchunk;
}

size_t decode_workspace_bytes(int64_t T, int64_t d_in, int64_t r) {
  int S, kc;
  stage1_split((int)r, (int)d_in, &S, &kc);
  const int64_t ldtb = round_up(r, 8);
  size_t part = S > 1 ? (size_t)S * T * r * sizeof(float) : 0;
  part = (size_t)round_up((int64_t)part, 256);
  size_t tb = (size_t)round_up(T * ldtb * 2, 256);
  return part + 2 * tb;
}

hipError_t decode_linear_bf16(const DecodeLinear& d, hipStream_t st) {
  int S, kchunk;
  stage1_split((int)d.r, (int)d.d_in, &S, &kchunk);
  const int64_t ldtb = round_up(d.r, 8);
  char* ws = static_cast<char*>(d.workspace);
  size_t part_bytes = S > 1 ? (size_t)S * d.T * d.r * sizeof(float) : 0;
  part_bytes = (size_t)round_up((int64_t)part_bytes, 256);
  float* part = reinterpret_cast<float*>(ws);
  uint16_t* thi = reinterpret_cast<uint16_t*>(ws + part_bytes);
  uint16_t* tlo = thi + round_up(d.T * ldtb * 2, 256) / 2;
  const int T = (int)d.T;
  hipError_t e = hipSuccess;

  if (d.flags != 2 /* not stage-2-only */) {
    SkinnyArgs a{};
    a.a_hi = static_cast<const uint16_t*>(d.x);
    a.lda = d.ldx;
    a.b = static_cast<const uint16_t*>(d.Ut);
    a.ldb = d.ldu;
    a.T = T;
    a.N = (int)d.r;
    a.K = (int)d.d_in;
    a.kchunk = kchunk;
    if (S > 1) {
      a.part = part;
      e = dispatch_tb<false, EPI_PARTIAL>(T, a, S, st);
      if (e != hipSuccess) return e;
      const int64_t total = d.T * ldtb;
      int blocks = (int)((total + 255) / 256);
      if (blocks > 1024) blocks = 1024;
      hipLaunchKernelGGL(reduce_partials_kernel, dim3(blocks), dim3(256), 0, st, part, S, T,
                         (int)d.r, d.t_io, d.ldt, thi, tlo, ldtb);
      e = hipGetLastError();
    } else {
      a.t32 = d.t_io;
      a.ldt32 = d.ldt;
      a.thi = thi;
      a.tlo = tlo;
      a.ldtb = ldtb;
      e = dispatch_tb<false, EPI_T>(T, a, 1, st);
    }
    if (e != hipSuccess) return e;
  } else {
    const int64_t total = d.T * ldtb;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(split_t_kernel, dim3(blocks), dim3(256), 0, st, d.t_io, d.ldt, T,
                       (int)d.r, thi, tlo, ldtb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d.flags == 1 /* stage-1 only */) return hipSuccess;

  SkinnyArgs b{};
  b.a_hi = thi;
  b.a_lo = tlo;
  b.lda = ldtb;
  b.b = static_cast<const uint16_t*>(d.Vt);
  b.ldb = d.ldv;
  b.T = T;
  b.N = (int)d.d_out;
  b.K = (int)d.r;  // chunks straddling r are masked on both operands
  b.kchunk = (int)round_up(d.r, 32);
  b.y = static_cast<uint16_t*>(d.y);
  b.ldy = d.ldy;
  return dispatch_tb<true, EPI_Y>(T, b, 1, st);
}

}  // namespace lr
