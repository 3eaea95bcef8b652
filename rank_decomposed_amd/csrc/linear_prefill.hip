// Prefill path of the decomposed linear (many token rows, MFMA-bound).
//
// DeInfer/en §2.A: t = x U_r (downward projection), y = t V_r (upward
// projection).  For T > 64 both contractions are dense bf16 GEMMs.
//
// Fused kernel: a workgroup owns BM = 64 token rows.  Stage 1 computes the
// whole rank-r tile t[64, r] chunk by chunk on MFMA 16x16x32 and parks it in
// LDS as bf16 (round to nearest even); stage 2 reads it straight from LDS as
// the A operand of y = t V_r.  t never touches HBM.  Every workgroup streams
// all of U_r and V_r, so the kernel's intensity against L2 is BM flop per
// weight byte; the weights stay L2/MALL-resident while the 256 CUs walk them
// in the same order.
//
// Wave layout: the 4 waves share the 64 rows (4 row blocks of 16) and split
// each 512-wide column chunk into 4 x 128 (8 column blocks of 16 per wave).
// Operands come straight from memory into registers with raw buffer loads
// (rows past a matrix edge read zero, so no branches), two 32-wide k-steps
// ahead in a register ring.  The k-loop body has no conditionals, so the
// compiler keeps the ring's loads in flight across steps; the one partial
// k-step (K not a multiple of 32) is masked after the loop.
//
// Plain kernel: C = A . B^T on a 128x128 tile with LDS double buffering, for
// the stage-only calls (tensor-parallel share) and for ranks too large for the
// on-chip tile.
#include <algorithm>
#include <mutex>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kBM = 64;                 // fused: token rows per workgroup
constexpr int kMB = kBM / 16;           // fused: 16-row blocks per wave
constexpr int kNB = 8;                  // fused: 16-wide column blocks per wave
constexpr int kChunk = 4 * kNB * 16;    // 512 columns per chunk
constexpr int kRing = 2;                // k-steps of operands in flight per wave
constexpr int kLdsMax = 163840;         // gfx950 LDS per workgroup

struct FusedArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* ut;
  int64_t ldu;
  const uint16_t* vt;
  int64_t ldv;
  uint16_t* y;
  int64_t ldy;
  int M, d_in, r, d_out;
  int r_pad;  // multiple of 32
};

__global__ __launch_bounds__(256, 1) void fused_kernel(FusedArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int tpitch = p.r_pad + 8;
  uint16_t* ts = smem;  // [64][tpitch] bf16 rank tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kBM;
  const int rr = lane & 15, kq = (lane >> 4) * 8;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, view_bytes(p.M, p.d_in, p.ldx));
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.ut, view_bytes(p.r, p.d_in, p.ldu));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vt, view_bytes(p.d_out, p.r, p.ldv));

  // ---------------- stage 1: ts = bf16(x[m0:m0+64] . U_r) ----------------
  {
    const int ks = (p.d_in + 31) / 32;
    const bool tail = (p.d_in % 32) != 0;
    const int kf = tail ? ks - 1 : ks;  // k-steps needing no mask
    for (int c0 = 0; c0 < p.r_pad; c0 += kChunk) {
      const int row0 = c0 + wave * kNB * 16;
      if (row0 >= p.r_pad) continue;  // wave-uniform
      f32x4 acc[kMB][kNB];
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 bq[kRing][kNB], aq[kRing][kMB];
#pragma unroll
      for (int q = 0; q < kRing; ++q) {
        frag_load<kNB>(bq[q], ru, p.ldu, row0, q * 32, lane);
        frag_load<kMB>(aq[q], rx, p.ldx, m0, q * 32, lane);
      }
      int s = 0;
      for (; s + kRing <= kf; s += kRing) {
#pragma unroll
        for (int q = 0; q < kRing; ++q) {
          frag_mma<kMB, kNB>(acc, aq[q], bq[q]);
          // steps past the end load in-range junk or zeros and are never used
          frag_load<kNB>(bq[q], ru, p.ldu, row0, (s + q + kRing) * 32, lane);
          frag_load<kMB>(aq[q], rx, p.ldx, m0, (s + q + kRing) * 32, lane);
        }
      }
#pragma unroll
      for (int q = 0; q < kRing; ++q) {
        if (s + q < kf) {
          frag_mma<kMB, kNB>(acc, aq[q], bq[q]);
        } else if (tail && s + q == kf) {
          frag_mask<kNB>(bq[q], kf * 32, p.d_in, lane);
          frag_mask<kMB>(aq[q], kf * 32, p.d_in, lane);
          frag_mma<kMB, kNB>(acc, aq[q], bq[q]);
        }
      }
      // rows of U_r^T past r read as zero, so columns [r, r_pad) of ts are 0
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          const int col = row0 + j * 16 + rr;
          if (col < p.r_pad) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              ts[(i * 16 + (lane >> 4) * 4 + v) * tpitch + col] = (uint16_t)f2bf(acc[i][j][v]);
          }
        }
    }
  }
  __syncthreads();

  // ---------------- stage 2: y[m0:m0+64] = ts . V_r ----------------
  {
    const int ks = p.r_pad / 32;
    const bool tail = (p.r % 32) != 0;
    const int kf = tail ? ks - 1 : ks;
    for (int c0 = 0; c0 < p.d_out; c0 += kChunk) {
      const int row0 = c0 + wave * kNB * 16;
      if (row0 >= p.d_out) continue;
      f32x4 acc[kMB][kNB];
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 bq[kRing][kNB];
#pragma unroll
      for (int q = 0; q < kRing; ++q) frag_load<kNB>(bq[q], rv, p.ldv, row0, q * 32, lane);
      int s = 0;
      for (; s + kRing <= kf; s += kRing) {
#pragma unroll
        for (int q = 0; q < kRing; ++q) {
          u32x4 a[kMB];
#pragma unroll
          for (int i = 0; i < kMB; ++i) a[i] = lds16(ts + (i * 16 + rr) * tpitch + (s + q) * 32 + kq);
          frag_mma<kMB, kNB>(acc, a, bq[q]);
          frag_load<kNB>(bq[q], rv, p.ldv, row0, (s + q + kRing) * 32, lane);
        }
      }
#pragma unroll
      for (int q = 0; q < kRing; ++q) {
        if (s + q < kf || (tail && s + q == kf)) {
          if (s + q == kf) frag_mask<kNB>(bq[q], kf * 32, p.r, lane);
          u32x4 a[kMB];
#pragma unroll
          for (int i = 0; i < kMB; ++i) a[i] = lds16(ts + (i * 16 + rr) * tpitch + (s + q) * 32 + kq);
          frag_mma<kMB, kNB>(acc, a, bq[q]);
        }
      }
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          const int col = row0 + j * 16 + rr;
          if (col >= p.d_out) continue;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tok = m0 + i * 16 + (lane >> 4) * 4 + v;
            if (tok < p.M) p.y[(int64_t)tok * p.ldy + col] = (uint16_t)f2bf(acc[i][j][v]);
          }
        }
    }
  }
}

// ------------------------------------------------------------------ plain GEMM
// C[M, N] = A[M, K] . B[N, K]^T ; A bf16 or fp32 (rounded to bf16 on load),
// B bf16, C fp32 or bf16.
constexpr int gBM = 128, gBN = 128, gBK = 32, gPitch = 40;

struct GemmArgs {
  const void* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  void* c;
  int64_t ldc;
  int M, N, K;
};

template <bool A_F32, bool C_F32>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][gBM * gPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][gBN * gPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int m0 = blockIdx.y * gBM, n0 = blockIdx.x * gBN;
  const int rr = lane & 15, kq = (lane >> 4) * 8;

  // staging map: 512 chunks of 8 elements per tile; thread t takes t and t+256
  auto load_a = [&](int k, u32x4 (&reg)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = threadIdx.x + i * 256;
      const int row = ch >> 2, kk = k + (ch & 3) * 8;
      const int grow = m0 + row;
      reg[i] = u32x4{0, 0, 0, 0};
      if (grow < p.M && kk < p.K) {
        if (A_F32) {
          const float* src = static_cast<const float*>(p.a) + (int64_t)grow * p.lda + kk;
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = (kk + e < p.K) ? src[e] : 0.f;
          reg[i] = u32x4{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                         pack_bf2(f[6], f[7])};
        } else {
          u32x4 v = ldg16(static_cast<const uint16_t*>(p.a) + (int64_t)grow * p.lda + kk);
          reg[i] = (kk + 8 > p.K) ? mask_tail(v, kk, p.K) : v;
        }
      }
    }
  };
  auto load_b = [&](int k, u32x4 (&reg)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = threadIdx.x + i * 256;
      const int row = ch >> 2, kk = k + (ch & 3) * 8;
      const int grow = n0 + row;
      reg[i] = u32x4{0, 0, 0, 0};
      if (grow < p.N && kk < p.K) {
        u32x4 v = ldg16(p.b + (int64_t)grow * p.ldb + kk);
        reg[i] = (kk + 8 > p.K) ? mask_tail(v, kk, p.K) : v;
      }
    }
  };
  auto store = [&](uint16_t* dst, const u32x4 (&reg)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = threadIdx.x + i * 256;
      *reinterpret_cast<u32x4*>(dst + (ch >> 2) * gPitch + (ch & 3) * 8) = reg[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = (p.K + gBK - 1) / gBK;
  u32x4 ra[2], rb[2];
  load_a(0, ra);
  load_b(0, rb);
  store(As[0], ra);
  store(Bs[0], rb);
  __syncthreads();
  for (int s = 0; s < ksteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < ksteps) {
      load_a((s + 1) * gBK, ra);
      load_b((s + 1) * gBK, rb);
    }
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = lds16(As[buf] + (wm + i * 16 + rr) * gPitch + kq);
      b[i] = lds16(Bs[buf] + (wn + i * 16 + rr) * gPitch + kq);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    if (s + 1 < ksteps) {
      store(As[buf ^ 1], ra);
      store(Bs[buf ^ 1], rb);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 16 + rr;
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + v;
        if (row >= p.M) continue;
        if (C_F32)
          static_cast<float*>(p.c)[(int64_t)row * p.ldc + col] = acc[i][j][v];
        else
          static_cast<uint16_t*>(p.c)[(int64_t)row * p.ldc + col] = (uint16_t)f2bf(acc[i][j][v]);
      }
    }
}

template <bool A_F32, bool C_F32>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  dim3 grid((g.N + gBN - 1) / gBN, (g.M + gBM - 1) / gBM);
  hipLaunchKernelGGL((gemm_nt_kernel<A_F32, C_F32>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

int64_t rup(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

hipError_t gemm_nt_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                        int64_t ldc, int M, int N, int K, hipStream_t st) {
  GemmArgs g{};
  g.a = A;
  g.lda = lda;
  g.b = static_cast<const uint16_t*>(B);
  g.ldb = ldb;
  g.c = C;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  return launch_gemm<false, false>(g, st);
}

namespace {

size_t fused_lds_bytes(int64_t r) { return (size_t)kBM * (rup(r, 32) + 8) * 2; }

}  // namespace

static bool fused_fits(int64_t r) { return fused_lds_bytes(r) <= (size_t)kLdsMax; }

// From this many rows on, both stages run as large-tile GEMMs through a bf16
// t in the workspace: the round trip of t through HBM costs well under 1 % of
// the time of either contraction, and the 256-row tiles run the MFMA units
// far closer to their peak than the fused kernel's 64-row tiles.
constexpr int64_t kBigT = 1024;

// fp32 scratch after t on the large-tile path: the partials of a stage 1
// that splits d_in, or of either stage's split tail (one at a time).
static size_t big_part_bytes(int64_t T, int64_t r, int64_t d_out) {
  return std::max({gemm_split_bytes(T, r), gemm_tail_bytes(T, r), gemm_tail_bytes(T, d_out)});
}

// Calls from kBigT rows on, and calls whose rank tile does not fit on chip,
// park t in the workspace as bf16 [T, round_up(r, 8)], past the decode
// path's control area; the fused kernel needs none.  From kBigT rows on, a
// stage 1 with too few tiles to fill the chip splits its d_in range, and a
// stage whose last round of tiles is part-filled may split that round's
// tiles over K: the fp32 partials follow t.
size_t prefill_workspace_bytes(int64_t T, int64_t r, int64_t d_out) {
  (void)d_out;
  if (T < kBigT && fused_fits(r)) return 0;
  const size_t tb = (size_t)rup(T * rup(r, 8) * 2, 256);
  return kCtlAreaBytes + (T >= kBigT ? tb + big_part_bytes(T, r, d_out) : tb);
}

// Where t starts in a workspace (the control area's words are never touched).
static uint16_t* parked_t(void* workspace) {
  return reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + kCtlAreaBytes);
}

namespace {

// bf16 copy (round to nearest even) of an fp32 [rows, cols] matrix.
__global__ void to_bf16_kernel(const float* src, int64_t lds, uint16_t* dst, int64_t ldd,
                               int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / cols, col = i % cols;
    dst[row * ldd + col] = (uint16_t)f2bf(src[row * lds + col]);
  }
}

// Stage 2 on the large-tile GEMM from the bf16 t at tws: y, y_acc += y, or
// act(y); part (part_bytes) takes a split tail's partials.
hipError_t big_stage2(const DecodeLinear& d, const uint16_t* tws, int64_t ldtb, float* part,
                      size_t part_bytes, hipStream_t st) {
  if (d.y_acc)
    return gemm_nt_big_acc(tws, ldtb, d.Vt, d.ldv, d.y_acc, d.ld_acc, d.T, d.d_out, d.r, st);
  if (d.act)
    return gemm_nt_big_act(tws, ldtb, d.Vt, d.ldv, static_cast<uint16_t*>(d.y), d.ldy, d.act,
                           static_cast<const uint16_t*>(d.glu), d.ldglu, d.T, d.d_out, d.r, st);
  return gemm_nt_big(tws, ldtb, d.Vt, d.ldv, d.y, d.ldy, false, nullptr, 0, d.T, d.d_out, d.r, st,
                     part, part_bytes);
}

// Both stages on the large-tile GEMM: t (bf16, [T, ldtb]) in the workspace;
// an fp32 t_io is written by stage 1 beside it, or read by a stage-2-only
// call and rounded into it first.
hipError_t prefill_big(const DecodeLinear& d, hipStream_t st) {
  const int64_t ldtb = rup(d.r, 8);
  uint16_t* tws = parked_t(d.workspace);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(tws) + rup(d.T * ldtb * 2, 256));
  const size_t part_bytes = big_part_bytes(d.T, d.r, d.d_out);
  hipError_t e = hipSuccess;
  if (d.flags != 2) {
    if (gemm_split_ranges(d.T, d.r, d.d_in) > 1) {
      e = gemm_nt_big_split(d.x, d.ldx, d.Ut, d.ldu, part, d.t_io, d.ldt,
                            d.t_io && d.flags == 1 ? nullptr : tws, ldtb, d.T, d.r, d.d_in, st);
    } else if (d.t_io)
      e = gemm_nt_big(d.x, d.ldx, d.Ut, d.ldu, d.t_io, d.ldt, true, d.flags == 1 ? nullptr : tws,
                      ldtb, d.T, d.r, d.d_in, st);
    else
      e = gemm_nt_big(d.x, d.ldx, d.Ut, d.ldu, tws, ldtb, false, nullptr, 0, d.T, d.r, d.d_in, st,
                      part, part_bytes);
    if (e != hipSuccess || d.flags == 1) return e;
  } else {
    const int64_t n = d.T * d.r;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, st, d.t_io, d.ldt, tws, ldtb,
                       d.T, d.r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return big_stage2(d, tws, ldtb, part, part_bytes, st);
}

// Workspace of a grouped call: the control area, each full member's bf16 t
// and fp32 t (the latter unused when the member has a t_io), then the
// split-tail scratch of the largest stage 2.
struct GroupLayout {
  size_t tb[kMaxGemmGroup], t32[kMaxGemmGroup], part, part_bytes, total;
};
GroupLayout group_layout(const DecodeLinear* ds, int n) {
  GroupLayout L{};
  size_t off = kCtlAreaBytes;
  for (int i = 0; i < n; ++i) {
    if (ds[i].flags != 0) continue;
    const int64_t ldtb = rup(ds[i].r, 8);
    L.tb[i] = off;
    off += (size_t)rup(ds[i].T * ldtb * 2, 256);
    L.t32[i] = off;
    off += (size_t)rup(ds[i].T * ldtb * 4, 256);
  }
  L.part = off;
  for (int i = 0; i < n; ++i)
    if (ds[i].flags == 0) L.part_bytes = std::max(L.part_bytes, gemm_tail_bytes(ds[i].T, ds[i].d_out));
  L.total = off + L.part_bytes;
  return L;
}

}  // namespace

bool prefill_group_ok(const DecodeLinear* ds, int n) {
  if (n < 2 || n > kMaxGemmGroup || ds[0].T < kBigT) return false;
  int64_t N[kMaxGemmGroup];
  for (int i = 0; i < n; ++i) {
    const DecodeLinear& d = ds[i];
    if (d.T != ds[0].T || d.x != ds[0].x || d.ldx != ds[0].ldx || d.d_in != ds[0].d_in) return false;
    if (d.force_fused || d.packed || (d.flags != 0 && d.flags != 1)) return false;
    if (!gemm_big_supported(d.ldx, d.ldu)) return false;
    if (d.flags == 1 && !d.t_io) return false;
    if (d.flags == 0 && (!prefill_accumulates(d) || (d.act && !prefill_act_ok(d)))) return false;
    N[i] = d.r;
  }
  // only where the members alone would leave CUs idle: the group fills at
  // most one round of tiles
  return gemm_group_tiles(N, n, ds[0].T) <= 256;
}

size_t prefill_group_workspace_bytes(const DecodeLinear* ds, int n) {
  return group_layout(ds, n).total;
}

hipError_t prefill_group_bf16(const DecodeLinear* ds, int n, hipStream_t st) {
  if (!prefill_group_ok(ds, n)) return hipErrorInvalidValue;
  const GroupLayout L = group_layout(ds, n);
  uint8_t* ws = static_cast<uint8_t*>(ds[0].workspace);
  GemmMember g[kMaxGemmGroup];
  for (int i = 0; i < n; ++i) {
    const DecodeLinear& d = ds[i];
    if (d.flags == 1) {
      g[i] = GemmMember{d.Ut, d.ldu, d.t_io, d.ldt, nullptr, 0, d.r};
    } else {
      const int64_t ldtb = rup(d.r, 8);
      float* t32 = d.t_io ? d.t_io : reinterpret_cast<float*>(ws + L.t32[i]);
      g[i] = GemmMember{d.Ut, d.ldu, t32, d.t_io ? d.ldt : ldtb,
                        reinterpret_cast<uint16_t*>(ws + L.tb[i]), ldtb, d.r};
    }
  }
  hipError_t e = gemm_nt_big_group(ds[0].x, ds[0].ldx, g, n, ds[0].T, ds[0].d_in, st);
  for (int i = 0; i < n && e == hipSuccess; ++i)
    if (ds[i].flags == 0)
      e = big_stage2(ds[i], reinterpret_cast<const uint16_t*>(ws + L.tb[i]), rup(ds[i].r, 8),
                     reinterpret_cast<float*>(ws + L.part), L.part_bytes, st);
  return e;
}

bool prefill_accumulates(const DecodeLinear& d) {
  return d.T >= kBigT && gemm_big_supported(d.ldx, d.ldu) && gemm_big_supported(rup(d.r, 8), d.ldv);
}

bool prefill_act_ok(const DecodeLinear& d) {
  const auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return prefill_accumulates(d) && d.y && a16(d.y) && d.ldy % 8 == 0 &&
         (d.act != 1 || (d.glu && a16(d.glu) && d.ldglu % 8 == 0));
}

bool prefill_fused_supported(const DecodeLinear& d) {
  // buffer-load offsets are 32-bit: the fused kernel needs every operand
  // (plus one tile of rows past its end) under 2 GiB
  const bool small = (d.T + kBM) * d.ldx * 2 < (1ll << 31) &&
                     (d.r + 128) * d.ldu * 2 < (1ll << 31) &&
                     (d.d_out + 512) * d.ldv * 2 < (1ll << 31);
  return d.flags == 0 && d.t_io == nullptr && !d.y_acc && !d.act && fused_fits(d.r) && small;
}

hipError_t prefill_linear_bf16(const DecodeLinear& d, hipStream_t st) {
  if (d.act && !prefill_act_ok(d)) return hipErrorInvalidValue;
  if (d.force_fused && !prefill_fused_supported(d)) return hipErrorInvalidValue;
  if (!d.force_fused && prefill_accumulates(d)) return prefill_big(d, st);
  if (d.y_acc) return hipErrorInvalidValue;
  if (prefill_fused_supported(d)) {
    FusedArgs f{};
    f.x = static_cast<const uint16_t*>(d.x);
    f.ldx = d.ldx;
    f.ut = static_cast<const uint16_t*>(d.Ut);
    f.ldu = d.ldu;
    f.vt = static_cast<const uint16_t*>(d.Vt);
    f.ldv = d.ldv;
    f.y = static_cast<uint16_t*>(d.y);
    f.ldy = d.ldy;
    f.M = (int)d.T;
    f.d_in = (int)d.d_in;
    f.r = (int)d.r;
    f.d_out = (int)d.d_out;
    f.r_pad = (int)rup(d.r, 32);
    const size_t lds = fused_lds_bytes(d.r);
    static std::once_flag lds_once;  // raise the dynamic-LDS limit once per process
    std::call_once(lds_once, [] {
      (void)hipFuncSetAttribute((const void*)fused_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    });
    hipLaunchKernelGGL(fused_kernel, dim3((unsigned)((d.T + kBM - 1) / kBM)), dim3(256), lds, st, f);
    return hipGetLastError();
  }

  // Unfused: stage 1 into fp32 t_io (stage-1-only / t requested) or bf16
  // workspace, then stage 2 from it.
  hipError_t e = hipSuccess;
  const int64_t ldtb = rup(d.r, 8);
  uint16_t* tws = parked_t(d.workspace);
  if (d.flags != 2) {
    GemmArgs g{};
    g.a = d.x;
    g.lda = d.ldx;
    g.b = static_cast<const uint16_t*>(d.Ut);
    g.ldb = d.ldu;
    g.M = (int)d.T;
    g.N = (int)d.r;
    g.K = (int)d.d_in;
    if (d.t_io) {
      g.c = d.t_io;
      g.ldc = d.ldt;
      e = launch_gemm<false, true>(g, st);
    } else {
      g.c = tws;
      g.ldc = ldtb;
      e = launch_gemm<false, false>(g, st);
    }
    if (e != hipSuccess || d.flags == 1) return e;
  }
  GemmArgs g{};
  if (d.t_io) {
    g.a = d.t_io;
    g.lda = d.ldt;
  } else {
    g.a = tws;
    g.lda = ldtb;
  }
  g.b = static_cast<const uint16_t*>(d.Vt);
  g.ldb = d.ldv;
  g.c = d.y;
  g.ldc = d.ldy;
  g.M = (int)d.T;
  g.N = (int)d.d_out;
  g.K = (int)d.r;
  return d.t_io ? launch_gemm<true, false>(g, st) : launch_gemm<false, false>(g, st);
}

}  // namespace lr
