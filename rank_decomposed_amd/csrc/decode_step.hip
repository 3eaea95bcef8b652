// One decode step of a decoder layer whose linears are all decomposed, with a
// paged cache of rank-r latents that is reconstructed every step.
//
// DeInfer/en §1 (third bottleneck) and §2.C: decomposed models rebuild the KV
// cache while decoding by multiplying the cached low-rank rows by the upward
// projections; to keep that inside a static graph, a preparation stage on the
// host builds a remapping index list, and the replayed graph copies the rows
// into a compact buffer at a fixed address and runs one large fixed-size GEMM.
// The layer around it is LLaMA-shaped (MHA/GQA, GLU MLP; DeInfer/en §2.D).
//
// Every grid here is sized from fixed capacities (B, cap, max_seq_rows), never
// from live lengths: live counts (n_valid, seq_off, pos, slot_mapping, remap)
// are read from device buffers, so one captured graph serves every step.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "lowrank.h"
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kAttnChunk = 256;  // cached rows per attention workgroup
constexpr int kPrefQB = 128;     // query tokens per prefill-attention workgroup (32 per wave)

int64_t rup(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// ---------------------------------------------------------------- rotary table
// table[p][i] = (cos(p * theta^(-2i/hd)), sin(...)), computed in double.
__global__ void rope_table_kernel(float* table, int64_t max_pos, int half, double theta) {
  const int64_t n = max_pos * half;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t p = e / half;
    const int i = (int)(e % half);
    const double inv = pow(theta, -2.0 * i / (2.0 * half));
    double s, c;
    sincos((double)p * inv, &s, &c);
    table[2 * e] = (float)c;
    table[2 * e + 1] = (float)s;
  }
}

// ---------------------------------------------------------------- RMSNorm
// x[b] = bf16(h[b] / sqrt(mean(h[b]^2) + eps) * g), one workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int64_t ldh,
                                                      const uint16_t* __restrict__ g,
                                                      uint16_t* __restrict__ x, int64_t ldx, int d,
                                                      float eps) {
  __shared__ float red[4];
  const float* row = h + (int64_t)blockIdx.x * ldh;
  uint16_t* out = x + (int64_t)blockIdx.x * ldx;
  // rows of whole 4-element groups (d, ldh, ldx multiples of 4, aligned
  // pointers): 16-byte loads and 8-byte stores; otherwise element by element
  const bool vec = (d & 3) == 0 && (ldh & 3) == 0 && (ldx & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(h) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(x) & 7) == 0 &&
                   (reinterpret_cast<uintptr_t>(g) & 7) == 0;
  float ss = 0.f;
  if (vec) {
    for (int c = threadIdx.x; c < d / 4; c += 256) {
      const f32x4 v = reinterpret_cast<const f32x4*>(row)[c];
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    }
  } else {
    for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(row[i], row[i], ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float scale = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
  if (vec) {
    for (int c = threadIdx.x; c < d / 4; c += 256) {
      const f32x4 v = reinterpret_cast<const f32x4*>(row)[c];
      const u32x2 gw = reinterpret_cast<const u32x2*>(g)[c];
      reinterpret_cast<u32x2*>(out)[c] =
          u32x2{pack_bf2(v.x * scale * bf2f(gw.x & 0xffffu), v.y * scale * bf2f(gw.x >> 16)),
                pack_bf2(v.z * scale * bf2f(gw.y & 0xffffu), v.w * scale * bf2f(gw.y >> 16))};
    }
  } else {
    for (int i = threadIdx.x; i < d; i += 256)
      out[i] = (uint16_t)f2bf(row[i] * scale * bf2f(g[i]));
  }
}

// The same per row for rows of whole 4-element groups (the vec case above):
// one wave per row with the row held in registers, NV 16-byte chunks per
// lane, all of a lane's loads in flight at once and h read once.  Each
// lane's squares fold in the order of rmsnorm_kernel's threads.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_wave_kernel(const float* __restrict__ h,
                                                           int64_t ldh,
                                                           const uint16_t* __restrict__ g,
                                                           uint16_t* __restrict__ x, int64_t ldx,
                                                           int rows, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int b = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (b >= rows) return;
  const f32x4* row = reinterpret_cast<const f32x4*>(h + (int64_t)b * ldh);
  const int nc = d / 4;
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nc ? row[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float scale = 1.0f / sqrtf(ss / (float)d + eps);
  const u32x2* gw = reinterpret_cast<const u32x2*>(g);
  u32x2* out = reinterpret_cast<u32x2*>(x + (int64_t)b * ldx);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= nc) break;
    const u32x2 w = gw[c];
    out[c] = u32x2{pack_bf2(v[i].x * scale * bf2f(w.x & 0xffffu), v[i].y * scale * bf2f(w.x >> 16)),
                   pack_bf2(v[i].z * scale * bf2f(w.y & 0xffffu), v[i].w * scale * bf2f(w.y >> 16))};
  }
}

// RMSNorm of `rows` rows of h [rows, ldh] into x: the wave-per-row kernel
// where a row fits its registers (d <= 8192, whole 4-element groups, aligned
// rows) and the rows fill the chip (at 4096 rows of 4096: 21 against 23 us),
// else one workgroup per row (at 64 rows: 5 us, against 10 on 16 workgroups).
hipError_t launch_rmsnorm(const float* h, int64_t ldh, const uint16_t* g, uint16_t* x,
                          int64_t ldx, int64_t rows, int64_t d, float eps, hipStream_t st) {
  const bool vec = (d & 3) == 0 && (ldh & 3) == 0 && (ldx & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(h) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(x) & 7) == 0 &&
                   (reinterpret_cast<uintptr_t>(g) & 7) == 0;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int nv = (int)((d + 255) / 256);  // 16-byte chunks per lane
  if (rows < 1024)
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)rows), block, 0, st, h, ldh, g, x, ldx, (int)d, eps);
  else if (vec && nv <= 4)
    hipLaunchKernelGGL(rmsnorm_wave_kernel<4>, grid, block, 0, st, h, ldh, g, x, ldx, (int)rows, (int)d, eps);
  else if (vec && nv <= 8)
    hipLaunchKernelGGL(rmsnorm_wave_kernel<8>, grid, block, 0, st, h, ldh, g, x, ldx, (int)rows, (int)d, eps);
  else if (vec && nv <= 16)
    hipLaunchKernelGGL(rmsnorm_wave_kernel<16>, grid, block, 0, st, h, ldh, g, x, ldx, (int)rows, (int)d, eps);
  else if (vec && nv <= 24)
    hipLaunchKernelGGL(rmsnorm_wave_kernel<24>, grid, block, 0, st, h, ldh, g, x, ldx, (int)rows, (int)d, eps);
  else if (vec && nv <= 32)
    hipLaunchKernelGGL(rmsnorm_wave_kernel<32>, grid, block, 0, st, h, ldh, g, x, ldx, (int)rows, (int)d, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)rows), block, 0, st, h, ldh, g, x, ldx, (int)d, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------- append
// pool[slot[b], 0:r] = bf16(lat[b, 0:r]); out-of-range slots are skipped.
__global__ __launch_bounds__(256) void append_kernel(const float* __restrict__ lat, int64_t ldl,
                                                     int r, const int32_t* __restrict__ slot,
                                                     int64_t pool_rows, uint16_t* pool,
                                                     int64_t pool_ld) {
  const int b = blockIdx.x;
  const int64_t s = slot[b];
  if (s < 0 || s >= pool_rows) return;
  for (int j = threadIdx.x; j < r; j += 256)
    pool[s * pool_ld + j] = (uint16_t)f2bf(lat[(int64_t)b * ldl + j]);
}

// ---------------------------------------------------------------- residual add
// h[t, :] += y[t, :] (bf16 projection output into the fp32 residual).
__global__ __launch_bounds__(256) void add_residual_kernel(float* __restrict__ h,
                                                           const uint16_t* __restrict__ y,
                                                           int64_t n) {
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    h[e] += bf2f(y[e]);
}

// ---------------------------------------------------------------- ReLU
// m = max(z, 0) on bf16, the non-GLU MLP's activation (NaN passes through).
__global__ __launch_bounds__(256) void relu_kernel(const uint16_t* __restrict__ z,
                                                   uint16_t* __restrict__ m, int64_t n) {
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    m[e] = bf2f(z[e]) < 0.f ? (uint16_t)0 : z[e];
}

// ---------------------------------------------------------------- SiLU * up
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gate,
                                                       const uint16_t* __restrict__ up,
                                                       uint16_t* __restrict__ m, int64_t n) {
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const float gv = bf2f(gate[e]);
    const float s = gv / (1.0f + expf(-gv));
    m[e] = (uint16_t)f2bf(s * bf2f(up[e]));
  }
}

// ---------------------------------------------------------------- attention
// Partial softmax attention of one query (sequence i, head h) over one chunk
// of its packed rows [seq_off[i] + c*256, ...).  Output per chunk: running max
// m, sum l and unnormalised o[hd] (fp32).  K rows are already rotated.
//
// Rows are read coalesced: HD/8 lanes share a row, each holding 8 consecutive
// elements (16 bytes), so one wave instruction reads 64 * 16 contiguous bytes
// per row group.  A lane's slice of q stays in registers; a row's score is
// summed over its lanes by cross-lane shuffles, and the p-weighted V rows are
// summed per lane and then over the row groups in LDS.
// Rows the query of token i attends to: [beg, beg + n) of the packed
// buffer.  With tok_seq (a chunk of several tokens per sequence) token i
// belongs to sequence tok_seq[i] and sees its rows up to its own position
// (causal); without, token i is sequence i's new token and sees all its rows.
__device__ __forceinline__ void query_rows(const int32_t* seq_off, const int32_t* tok_seq,
                                           const int32_t* pos, int S, int i, int cap, int* beg,
                                           int* n) {
  int sq = tok_seq ? tok_seq[i] : i;
  sq = sq < 0 ? 0 : (sq >= S ? S - 1 : sq);
  const int b = seq_off[sq];
  *beg = b;
  *n = 0;
  if (b < 0 || b >= cap) return;          // offsets are device data: stay inside cap
  int len = seq_off[sq + 1] - b;
  if (tok_seq) len = min(len, pos[i] + 1);
  len = len < cap - b ? len : cap - b;
  *n = len < 0 ? 0 : len;
}

template <int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t ldkv, const int32_t* __restrict__ seq_off,
    const int32_t* __restrict__ tok_seq, int S, const int32_t* __restrict__ pos,
    const float* __restrict__ rope, int64_t max_pos, int H, int Hkv, int nch, int cap,
    float* __restrict__ part) {
  constexpr int HALF = HD / 2;
  constexpr int LPR = HD / 8;          // lanes per row
  constexpr int RG = 256 / LPR;        // row groups in the workgroup
  __shared__ float qs[HD];
  __shared__ float sc[kAttnChunk];
  __shared__ float red[256];
  __shared__ float opart[RG][HD + 4];
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  int beg, n;
  query_rows(seq_off, tok_seq, pos, S, i, cap, &beg, &n);
  const int r0 = c * kAttnChunk;
  if (r0 >= n) return;
  const int cnt = min(kAttnChunk, n - r0);
  const int kvh = h / (H / Hkv);
  // rotated, scaled query
  if (threadIdx.x < HALF) {
    int p = pos[i];
    p = p < 0 ? 0 : (p >= max_pos ? (int)max_pos - 1 : p);
    const float cs = rope[((int64_t)p * HALF + threadIdx.x) * 2];
    const float sn = rope[((int64_t)p * HALF + threadIdx.x) * 2 + 1];
    const float a = bf2f(q[(int64_t)i * ldq + h * HD + threadIdx.x]);
    const float b = bf2f(q[(int64_t)i * ldq + h * HD + threadIdx.x + HALF]);
    const float scale = 1.0f / sqrtf((float)HD);
    qs[threadIdx.x] = (a * cs - b * sn) * scale;
    qs[threadIdx.x + HALF] = (b * cs + a * sn) * scale;
  }
  __syncthreads();
  const int sub = threadIdx.x % LPR, grp = threadIdx.x / LPR;  // element slice, row group
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[sub * 8 + e];
  const uint16_t* kb = K + (int64_t)(beg + r0) * ldkv + kvh * HD + sub * 8;
  const uint16_t* vb = V + (int64_t)(beg + r0) * ldkv + kvh * HD + sub * 8;
  // scores: row group g takes rows g, g + RG, ...
#pragma unroll 4
  for (int r = grp; r < kAttnChunk; r += RG) {
    float acc = 0.f;
    if (r < cnt) {
      const u32x4 w = ldg16_stream(kb + (int64_t)r * ldkv);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf2f(ww[e] & 0xffffu), qv[2 * e], acc);
        acc = fmaf(bf2f(ww[e] >> 16), qv[2 * e + 1], acc);
      }
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, LPR);
    if (sub == 0) sc[r] = r < cnt ? acc : -INFINITY;
  }
  __syncthreads();
  const float s = sc[threadIdx.x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + k]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();
  const float pexp = ((int)threadIdx.x < cnt) ? expf(s - m) : 0.f;
  sc[threadIdx.x] = pexp;
  red[threadIdx.x] = pexp;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  const float l = red[0];
  // o = sum_r p_r V_r: each lane sums its 8 elements over its group's rows
  float ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = grp; r < cnt; r += RG) {
    const u32x4 w = ldg16_stream(vb + (int64_t)r * ldkv);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const float pr = sc[r];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ov[2 * e] = fmaf(pr, bf2f(ww[e] & 0xffffu), ov[2 * e]);
      ov[2 * e + 1] = fmaf(pr, bf2f(ww[e] >> 16), ov[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) opart[grp][sub * 8 + e] = ov[e];
  __syncthreads();
  float* out = part + (((int64_t)i * H + h) * nch + c) * (HD + 2);
  if (threadIdx.x < HD) {
    float acc = 0.f;
#pragma unroll 8
    for (int gg = 0; gg < RG; ++gg) acc += opart[gg][threadIdx.x];
    out[2 + threadIdx.x] = acc;
  }
  if (threadIdx.x == 0) {
    out[0] = m;
    out[1] = l;
  }
}

// ---------------------------------------------------------------- prefill attention
// tok_off[i] = first new token of sequence i (tokens come sequence by
// sequence), tok_off[S] = T; a sequence without tokens gets an empty range.
// blk_off[i] = first kPrefQB-token query block of sequence i when the blocks of
// all sequences are numbered in order, blk_off[S] = their count.  One
// workgroup.
__global__ __launch_bounds__(256) void tok_offsets_kernel(const int32_t* __restrict__ tok_seq,
                                                          int T, int S,
                                                          int32_t* __restrict__ tok_off,
                                                          int32_t* __restrict__ blk_off) {
  for (int i = threadIdx.x; i <= S; i += 256) tok_off[i] = -1;
  __syncthreads();
  // a contiguous run of tokens per thread, its loads unrolled
  const int per = (T + 255) / 256, tb = threadIdx.x * per, te = min(T, tb + per);
  int prev = tb > 0 && tb < T ? tok_seq[tb - 1] : -1;
#pragma unroll 8
  for (int t = tb; t < te; ++t) {
    const int sq = tok_seq[t];
    if (sq >= 0 && sq < S && (t == 0 || prev != sq)) tok_off[sq] = t;
    prev = sq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    tok_off[S] = T;
    for (int i = S - 1; i >= 0; --i)
      if (tok_off[i] < 0 || tok_off[i] > tok_off[i + 1]) tok_off[i] = tok_off[i + 1];
    int nb = 0;
    for (int i = 0; i < S; ++i) {
      blk_off[i] = nb;
      nb += (tok_off[i + 1] - tok_off[i] + kPrefQB - 1) / kPrefQB;
    }
    blk_off[S] = nb;
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D = A(32x16) * B(16x32) + C on bf16 inputs: lane l supplies row (l % 32)
// of A / column (l % 32) of B with the k-group 8 * (l / 32) .. + 7; lane l
// holds D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32], v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Causal attention of a chunk of new tokens on MFMA 32x32x16 (flash style).
//
// Work split: a workgroup takes one (head h, 128-token query block) pair,
// 32 tokens per wave, and walks its sequence's reconstructed K/V rows in
// 64-row tiles up to the block's last position.  The pairs are listed head
// by head (nbpad slots per head; blk_off numbers the blocks of all sequences)
// and each XCD (workgroup id % 8) takes a contiguous range of the list, so
// the blocks that read the same K/V rows share one L2; within a sequence the
// later blocks, which walk more tiles, start first.
//
// Per tile a wave forms S^T = K Q^T, so that a lane holds 32 keys of its own
// query: the causal mask, the running max m and sum l (base-2 softmax, the
// scale log2(e)/sqrt(hd) folded into Q) stay in the lane but for one
// exchange between the two lane halves.  The probabilities P^T then serve
// directly as the B operand of O^T += V^T P^T: the MFMA's contraction runs
// over the keys in the order the S^T layout leaves them in the lane (4
// consecutive keys, a gap of 4, 4 more), and V^T is staged in LDS in 8-byte
// units of 4 consecutive keys of one column, so each A fragment is two
// 8-byte reads.  K stays row-major in LDS (one 16-byte read per fragment).
// The next tile's K/V rows are loaded into registers while the current one
// multiplies.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t ldkv, const int32_t* __restrict__ seq_off,
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ blk_off, int S, int nbpad,
    const int32_t* __restrict__ pos, const float* __restrict__ rope, int64_t max_pos, int H,
    int Hkv, int cap, uint16_t* __restrict__ o, int64_t ldo) {
  constexpr int KS = HD / 16;        // k-steps of S^T = K Q^T
  constexpr int DB = HD / 32;        // 32-row blocks of O^T
  constexpr int KP = HD + 8;         // K tile pitch (elements)
  constexpr int VROW = HD + HD / 8;  // 8-byte V^T units per key group (column d at d + d / 8)
  __shared__ __attribute__((aligned(16))) uint16_t ktile[64 * KP];
  __shared__ __attribute__((aligned(16))) u32x2 vtile[16 * VROW];
  const int nitems = H * nbpad, per_xcd = (nitems + 7) / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if ((int)blockIdx.x / 8 >= per_xcd || item >= nitems) return;
  const int h = item / nbpad, gb = item % nbpad;
  if (gb >= blk_off[S]) return;
  int sq = 0, hi = S;  // the sequence: the last i with blk_off[i] <= gb
  while (hi - sq > 1) {
    const int mid = (sq + hi) >> 1;
    if (blk_off[mid] <= gb) sq = mid; else hi = mid;
  }
  const int b = blk_off[sq + 1] - 1 - gb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int t0 = tok_off[sq], t1 = tok_off[sq + 1];
  const int qt0 = t0 + b * kPrefQB;
  if (qt0 >= t1) return;
  const int beg = seq_off[sq];
  if (beg < 0 || beg >= cap) return;      // offsets are device data: stay inside cap
  int rows = seq_off[sq + 1] - beg;
  rows = rows < cap - beg ? rows : cap - beg;
  if (rows <= 0) return;
  int plast = pos[min(qt0 + kPrefQB - 1, t1 - 1)];
  plast = plast < 0 ? 0 : (plast >= rows ? rows - 1 : plast);
  const int nkt = (plast + 64) / 64;
  const int kvh = h / (H / Hkv);
  const float qscale = 1.4426950408889634f / sqrtf((float)HD);

  // this lane's query (column of S^T and O^T); rows past the chunk see key 0
  const int tq = qt0 + 32 * wave + (lane & 31);
  int rp = tq < t1 ? pos[tq] : 0;
  rp = rp < 0 ? 0 : rp;
  // Q fragments: elements 16 ks + 8 half .. + 7 of the lane's query; rotary
  // pairs (i, i + HD/2) sit in k-steps ks and ks + KS/2 of the same lane
  u32x4 qf[KS];
  {
    const bool ok = tq < t1;
    int p = ok ? pos[tq] : 0;
    p = p < 0 ? 0 : (p >= max_pos ? (int)max_pos - 1 : p);
    float v[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = ok ? ldg16(q + (int64_t)tq * ldq + h * HD + ks * 16 + 8 * half)
                         : u32x4{0, 0, 0, 0};
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[ks][2 * e] = bf2f(ww[e] & 0xffffu);
        v[ks][2 * e + 1] = bf2f(ww[e] >> 16);
      }
    }
    const float* tb = rope + (int64_t)p * HD;  // (cos, sin) of frequency i at 2i
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = ks * 16 + 8 * half + e;
        const float c = tb[2 * i], sn = tb[2 * i + 1];
        const float a0 = v[ks][e], b0 = v[ks + KS / 2][e];
        v[ks][e] = a0 * c - b0 * sn;
        v[ks + KS / 2][e] = b0 * c + a0 * sn;
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = u32x4{pack_bf2(v[ks][0] * qscale, v[ks][1] * qscale),
                     pack_bf2(v[ks][2] * qscale, v[ks][3] * qscale),
                     pack_bf2(v[ks][4] * qscale, v[ks][5] * qscale),
                     pack_bf2(v[ks][6] * qscale, v[ks][7] * qscale)};
  }
  float m = -INFINITY, l = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // tile staging: K as 16-byte row chunks; V as (key group of 4 rows, 8-column
  // chunk) items, each transposed into 8 units on the way to LDS
  constexpr int KN = 64 * HD / 8 / 256, VITEMS = 16 * (HD / 8);
  const int vg = threadIdx.x / (HD / 8), vch = threadIdx.x % (HD / 8);
  u32x4 kreg[KN], vreg[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = threadIdx.x + 256 * i, r = c / (HD / 8), ch = c % (HD / 8), j = kt * 64 + r;
      kreg[i] = j < rows ? ldg16(K + (int64_t)(beg + j) * ldkv + kvh * HD + ch * 8)
                         : u32x4{0, 0, 0, 0};
    }
    if ((int)threadIdx.x < VITEMS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = kt * 64 + 4 * vg + u;
        vreg[u] = j < rows ? ldg16(V + (int64_t)(beg + j) * ldkv + kvh * HD + vch * 8)
                           : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KN; ++i) {
      const int c = threadIdx.x + 256 * i, r = c / (HD / 8), ch = c % (HD / 8);
      *reinterpret_cast<u32x4*>(ktile + r * KP + ch * 8) = kreg[i];
    }
    if ((int)threadIdx.x < VITEMS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t k0 = (vreg[0][e >> 1] >> sh) & 0xffffu, k1 = (vreg[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t k2 = (vreg[2][e >> 1] >> sh) & 0xffffu, k3 = (vreg[3][e >> 1] >> sh) & 0xffffu;
        const int d = vch * 8 + e;
        vtile[vg * VROW + d + (d >> 3)] = u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
      }
    }
  };
  load_tile(0);

  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1);  // in flight while this tile multiplies
    // S^T over the tile's 64 keys: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(ktile + (kb * 32 + (lane & 31)) * KP +
                                                         ks * 16 + 8 * half);
        sacc[kb] = mfma32x32x16(kf, qf[ks], sacc[kb]);
      }
    }
    // causal mask and online softmax: register v of block kb is key
    // kt*64 + 32 kb + 8 (v / 4) + 4 half + v % 4 of the lane's query
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kt * 64 + kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        const float s = (j <= rp && j < rows) ? sacc[kb][v] : -INFINITY;
        sacc[kb][v] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 while m is still -inf
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][v] - mn);
        sacc[kb][v] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    // O^T += V^T P^T, 16 keys per step: P^T registers 8 kk .. 8 kk + 7 of a
    // block are keys 16 kk + {0..3, 8..11} + 4 half, the V^T units of key
    // groups 4 kk + half and 4 kk + 2 + half of the block
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f32x16& pv = sacc[kb];
        const u32x4 pf = u32x4{pack_bf2(pv[8 * kk + 0], pv[8 * kk + 1]),
                               pack_bf2(pv[8 * kk + 2], pv[8 * kk + 3]),
                               pack_bf2(pv[8 * kk + 4], pv[8 * kk + 5]),
                               pack_bf2(pv[8 * kk + 6], pv[8 * kk + 7])};
        const int g0 = 8 * kb + 4 * kk + half;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + (lane & 31);
          const u32x2 lo = vtile[g0 * VROW + d + (d >> 3)];
          const u32x2 hi2 = vtile[(g0 + 2) * VROW + d + (d >> 3)];
          oacc[db] = mfma32x32x16(u32x4{lo.x, lo.y, hi2.x, hi2.y}, pf, oacc[db]);
        }
      }
  }
  if (tq >= t1) return;
  const float inv = 1.0f / l;
  uint16_t* orow = o + (int64_t)tq * ldo + h * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = db * 32 + 8 * rq + 4 * half;
      *reinterpret_cast<u32x2*>(orow + d) =
          u32x2{pack_bf2(oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv),
                pack_bf2(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv)};
    }
}

// Combine the chunks of (sequence i, head h): o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
template <int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(const float* __restrict__ part, int H,
                                                          int nch,
                                                          const int32_t* __restrict__ seq_off,
                                                          const int32_t* __restrict__ tok_seq,
                                                          int S, const int32_t* __restrict__ pos,
                                                          int cap, uint16_t* __restrict__ o,
                                                          int64_t ldo) {
  const int h = blockIdx.x, i = blockIdx.y;
  int beg, n;
  query_rows(seq_off, tok_seq, pos, S, i, cap, &beg, &n);
  int used = (n + kAttnChunk - 1) / kAttnChunk;
  used = used < 0 ? 0 : (used > nch ? nch : used);
  const float* base = part + ((int64_t)i * H + h) * nch * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < used; ++c) M = fmaxf(M, base[(int64_t)c * (HD + 2)]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < used; ++c) {
    const float* pc = base + (int64_t)c * (HD + 2);
    const float w = expf(pc[0] - M);
    L = fmaf(w, pc[1], L);
    acc = fmaf(w, pc[2 + threadIdx.x], acc);
  }
  o[(int64_t)i * ldo + h * HD + threadIdx.x] = (uint16_t)f2bf(used > 0 ? acc / L : 0.f);
}

// ---------------------------------------------------------------- fused decode attention
// blk_off[i] = first 256-row block of sequence i's rows [seq_off[i],
// seq_off[i+1]) (clamped to cap), blocks numbered sequence by sequence;
// blk_off[S] = their count.  One thread.
__global__ void row_blocks_kernel(const int32_t* __restrict__ seq_off, int S, int cap,
                                  int32_t* __restrict__ blk_off) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int nb = 0;
  for (int i = 0; i < S; ++i) {
    blk_off[i] = nb;
    const int b = seq_off[i], e = min(seq_off[i + 1], cap);
    const int n = (b < 0 || b >= cap || e < b) ? 0 : e - b;
    nb += (n + 255) / 256;
  }
  blk_off[S] = nb;
}

// o[i, h] from the block partials of sequence i, each (m_b, l_b, w_b) with w_b
// the block's p-weighted sum of V latent rows (r_v wide):
//   o = (sum_b e^(m_b - M) w_b) V_v^T / sum_b e^(m_b - M) l_b
// over the rows of kv head h / (H / Hkv) of V_v^T.  Up to 64 blocks at a
// time, thread j takes block j: the maximum M by wave shuffles, the weights
// e^(m_b - M) and the l_b into LDS, the sum L in block order; then each thread's
// latent sums with four blocks' loads in flight.  Thread t then takes output
// column t / 4 and every fourth 8-wide step of r_v (t % 4), summed by two
// shuffles.  Blocks past nbpad (only from corrupt offsets) are skipped.
template <int HD>
__global__ __launch_bounds__(4 * HD) void fused_combine_kernel(
    const float* __restrict__ part, int H, int Hkv, int rv, const int32_t* __restrict__ blk_off,
    int nbpad, const uint16_t* __restrict__ vt, int64_t ldv, uint16_t* __restrict__ o,
    int64_t ldo) {
  extern __shared__ float vec[];  // [rv]
  __shared__ float wb[64], wl[64];
  __shared__ float msh[2];
  const int h = blockIdx.x, i = blockIdx.y, kvh = h / (H / Hkv);
  const int b0 = max(0, blk_off[i]), b1 = min(nbpad, blk_off[i + 1]);
  const int64_t pw = rv + 2, bs = (int64_t)H * pw;
  const float* ph = part + (int64_t)h * pw;  // block b: m at ph[b * bs], l at + 1, sums from + 2
  const int tid = (int)threadIdx.x;
  // the maximum over the blocks (wave 0, 64 blocks per pass)
  if (tid < 64) {
    float M = -INFINITY;
    for (int c0 = b0; c0 < b1; c0 += 64)
      if (c0 + tid < b1) M = fmaxf(M, ph[(c0 + tid) * bs]);
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
    if (tid == 0) msh[0] = M;
  }
  __syncthreads();
  const float M = msh[0];
  float L = 0.f;  // thread 0's sum, in block order
  float acc = 0.f;
  const int n = tid;  // this thread's latent element (rv <= 4 * HD; larger rv: the loop below)
  for (int c0 = b0; c0 < b1; c0 += 64) {
    const int nb = min(64, b1 - c0);
    __syncthreads();  // the previous weights are consumed
    if (tid < nb) {
      wb[tid] = expf(ph[(c0 + tid) * bs] - M);
      wl[tid] = ph[(c0 + tid) * bs + 1];
    }
    __syncthreads();
    if (tid == 0)
      for (int j = 0; j < nb; ++j) L = fmaf(wb[j], wl[j], L);
    if (n < rv) {
      const float* pc = ph + c0 * bs + 2 + n;
      int j = 0;
      for (; j + 4 <= nb; j += 4) {
        const float x0 = pc[j * bs], x1 = pc[(j + 1) * bs], x2 = pc[(j + 2) * bs],
                    x3 = pc[(j + 3) * bs];
        acc = fmaf(wb[j], x0, acc);
        acc = fmaf(wb[j + 1], x1, acc);
        acc = fmaf(wb[j + 2], x2, acc);
        acc = fmaf(wb[j + 3], x3, acc);
      }
      for (; j < nb; ++j) acc = fmaf(wb[j], pc[j * bs], acc);
    }
    // latent elements past the block size (rv > 4 * HD), one block at a time
    for (int n2 = n + (int)blockDim.x; n2 < rv; n2 += blockDim.x) {
      float a2 = c0 == b0 ? 0.f : vec[n2];
      for (int j = 0; j < nb; ++j) a2 = fmaf(wb[j], ph[(c0 + j) * bs + 2 + n2], a2);
      vec[n2] = a2;
    }
  }
  if (n < rv) vec[n] = acc;
  if (tid == 0) msh[1] = L;
  __syncthreads();
  const int c = tid >> 2, qtr = tid & 3;
  const uint16_t* row = vt + (int64_t)(kvh * HD + c) * ldv;
  float ac = 0.f;
#pragma unroll 4
  for (int k = qtr * 8; k < rv; k += 32) {
    if (k + 8 <= rv) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + k);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ac = fmaf(vec[k + 2 * e], bf2f(ww[e] & 0xffffu), ac);
        ac = fmaf(vec[k + 2 * e + 1], bf2f(ww[e] >> 16), ac);
      }
    } else {
      for (int e = k; e < rv; ++e) ac = fmaf(vec[e], bf2f(row[e]), ac);
    }
  }
  ac += __shfl_xor(ac, 1);
  ac += __shfl_xor(ac, 2);
  if (qtr == 0) o[(int64_t)i * ldo + h * HD + c] = (uint16_t)f2bf(b1 > b0 ? ac / msh[1] : 0.f);
}

// fused_combine_kernel for NS = 4 * HD / 64 consecutive sequences at once, one
// wave each (sequence blockIdx.y * NS + wave), so the V_v rows of head h's kv
// head are read once for all of them: each wave finds its sequence's maximum
// by shuffles, puts the weights e^(m_b - M) and the l_b of up to 64 blocks at
// a time in its LDS slots, sums L in block order (lane 0), and accumulates its
// latent sums (lane: elements lane, lane + 64, ... of r_v, 8 at a time) with
// four blocks' loads in flight per element; then every thread takes one
// output column and quarter of r_v for every sequence (four steps of V_v in
// flight).  Each sequence's sums follow
// fused_combine_kernel's order, so both give the same bits.  The latent sums
// take NS * round_up(rv, 4) * 4 bytes of LDS (rows of whole 16-byte chunks, so
// the V_v step reads each sequence's 8 values as two 16-byte loads).
template <int HD>
__global__ __launch_bounds__(4 * HD) void fused_combine_group_kernel(
    const float* __restrict__ part, int H, int Hkv, int rv, const int32_t* __restrict__ blk_off,
    int nbpad, int S, const uint16_t* __restrict__ vt, int64_t ldv, uint16_t* __restrict__ o,
    int64_t ldo) {
  constexpr int NS = 4 * HD / 64;
  extern __shared__ float vec[];  // [NS][ldv4]
  const int ldv4 = (rv + 3) & ~3;
  __shared__ float wb[NS][64], wl[NS][64], Ls[NS];
  __shared__ int live[NS];
  const int h = blockIdx.x, kvh = h / (H / Hkv);
  const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i0 = (int)blockIdx.y * NS, i = i0 + wv;
  const int64_t pw = rv + 2, bs = (int64_t)H * pw;
  const float* ph = part + (int64_t)h * pw;  // block b: m at ph[b * bs], l at + 1, sums from + 2
  if (i < S) {
    float* myv = vec + (int64_t)wv * ldv4;
    const int b0 = max(0, blk_off[i]), b1 = min(nbpad, blk_off[i + 1]);
    float M = -INFINITY;
    for (int c0 = b0; c0 < b1; c0 += 64)
      if (c0 + lane < b1) M = fmaxf(M, ph[(c0 + lane) * bs]);
#pragma unroll
    for (int sft = 32; sft > 0; sft >>= 1) M = fmaxf(M, __shfl_xor(M, sft));
    float L = 0.f;
    for (int c0 = b0; c0 < b1; c0 += 64) {
      const int nb = min(64, b1 - c0);
      if (lane < nb) {
        wb[wv][lane] = expf(ph[(c0 + lane) * bs] - M);
        wl[wv][lane] = ph[(c0 + lane) * bs + 1];
      }
      // the reads below take other lanes' writes: LDS runs one wave's accesses in order
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
      if (lane == 0)
        for (int j = 0; j < nb; ++j) L = fmaf(wb[wv][j], wl[wv][j], L);
      const float* pc = ph + c0 * bs + 2;
      for (int nc = 0; nc < rv; nc += 512) {
        float acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int n = nc + 64 * k + lane;
          acc[k] = c0 == b0 || n >= rv ? 0.f : myv[n];
        }
        int j = 0;
        for (; j + 4 <= nb; j += 4) {
          float x[4][8];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int n = nc + 64 * k + lane;
              x[jj][k] = n < rv ? pc[(j + jj) * bs + n] : 0.f;
            }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = fmaf(wb[wv][j + jj], x[jj][k], acc[k]);
        }
        for (; j < nb; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int n = nc + 64 * k + lane;
            acc[k] = fmaf(wb[wv][j], n < rv ? pc[j * bs + n] : 0.f, acc[k]);
          }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int n = nc + 64 * k + lane;
          if (n < rv) myv[n] = acc[k];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // this chunk's slots are read before the next overwrites them
      asm volatile("" ::: "memory");
    }
    if (lane == 0) {
      Ls[wv] = L;
      live[wv] = b1 > b0;
    }
  }
  __syncthreads();
  const int c = tid >> 2, qtr = tid & 3;
  const uint16_t* row = vt + (int64_t)(kvh * HD + c) * ldv;
  const int ns = min(NS, S - i0);
  float ac[NS];
#pragma unroll
  for (int si = 0; si < NS; ++si) ac[si] = 0.f;
#pragma unroll 4
  for (int k = qtr * 8; k < rv; k += 32) {
    if (k + 8 <= rv) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + k);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int si = 0; si < NS; ++si) {
        if (si >= ns) break;
        const f32x4* v4 = reinterpret_cast<const f32x4*>(vec + (int64_t)si * ldv4 + k);
        const f32x4 va = v4[0], vb = v4[1];
        const float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ac[si] = fmaf(v[2 * e], bf2f(ww[e] & 0xffffu), ac[si]);
          ac[si] = fmaf(v[2 * e + 1], bf2f(ww[e] >> 16), ac[si]);
        }
      }
    } else {
#pragma unroll
      for (int si = 0; si < NS; ++si) {
        if (si >= ns) break;
        for (int e = k; e < rv; ++e) ac[si] = fmaf(vec[(int64_t)si * ldv4 + e], bf2f(row[e]), ac[si]);
      }
    }
  }
#pragma unroll
  for (int si = 0; si < NS; ++si) {
    if (si >= ns) break;
    float a = ac[si];
    a += __shfl_xor(a, 1);
    a += __shfl_xor(a, 2);
    if (qtr == 0)
      o[(int64_t)(i0 + si) * ldo + h * HD + c] = (uint16_t)f2bf(live[si] ? a / Ls[si] : 0.f);
  }
}

// ---------------------------------------------------------------- workspace
// One layer step over T new tokens in S sequences: the decode step (one new
// token per sequence, tok_seq null) and the chunked-prefill step share it.
struct StepIn {
  void* k_pool;
  void* v_pool;
  int64_t pool_rows, pool_ld;
  const int32_t* slot_mapping;  // [T]
  const int32_t* remap;         // [cap]
  const int32_t* seq_off;       // [S + 1]
  const int32_t* tok_seq;       // [T] or null (token i is sequence i's)
  const int32_t* pos;           // [T]
  const int32_t* n_valid;
  int64_t T, S, cap, max_seq_rows;
};

StepIn from_decode(const lr_decode_state* s) {
  return StepIn{s->k_pool, s->v_pool,  s->pool_rows, s->pool_ld, s->slot_mapping, s->remap,
                s->seq_off, nullptr,   s->pos,       s->n_valid, s->B,            s->B,
                s->cap,     s->max_seq_rows};
}

StepIn from_prefill(const lr_prefill_state* s) {
  return StepIn{s->k_pool,   s->v_pool, s->pool_rows, s->pool_ld, s->slot_mapping, s->remap,
                s->seq_off,  s->tok_seq, s->pos,      s->n_valid, s->T,            s->S,
                s->cap,      s->max_seq_rows};
}

// Projections of up to 64 tokens run on the decode path (streamed weights,
// grouped launches); more tokens take the prefill path.
constexpr int64_t kDecodeTokens = 64;

struct StepLayout {
  size_t lin, x, q, latk, latv, kbuf, vbuf, krec, vrec, part, o, gate, up, m, yb, tok_off, total;
  int64_t rk_ld, rv_ld, dkv, nch, nbpad;
};

// fused: decode attention with the reconstruction on chip (no reconstructed
// K/V buffers; block partials instead of chunk partials)
StepLayout step_layout(const lr_layer_weights* w, const StepIn& s, bool fused = false) {
  StepLayout L{};
  const int64_t T = s.T, d = w->d_model, dq = w->n_heads * w->head_dim;
  const bool dec = T <= kDecodeTokens;
  L.dkv = w->n_kv_heads * w->head_dim;
  L.rk_ld = rup(w->r[1], 8);
  L.rv_ld = rup(w->r[2], 8);
  L.nch = (s.max_seq_rows + kAttnChunk - 1) / kAttnChunk;
  const int64_t din[7] = {d, d, d, dq, d, d, w->d_ffn};
  const int64_t dout[7] = {dq, L.dkv, L.dkv, d, w->d_ffn, w->d_ffn, d};
  size_t lin = 0;
  if (dec) {
    // the projections' scratch: q,k,v and gate,up go out as groups
    DecodeLinear g[7];
    for (int k = 0; k < 7; ++k) g[k] = DecodeLinear{T, din[k], w->r[k], dout[k]};
    lin = decode_group_workspace_bytes(g, 3);
    lin = std::max(lin, w->mlp == LR_MLP_RELU ? decode_workspace_bytes(T, din[4], w->r[4], dout[4])
                                              : decode_group_workspace_bytes(g + 4, 2));
    lin = std::max(lin, decode_workspace_bytes(T, din[3], w->r[3], dout[3]));
    lin = std::max(lin, decode_workspace_bytes(T, din[6], w->r[6], dout[6]));
  } else {
    for (int k = 0; k < 7; ++k)
      if (!(k == 5 && w->mlp == LR_MLP_RELU))
        lin = std::max(lin, prefill_workspace_bytes(T, w->r[k], dout[k]));
    // stage 1 of q, k, v (k, v: the latents only) and of gate, up as groups
    DecodeLinear g[3];
    for (int k = 0; k < 3; ++k) g[k] = DecodeLinear{T, din[k], w->r[k], dout[k]};
    g[1].flags = g[2].flags = 1;
    lin = std::max(lin, prefill_group_workspace_bytes(g, 3));
    for (int k = 0; k < 2; ++k) g[k] = DecodeLinear{T, din[4 + k], w->r[4 + k], dout[4 + k]};
    lin = std::max(lin, prefill_group_workspace_bytes(g, 2));
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = rup(off + bytes, 256);
    return at;
  };
  L.lin = take(lin);  // first: zero-filled once by the caller, kept zero by the kernels
  L.x = take(T * d * 2);
  L.q = take(T * dq * 2);
  L.latk = take(T * w->r[1] * 4);
  L.latv = take(T * w->r[2] * 4);
  L.kbuf = take(s.cap * L.rk_ld * 2);
  L.vbuf = take(s.cap * L.rv_ld * 2);
  L.nbpad = (s.cap + 255) / 256 + s.S;
  L.krec = fused ? 0 : take(s.cap * L.dkv * 2);
  L.vrec = fused ? 0 : take(s.cap * L.dkv * 2);
  L.part = fused ? take(L.nbpad * w->n_heads * (w->r[2] + 2) * 4)
                 : take(T * w->n_heads * L.nch * (w->head_dim + 2) * 4);
  L.o = take(T * dq * 2);
  L.gate = take(T * w->d_ffn * 2);
  L.up = w->mlp == LR_MLP_RELU ? L.gate : take(T * w->d_ffn * 2);
  L.m = take(T * w->d_ffn * 2);
  L.yb = dec ? L.m : take(T * d * 2);  // prefill path: o / down output before the residual add
  L.tok_off = take(2 * (s.S + 1) * 4);  // chunked prefill: first token and first
                                        // query block of each sequence
  L.total = off;
  return L;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

lr_status check_step(const lr_layer_weights* w, const StepIn& s, const float* h) {
  if (!w || !h) return LR_ERR_ARG;
  if (w->d_model <= 0 || w->n_heads <= 0 || w->n_kv_heads <= 0 || w->d_ffn <= 0) return LR_ERR_ARG;
  if (w->head_dim != 64 && w->head_dim != 128) return LR_ERR_UNSUPPORTED;
  if (w->n_heads % w->n_kv_heads) return LR_ERR_ARG;
  if (s.T <= 0 || s.S <= 0 || s.cap <= 0 || s.max_seq_rows <= 0 || s.pool_rows <= 0)
    return LR_ERR_ARG;
  if (s.cap > INT32_MAX || s.T > INT32_MAX) return LR_ERR_ARG;
  if (s.S > 255) return LR_ERR_UNSUPPORTED;  // the rotary epilogue stages S + 1 offsets
  if (!w->rope || w->rope_max_pos <= 0 || !w->attn_norm || !w->ffn_norm) return LR_ERR_ARG;
  if (!s.k_pool || !s.v_pool || !s.slot_mapping || !s.remap || !s.seq_off || !s.pos ||
      !s.n_valid)
    return LR_ERR_ARG;
  const int64_t dq = w->n_heads * w->head_dim, dkv = w->n_kv_heads * w->head_dim;
  const int64_t din[7] = {w->d_model, w->d_model, w->d_model, dq, w->d_model, w->d_model, w->d_ffn};
  if (w->mlp != LR_MLP_SWIGLU && w->mlp != LR_MLP_RELU) return LR_ERR_ARG;
  for (int k = 0; k < 7; ++k) {
    if (k == 5 && w->mlp == LR_MLP_RELU) continue;  // no up projection
    if (!w->Ut[k] || !w->Vt[k] || w->r[k] <= 0) return LR_ERR_ARG;
    if (w->ldu[k] < din[k] || w->ldv[k] < w->r[k]) return LR_ERR_ARG;
    if (!al16(w->Ut[k]) || !al16(w->Vt[k]) || w->ldu[k] % 8 || w->ldv[k] % 8) return LR_ERR_ALIGN;
    if (w->ldu[k] >= (1 << 22) || w->ldv[k] >= (1 << 22) || din[k] >= (1 << 22))
      return LR_ERR_UNSUPPORTED;
  }
  (void)dkv;
  if (s.pool_ld < w->r[1] || s.pool_ld < w->r[2]) return LR_ERR_ARG;
  // the reconstruction's rotary epilogue copies (cos, sin) rows in 16-byte
  // chunks, addressed with 32-bit offsets
  if (!al16(w->rope)) return LR_ERR_ALIGN;
  if (w->rope_max_pos * w->head_dim * 4 >= (int64_t(1) << 31)) return LR_ERR_UNSUPPORTED;
  // the reconstruction GEMM addresses a 256-row tile with 32-bit offsets
  if (!gemm_big_supported(rup(w->r[1], 8), w->ldv[1]) ||
      !gemm_big_supported(rup(w->r[2], 8), w->ldv[2]))
    return LR_ERR_UNSUPPORTED;
  if (!al16(s.k_pool) || !al16(s.v_pool) || s.pool_ld % 8) return LR_ERR_ALIGN;
  if (w->d_model % 8 || w->d_ffn % 8) return LR_ERR_ALIGN;
  return LR_OK;
}

lr_status layer_step(const lr_layer_weights* w, const StepIn& s, float* h, void* workspace,
                     size_t workspace_bytes, hipStream_t st, bool fused = false) {
  const StepLayout L = step_layout(w, s, fused);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const int T = (int)s.T;
  const bool dec = s.T <= kDecodeTokens;
  const int64_t d = w->d_model, dq = w->n_heads * w->head_dim, ffn = w->d_ffn;
  uint16_t* x = reinterpret_cast<uint16_t*>(ws + L.x);
  uint16_t* q = reinterpret_cast<uint16_t*>(ws + L.q);
  float* latk = reinterpret_cast<float*>(ws + L.latk);
  float* latv = reinterpret_cast<float*>(ws + L.latv);
  uint16_t* kbuf = reinterpret_cast<uint16_t*>(ws + L.kbuf);
  uint16_t* vbuf = reinterpret_cast<uint16_t*>(ws + L.vbuf);
  uint16_t* krec = reinterpret_cast<uint16_t*>(ws + L.krec);
  uint16_t* vrec = reinterpret_cast<uint16_t*>(ws + L.vrec);
  float* part = reinterpret_cast<float*>(ws + L.part);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + L.o);
  uint16_t* gate = reinterpret_cast<uint16_t*>(ws + L.gate);
  uint16_t* up = reinterpret_cast<uint16_t*>(ws + L.up);
  uint16_t* m = reinterpret_cast<uint16_t*>(ws + L.m);
  uint16_t* yb = reinterpret_cast<uint16_t*>(ws + L.yb);
  void* lin = ws + L.lin;
  hipError_t e = hipSuccess;
#define LR_CHECK(expr)                \
  do {                                \
    e = (expr);                       \
    if (e != hipSuccess) return LR_ERR_HIP; \
  } while (0)

  auto linear = [&](int k, const void* in, int64_t din, int64_t ldin, int64_t dout, void* y,
                    float* yacc, float* t_out) -> DecodeLinear {
    DecodeLinear dl{};
    dl.T = T;
    dl.d_in = din;
    dl.r = w->r[k];
    dl.d_out = dout;
    dl.x = in;
    dl.ldx = ldin;
    dl.Ut = w->Ut[k];
    dl.ldu = w->ldu[k];
    dl.Vt = w->Vt[k];
    dl.ldv = w->ldv[k];
    dl.y = y;
    dl.ldy = dout;
    dl.t_io = t_out;
    dl.ldt = w->r[k];
    dl.flags = t_out ? 1u : 0u;
    dl.workspace = lin;
    dl.y_acc = yacc;
    dl.ld_acc = d;
    return dl;
  };
  const unsigned eb = (unsigned)((T * d + 255) / 256 < 4096 ? (T * d + 255) / 256 : 4096);
  // y = in . U_r V_r added into the residual h: in the decode kernel's
  // epilogue, or (prefill path) through a bf16 y and an add
  auto residual_linear = [&](int k, const void* in, int64_t din) -> hipError_t {
    if (dec) return decode_linear_bf16(linear(k, in, din, din, d, nullptr, h, nullptr), st);
    const DecodeLinear acc = linear(k, in, din, din, d, nullptr, h, nullptr);
    if (prefill_accumulates(acc)) return prefill_linear_bf16(acc, st);  // in the GEMM epilogue
    hipError_t r = prefill_linear_bf16(linear(k, in, din, din, d, yb, nullptr, nullptr), st);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(add_residual_kernel, dim3(eb), dim3(256), 0, st, h, yb, (int64_t)T * d);
    return hipGetLastError();
  };

  // attention block
  LR_CHECK(launch_rmsnorm(h, d, static_cast<const uint16_t*>(w->attn_norm), x, d, T, d, w->eps, st));
  {
    // q (full) and the k, v latents (stage 1 only) read the same x
    const DecodeLinear qkv[3] = {linear(0, x, d, d, dq, q, nullptr, nullptr),
                                 linear(1, x, d, d, L.dkv, nullptr, nullptr, latk),
                                 linear(2, x, d, d, L.dkv, nullptr, nullptr, latv)};
    if (dec) {
      LR_CHECK(decode_group_bf16(qkv, 3, st));  // one launch
    } else if (prefill_group_ok(qkv, 3)) {
      LR_CHECK(prefill_group_bf16(qkv, 3, st));  // stage 1 as one launch
    } else {
      for (int k = 0; k < 3; ++k) LR_CHECK(prefill_linear_bf16(qkv[k], st));
    }
  }
  hipLaunchKernelGGL(append_kernel, dim3(T), dim3(256), 0, st, latk, w->r[1], (int)w->r[1],
                     s.slot_mapping, s.pool_rows, static_cast<uint16_t*>(s.k_pool), s.pool_ld);
  LR_CHECK(hipGetLastError());
  hipLaunchKernelGGL(append_kernel, dim3(T), dim3(256), 0, st, latv, w->r[2], (int)w->r[2],
                     s.slot_mapping, s.pool_rows, static_cast<uint16_t*>(s.v_pool), s.pool_ld);
  LR_CHECK(hipGetLastError());
  // The fused attention reads the latents in place through the remap list
  // (32-bit offsets into a pool under 2 GiB); otherwise they are first
  // gathered into the compact buffers.
  const bool in_place = fused && s.pool_rows * s.pool_ld * 2 < (int64_t(1) << 31);
  if (!in_place) {
    LR_CHECK(remap_gather(2, s.k_pool, s.pool_rows, s.pool_ld, s.remap, s.cap, s.n_valid,
                          w->r[1], kbuf, L.rk_ld, st));
    LR_CHECK(remap_gather(2, s.v_pool, s.pool_rows, s.pool_ld, s.remap, s.cap, s.n_valid,
                          w->r[2], vbuf, L.rv_ld, st));
  }
  const int S = (int)s.S;
  if (fused) {
    // attention straight from the gathered latents: K and V expanded per
    // 256-row block on chip, block partials, then their combine per head
    int32_t* blk_off = reinterpret_cast<int32_t*>(ws + L.tok_off);
    float* fpart = reinterpret_cast<float*>(ws + L.part);
    hipLaunchKernelGGL(row_blocks_kernel, dim3(1), dim3(64), 0, st, s.seq_off, S, (int)s.cap,
                       blk_off);
    LR_CHECK(hipGetLastError());
    FusedAttnArgs fa{};
    fa.kl = in_place ? static_cast<const uint16_t*>(s.k_pool) : kbuf;
    fa.ldkl = in_place ? s.pool_ld : L.rk_ld;
    fa.rk = (int)w->r[1];
    fa.vl = in_place ? static_cast<const uint16_t*>(s.v_pool) : vbuf;
    fa.ldvl = in_place ? s.pool_ld : L.rv_ld;
    fa.rv = (int)w->r[2];
    fa.remap = in_place ? s.remap : nullptr;
    fa.pool_rows = s.pool_rows;
    fa.vk = static_cast<const uint16_t*>(w->Vt[1]);
    fa.ldvk = w->ldv[1];
    fa.vv = static_cast<const uint16_t*>(w->Vt[2]);
    fa.ldvv = w->ldv[2];
    fa.q = q;
    fa.ldq = dq;
    fa.rope = w->rope;
    fa.max_pos = w->rope_max_pos;
    fa.seq_off = s.seq_off;
    fa.pos = s.pos;
    fa.blk_off = blk_off;
    fa.S = S;
    fa.cap = (int)s.cap;
    fa.H = (int)w->n_heads;
    fa.Hkv = (int)w->n_kv_heads;
    fa.nbpad = (int)L.nbpad;
    fa.part = fpart;
    LR_CHECK(attn_fused_decode(fa, (int)w->head_dim, st));
    const size_t vec_lds = (size_t)w->r[2] * 4;
    const uint16_t* vv = static_cast<const uint16_t*>(w->Vt[2]);
    // several sequences per workgroup where their latent sums fit 64 KB of LDS
    const int gs = (int)(4 * w->head_dim / 64);
    const size_t gvec = (size_t)gs * (size_t)rup(w->r[2], 4) * 4;
    const dim3 ggrid((unsigned)w->n_heads, (unsigned)((S + gs - 1) / gs));
    if (gvec <= 65536 && w->head_dim == 128)
      hipLaunchKernelGGL(fused_combine_group_kernel<128>, ggrid, dim3(512), gvec, st, fpart,
                         (int)w->n_heads, (int)w->n_kv_heads, (int)w->r[2], blk_off,
                         (int)L.nbpad, S, vv, w->ldv[2], o, dq);
    else if (gvec <= 65536)
      hipLaunchKernelGGL(fused_combine_group_kernel<64>, ggrid, dim3(256), gvec, st, fpart,
                         (int)w->n_heads, (int)w->n_kv_heads, (int)w->r[2], blk_off,
                         (int)L.nbpad, S, vv, w->ldv[2], o, dq);
    else if (w->head_dim == 128)
      hipLaunchKernelGGL(fused_combine_kernel<128>, dim3((unsigned)w->n_heads, (unsigned)S),
                         dim3(512), vec_lds, st, fpart, (int)w->n_heads, (int)w->n_kv_heads,
                         (int)w->r[2], blk_off, (int)L.nbpad, vv, w->ldv[2], o, dq);
    else
      hipLaunchKernelGGL(fused_combine_kernel<64>, dim3((unsigned)w->n_heads, (unsigned)S),
                         dim3(256), vec_lds, st, fpart, (int)w->n_heads, (int)w->n_kv_heads,
                         (int)w->r[2], blk_off, (int)L.nbpad, vv, w->ldv[2], o, dq);
  } else {
    // rec[j, :] = buf[j, 0:r] . Vt^T for the live rows j < *n_valid: the
    // fixed-size GEMM of the replay stage (grid from the capacity), K rows
    // rotated by their positions in the epilogue.
    {
      const BigRope rope{w->rope, w->rope_max_pos, s.seq_off, (int)s.S, (int)w->head_dim};
      LR_CHECK(gemm_nt_big_rows(kbuf, L.rk_ld, w->Vt[1], w->ldv[1], krec, L.dkv, s.cap, s.n_valid,
                                L.dkv, w->r[1], &rope, st));
      LR_CHECK(gemm_nt_big_rows(vbuf, L.rv_ld, w->Vt[2], w->ldv[2], vrec, L.dkv, s.cap, s.n_valid,
                                L.dkv, w->r[2], nullptr, st));
    }
    const dim3 agrid((unsigned)L.nch, (unsigned)w->n_heads, (unsigned)T);
    if (s.tok_seq) {
      // chunked prefill: tiled causal attention over each sequence's rows
      int32_t* tok_off = reinterpret_cast<int32_t*>(ws + L.tok_off);
      int32_t* blk_off = tok_off + (S + 1);
      hipLaunchKernelGGL(tok_offsets_kernel, dim3(1), dim3(256), 0, st, s.tok_seq, T, S, tok_off,
                         blk_off);
      LR_CHECK(hipGetLastError());
      // at most T/kPrefQB + S query blocks over all sequences
      const int nbpad = (int)((T + kPrefQB - 1) / kPrefQB) + S;
      const int64_t nitems = (int64_t)w->n_heads * nbpad;
      const dim3 pgrid((unsigned)((nitems + 7) / 8 * 8));
      if (w->head_dim == 128)
        hipLaunchKernelGGL(attn_prefill_kernel<128>, pgrid, dim3(256), 0, st, q, dq, krec, vrec,
                           L.dkv, s.seq_off, tok_off, blk_off, S, nbpad, s.pos, w->rope,
                           w->rope_max_pos, (int)w->n_heads, (int)w->n_kv_heads, (int)s.cap, o, dq);
      else
        hipLaunchKernelGGL(attn_prefill_kernel<64>, pgrid, dim3(256), 0, st, q, dq, krec, vrec,
                           L.dkv, s.seq_off, tok_off, blk_off, S, nbpad, s.pos, w->rope,
                           w->rope_max_pos, (int)w->n_heads, (int)w->n_kv_heads, (int)s.cap, o, dq);
    } else if (w->head_dim == 128) {
      hipLaunchKernelGGL(attn_partial_kernel<128>, agrid, dim3(256), 0, st, q, dq, krec, vrec,
                         L.dkv, s.seq_off, s.tok_seq, S, s.pos, w->rope, w->rope_max_pos,
                         (int)w->n_heads, (int)w->n_kv_heads, (int)L.nch, (int)s.cap, part);
      LR_CHECK(hipGetLastError());
      hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)w->n_heads, (unsigned)T),
                         dim3(128), 0, st, part, (int)w->n_heads, (int)L.nch, s.seq_off, s.tok_seq,
                         S, s.pos, (int)s.cap, o, dq);
    } else {
      hipLaunchKernelGGL(attn_partial_kernel<64>, agrid, dim3(256), 0, st, q, dq, krec, vrec,
                         L.dkv, s.seq_off, s.tok_seq, S, s.pos, w->rope, w->rope_max_pos,
                         (int)w->n_heads, (int)w->n_kv_heads, (int)L.nch, (int)s.cap, part);
      LR_CHECK(hipGetLastError());
      hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)w->n_heads, (unsigned)T),
                         dim3(64), 0, st, part, (int)w->n_heads, (int)L.nch, s.seq_off, s.tok_seq,
                         S, s.pos, (int)s.cap, o, dq);
    }
  }
  LR_CHECK(hipGetLastError());
  LR_CHECK(residual_linear(3, o, dq));
  // MLP block
  LR_CHECK(launch_rmsnorm(h, d, static_cast<const uint16_t*>(w->ffn_norm), x, d, T, d, w->eps, st));
  const dim3 egrid((unsigned)((T * ffn + 255) / 256 < 4096 ? (T * ffn + 255) / 256 : 4096));
  // on the large-tile prefill path the activation runs in the epilogue of
  // the last MLP GEMM (relu of fc1; silu(gate) * up in the up projection)
  if (w->mlp == LR_MLP_RELU) {
    DecodeLinear fc1 = linear(4, x, d, d, ffn, m, nullptr, nullptr);
    fc1.act = 2;
    if (!dec && prefill_act_ok(fc1)) {
      LR_CHECK(prefill_linear_bf16(fc1, st));
    } else {
      fc1 = linear(4, x, d, d, ffn, gate, nullptr, nullptr);
      LR_CHECK(dec ? decode_linear_bf16(fc1, st) : prefill_linear_bf16(fc1, st));
      hipLaunchKernelGGL(relu_kernel, egrid, dim3(256), 0, st, gate, m, (int64_t)T * ffn);
    }
  } else {
    const DecodeLinear gu[2] = {linear(4, x, d, d, ffn, gate, nullptr, nullptr),
                                linear(5, x, d, d, ffn, up, nullptr, nullptr)};
    DecodeLinear upm = linear(5, x, d, d, ffn, m, nullptr, nullptr);
    upm.act = 1;
    upm.glu = gate;
    upm.ldglu = ffn;
    if (dec) {
      LR_CHECK(decode_group_bf16(gu, 2, st));
      hipLaunchKernelGGL(silu_mul_kernel, egrid, dim3(256), 0, st, gate, up, m, (int64_t)T * ffn);
    } else if (prefill_act_ok(upm)) {
      const DecodeLinear gup[2] = {gu[0], upm};
      if (prefill_group_ok(gup, 2)) {
        LR_CHECK(prefill_group_bf16(gup, 2, st));  // stage 1 as one launch; gate's y, then up's
      } else {
        LR_CHECK(prefill_linear_bf16(gu[0], st));
        LR_CHECK(prefill_linear_bf16(upm, st));
      }
    } else {
      LR_CHECK(prefill_linear_bf16(gu[0], st));
      LR_CHECK(prefill_linear_bf16(gu[1], st));
      hipLaunchKernelGGL(silu_mul_kernel, egrid, dim3(256), 0, st, gate, up, m, (int64_t)T * ffn);
    }
  }
  LR_CHECK(hipGetLastError());
  LR_CHECK(residual_linear(6, m, ffn));
#undef LR_CHECK
  return LR_OK;
}

}  // namespace

}  // namespace lr

using namespace lr;

extern "C" lr_status lowrank_rope_table(int64_t head_dim, int64_t max_pos, float theta,
                                        float* table, hipStream_t stream) {
  if (head_dim <= 0 || head_dim % 2 || max_pos <= 0 || !table || !(theta > 0.f)) return LR_ERR_ARG;
  const int64_t n = max_pos * (head_dim / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, stream, table, max_pos,
                     (int)(head_dim / 2), (double)theta);
  return hipGetLastError() == hipSuccess ? LR_OK : LR_ERR_HIP;
}

extern "C" size_t lowrank_decode_step_workspace_bytes(const lr_layer_weights* w,
                                                      const lr_decode_state* s) {
  if (!w || !s || s->B <= 0 || s->cap <= 0 || s->max_seq_rows <= 0) return 0;
  return step_layout(w, from_decode(s)).total;
}

extern "C" lr_status lowrank_layer_decode_step(const lr_layer_weights* w,
                                               const lr_decode_state* s, float* h,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t st) {
  if (!s) return LR_ERR_ARG;
  if (s->B > 64) return LR_ERR_UNSUPPORTED;  // projections run on the decode path
  const StepIn in = from_decode(s);
  const lr_status chk = check_step(w, in, h);
  if (chk != LR_OK) return chk;
  return layer_step(w, in, h, workspace, workspace_bytes, st);
}

extern "C" size_t lowrank_decode_step_fused_workspace_bytes(const lr_layer_weights* w,
                                                            const lr_decode_state* s) {
  if (!w || !s || s->B <= 0 || s->cap <= 0 || s->max_seq_rows <= 0) return 0;
  return step_layout(w, from_decode(s), true).total;
}

extern "C" lr_status lowrank_layer_decode_step_fused(const lr_layer_weights* w,
                                                     const lr_decode_state* s, float* h,
                                                     void* workspace, size_t workspace_bytes,
                                                     hipStream_t st) {
  if (!s) return LR_ERR_ARG;
  if (s->B > 64) return LR_ERR_UNSUPPORTED;  // projections run on the decode path
  const StepIn in = from_decode(s);
  const lr_status chk = check_step(w, in, h);
  if (chk != LR_OK) return chk;
  // the fused kernel stages at most 16 query heads per 256 K/V columns
  if ((256 / w->head_dim) * (w->n_heads / w->n_kv_heads) > 16) return LR_ERR_UNSUPPORTED;
  return layer_step(w, in, h, workspace, workspace_bytes, st, true);
}

extern "C" size_t lowrank_prefill_step_workspace_bytes(const lr_layer_weights* w,
                                                       const lr_prefill_state* s) {
  if (!w || !s || s->T <= 0 || s->S <= 0 || s->cap <= 0 || s->max_seq_rows <= 0) return 0;
  return step_layout(w, from_prefill(s)).total;
}

extern "C" lr_status lowrank_layer_prefill_step(const lr_layer_weights* w,
                                                const lr_prefill_state* s, float* h,
                                                void* workspace, size_t workspace_bytes,
                                                hipStream_t st) {
  if (!s) return LR_ERR_ARG;
  if (!s->tok_seq) return LR_ERR_ARG;
  const StepIn in = from_prefill(s);
  const lr_status chk = check_step(w, in, h);
  if (chk != LR_OK) return chk;
  return layer_step(w, in, h, workspace, workspace_bytes, st);
}
