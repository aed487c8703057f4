// Folded projections for MLA decode on MI355X (gfx950): the up-projections
// multiplied into their neighbouring weights ahead of time, and the two
// decode-time products that use the folded weights.
//
// Source (page title, section): "MLA from scratch", Absorbing projections
// (inference optimisation): W_O absorbs W_UV (a product of fixed weights
// computed once; at inference the attention-weighted latents go straight to
// the output space), and the same holds on the query side; "Multi-head latent
// attention" (octlm), What we didn't build, and why: at decode time the
// up-projection is folded into the query and output matrices.
//
// Kernels:
//   fold_gemm_kernel     one head's block of a folded weight, C = A B with K =
//                        d_head or d_v (32x32x16 bf16 MFMA, fp32 accumulation,
//                        one rounding to bf16); operands at arbitrary strides
//                        staged through LDS with k contiguous
//   wstream_kernel       decode-time product Y[b][n] = sum_k X[b][k] W[n][k]
//                        over a folded weight W with k-contiguous rows: the
//                        weight streamed from HBM straight into MFMA A
//                        fragments, the batch rows as B fragments, the four
//                        waves of a work-group on four quarters of its k range
//                        summed through LDS; fp32 X enters the bf16 MFMA as a
//                        high and a low bf16 part
//   wstream_reduce_kernel  the k groups of a split-k product summed in a fixed
//                        order (deterministic, no atomics)
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, wave64):
//   A[m][k]: lane i holds row m = i%32 and 8 consecutive k from 8*(i/32)
//   B[k][n]: lane i holds column n = i%32 and the same k slots
//   C[m][n]: lane i, accumulator r holds row 8*(r/4) + 4*(i/32) + r%4, column i%32
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla.h"
#include "mla_common.h"

namespace {

// ---------------------------------------------------------------------------
// Folding GEMM.  For head h (blockIdx.z):
//   C[m][n] = sum_k A(m, k) B(k, n),   A(m, k) = a[a_h*h + m*am + k*ak],
//                                      B(k, n) = b[b_h*h + k*bk + n*bn],
//   c[c_h*h + m*cm + n*cn] = bf16(C[m][n])
// Tile 64 x 64 per work-group, four waves in a 2 x 2 arrangement of 32 x 32
// blocks, k in chunks of 32 (two MFMA k-steps).  Each chunk's A and B tiles
// are read element by element (either operand may be transposed in memory; a
// one-time weight transform, so plain loads suffice) and stored in LDS with k
// contiguous, rows padded to 40 elements so that the 16-byte fragment reads
// of 32 rows spread over the banks.
// ---------------------------------------------------------------------------

constexpr int kFoldTile = 64;
constexpr int kFoldK = 32;
constexpr int kFoldLd = kFoldK + 8;  // LDS row length (elements)

struct FoldArgs {
  const u16* a;
  const u16* b;
  u16* c;
  int64_t a_h, am, ak;
  int64_t b_h, bk, bn;
  int64_t c_h, cm, cn;
  int M, N, K;
};

__global__ __launch_bounds__(256) void fold_gemm_kernel(FoldArgs p) {
  __shared__ __attribute__((aligned(16))) u16 As[kFoldTile * kFoldLd];
  __shared__ __attribute__((aligned(16))) u16 Bs[kFoldTile * kFoldLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kFoldTile, n0 = blockIdx.y * kFoldTile;
  const int64_t h = blockIdx.z;
  const u16* a = p.a + h * p.a_h;
  const u16* b = p.b + h * p.b_h;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;  // this wave's 32 x 32 block in the tile
  f32x16 acc = zero16();
  for (int k0 = 0; k0 < p.K; k0 += kFoldK) {
    // 64 x 32 elements per operand, 8 per thread; the index order follows the
    // operand's contiguous dimension so that neighbouring threads read
    // neighbouring elements
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = e * 256 + tid;
      int m, k;
      if (p.ak == 1) { m = idx >> 5; k = idx & 31; } else { m = idx & 63; k = idx >> 6; }
      As[m * kFoldLd + k] = a[(int64_t)(m0 + m) * p.am + (int64_t)(k0 + k) * p.ak];
      int n, kb;
      if (p.bk == 1) { n = idx >> 5; kb = idx & 31; } else { n = idx & 63; kb = idx >> 6; }
      Bs[n * kFoldLd + kb] = b[(int64_t)(k0 + kb) * p.bk + (int64_t)(n0 + n) * p.bn];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kFoldK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      const i16x8 af = *(const i16x8*)(As + (wm + (lane & 31)) * kFoldLd + kk);
      const i16x8 bf = *(const i16x8*)(Bs + (wn + (lane & 31)) * kFoldLd + kk);
      acc = Mma<u16>::mma(af, bf, acc);
    }
    __syncthreads();
  }
  u16* c = p.c + h * p.c_h;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int n = n0 + wn + (lane & 31);
    c[(int64_t)m * p.cm + (int64_t)n * p.cn] = f2bf(acc[r]);
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming product over a folded weight.  For group g = blockIdx.z
// (a head, or 0), row block blockIdx.x (64 rows of W) and k group blockIdx.y:
//   Y[b][n] = sum_{k in the k group} X[b][k] W[n][k]
//   X(b, k) = x[x_g*g + b*x_ld + k]   (bf16 or fp32),  b < nb (<= 64)
//   W(n, k) = w[w_g*g + n*w_ld + k]   (bf16, k contiguous)
// The k group is kspan long; wave w takes its quarter.  The product is formed
// transposed, C^T[n][b] = sum_k W[n][k] X[b][k]: A fragments are 16 bytes of
// one W row per lane straight from global memory, B fragments the same k
// slots of a batch row.  After the k loop the waves add their blocks through
// LDS in a fixed order, and the sum goes to
//   y[y_g*g + b*y_ld + n]   (bf16, one rounding; to_part == 0), or
//   part[(k group * nb + b) * n_total + n]   (fp32 partial; to_part == 1).
// ---------------------------------------------------------------------------

constexpr int kWsRows = 64;   // W rows per work-group (two 32-row MFMA blocks)
constexpr int kWsUnroll = 4;  // k-steps per loop iteration (64 k)

struct WsArgs {
  const void* x;
  const u16* w;
  void* y;        // bf16 output (to_part == 0)
  float* part;    // fp32 partials per k group (to_part == 1)
  int64_t x_g, x_ld, w_g, w_ld, y_g, y_ld;
  int nb, n_total, kspan, kgroups, to_part;
};

template <typename XT>
__device__ __forceinline__ void load_x(const XT* xrow, bool ok, i16x8& hi, i16x8& lo);

template <>
__device__ __forceinline__ void load_x<u16>(const u16* xrow, bool ok, i16x8& hi, i16x8& lo) {
  hi = ok ? *(const i16x8*)xrow : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
  lo = hi;  // (unused)
}

template <>
__device__ __forceinline__ void load_x<float>(const float* xrow, bool ok, i16x8& hi, i16x8& lo) {
  f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
  if (ok) {
    v0 = *(const f32x4*)xrow;
    v1 = *(const f32x4*)(xrow + 4);
  }
  const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float hv = round_bf16_finite(v[e]);
    hi[e] = (short)(__float_as_uint(hv) >> 16);
    lo[e] = (short)f2bf(v[e] - hv);
  }
}

template <typename XT, int NB>
__global__ __launch_bounds__(256) void wstream_kernel(WsArgs p) {
  constexpr bool SPLIT = sizeof(XT) == 4;  // fp32 X: high and low bf16 parts
  __shared__ float red[4][kWsRows][32 * NB + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.z;
  const int n0 = blockIdx.x * kWsRows;
  const int kq = p.kspan / 4;  // this wave's share of the k group
  const int kbeg = blockIdx.y * p.kspan + wave * kq;
  const XT* x = (const XT*)p.x + g * p.x_g;
  const u16* w = p.w + g * p.w_g;
  const int slot = 8 * (lane >> 5);
  const u16* wr0 = w + (int64_t)(n0 + (lane & 31)) * p.w_ld + kbeg + slot;
  const u16* wr1 = wr0 + 32 * p.w_ld;
  const XT* xr[NB];
  bool xok[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int bb = 32 * j + (lane & 31);
    xok[j] = bb < p.nb;
    xr[j] = x + (int64_t)(xok[j] ? bb : 0) * p.x_ld + kbeg + slot;
  }
  f32x16 acc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = zero16();
  for (int k = 0; k < kq; k += 16 * kWsUnroll) {
    i16x8 wa[kWsUnroll][2], xh[kWsUnroll][NB], xl[kWsUnroll][NB];
#pragma unroll
    for (int u = 0; u < kWsUnroll; ++u) {
      wa[u][0] = *(const i16x8*)(wr0 + k + 16 * u);
      wa[u][1] = *(const i16x8*)(wr1 + k + 16 * u);
#pragma unroll
      for (int j = 0; j < NB; ++j) load_x<XT>(xr[j] + k + 16 * u, xok[j], xh[u][j], xl[u][j]);
    }
#pragma unroll
    for (int u = 0; u < kWsUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[i][j] = Mma<u16>::mma(wa[u][i], xh[u][j], acc[i][j]);
          if constexpr (SPLIT) acc[i][j] = Mma<u16>::mma(wa[u][i], xl[u][j], acc[i][j]);
        }
  }
  // C^T[n][b]: lane holds batch column 32*j + lane%32 and rows 8*(r/4) +
  // 4*(lane/32) + r%4 of row block i
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red[wave][32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][32 * j + (lane & 31)] = acc[i][j][r];
  __syncthreads();
  for (int e = tid; e < kWsRows * 32 * NB; e += 256) {
    const int bcol = e / kWsRows, n = e % kWsRows;  // consecutive threads on consecutive rows n
    if (bcol >= p.nb) continue;
    const float s = ((red[0][n][bcol] + red[1][n][bcol]) + red[2][n][bcol]) + red[3][n][bcol];
    if (!p.to_part) {
      ((u16*)p.y)[g * p.y_g + (int64_t)bcol * p.y_ld + n0 + n] = f2bf(s);
    } else {
      p.part[((int64_t)blockIdx.y * p.nb + bcol) * p.n_total + n0 + n] = s;
    }
  }
}

// y[b][n] = sum over k groups (in order) of part[g][b][n]
__global__ __launch_bounds__(256) void wstream_reduce_kernel(const float* __restrict__ part, int kgroups, int nb,
                                                             int n_total, float* __restrict__ y, int64_t y_ld) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)nb * n_total) return;
  const int b = (int)(e / n_total), n = (int)(e % n_total);
  float s = 0.f;
  for (int gi = 0; gi < kgroups; ++gi) s += part[((int64_t)gi * nb + b) * n_total + n];
  y[(int64_t)b * y_ld + n] = s;
}

template <typename XT>
hipError_t launch_wstream(const WsArgs& a, int row_blocks, int groups, hipStream_t stream) {
  const dim3 grid((unsigned)row_blocks, (unsigned)a.kgroups, (unsigned)groups);
  if (a.nb > 32) {
    hipLaunchKernelGGL((wstream_kernel<XT, 2>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((wstream_kernel<XT, 1>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

namespace mla_detail {

// w_qk[h][j][i] = sum_d w_uk[h][d][j] w_uq[h*dh + d][i]
hipError_t launch_fold_query(int H, int dh, int r, int dcq, const void* w_uq, const void* w_uk, void* w_qk,
                             hipStream_t stream) {
  FoldArgs p{(const u16*)w_uk, (const u16*)w_uq, (u16*)w_qk,
             (int64_t)dh * r, 1, r,                 // A(j, d) = w_uk[h][d][j]
             (int64_t)dh * dcq, dcq, 1,             // B(d, i) = w_uq[h*dh + d][i]
             (int64_t)r * dcq, dcq, 1,              // C -> w_qk[h][j][i]
             r, dcq, dh};
  hipLaunchKernelGGL(fold_gemm_kernel, dim3(r / kFoldTile, dcq / kFoldTile, H), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// w_ov[m][h*r + j] = sum_d w_o[m][h*dv + d] w_uv[h][d][j]
hipError_t launch_fold_output(int H, int dv, int r, int d_model, const void* w_o, const void* w_uv, void* w_ov,
                              hipStream_t stream) {
  FoldArgs p{(const u16*)w_o, (const u16*)w_uv, (u16*)w_ov,
             dv, (int64_t)H * dv, 1,                // A(m, d) = w_o[m][h*dv + d]
             (int64_t)dv * r, r, 1,                 // B(d, j) = w_uv[h][d][j]
             r, (int64_t)H * r, 1,                  // C -> w_ov[m][h*r + j]
             d_model, r, dv};
  hipLaunchKernelGGL(fold_gemm_kernel, dim3(d_model / kFoldTile, r / kFoldTile, H), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// q_lat[b][h][j] = bf16(sum_i w_qk[h][j][i] c_q[b][i]), j < r, for every
// batch slice of up to 64 sequences
hipError_t launch_absorb_q_folded(int B, int H, int r, int W, int dcq, const void* c_q, const void* w_qk,
                                  void* q_lat, hipStream_t stream) {
  for (int b0 = 0; b0 < B; b0 += 64) {
    WsArgs a{};
    a.x = (const u16*)c_q + (int64_t)b0 * dcq;
    a.w = (const u16*)w_qk;
    a.y = (u16*)q_lat + (int64_t)b0 * H * W;
    a.x_g = 0, a.x_ld = dcq, a.w_g = (int64_t)r * dcq, a.w_ld = dcq, a.y_g = W, a.y_ld = (int64_t)H * W;
    a.nb = B - b0 < 64 ? B - b0 : 64;
    a.n_total = r, a.kspan = dcq, a.kgroups = 1, a.to_part = 0;
    hipError_t e = launch_wstream<u16>(a, r / kWsRows, H, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Split-k plan of the folded output product: k groups of kspan (a multiple
// of 4 * 64 dividing K; K is a multiple of 256), about 2048 k per wave.
int out_folded_kgroups(int64_t K) {
  int g = 1;
  while (K % (2 * g * 256) == 0 && K / (2 * g) >= 4 * 2048) g *= 2;
  return g;
}

// fp32 partials of one batch slice (up to 64 sequences), reused slice by slice
size_t out_folded_workspace_bytes(int B, int d_model, int64_t K) {
  const int nb = B < 64 ? B : 64;
  return (size_t)out_folded_kgroups(K) * nb * d_model * sizeof(float);
}

// y[b][m] = sum_k w_ov[m][k] o_lat[b][k], k < K = H*r, fp32 out
hipError_t launch_out_folded(int B, int d_model, int64_t K, const float* o_lat, const void* w_ov, float* y,
                             float* workspace, hipStream_t stream) {
  const int kg = out_folded_kgroups(K);
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int nb = B - b0 < 64 ? B - b0 : 64;
    WsArgs a{};
    a.x = o_lat + (int64_t)b0 * K;
    a.w = (const u16*)w_ov;
    a.y = nullptr;
    a.part = workspace;
    a.x_g = 0, a.x_ld = K, a.w_g = 0, a.w_ld = K, a.y_g = 0, a.y_ld = d_model;
    a.nb = nb, a.n_total = d_model, a.kspan = (int)(K / kg), a.kgroups = kg, a.to_part = 1;
    hipError_t e = launch_wstream<float>(a, d_model / kWsRows, 1, stream);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)nb * d_model;
    hipLaunchKernelGGL(wstream_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, workspace,
                       kg, nb, d_model, y + (int64_t)b0 * d_model, (int64_t)d_model);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla_detail
