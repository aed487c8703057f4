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
//                        over a folded weight W with k-contiguous rows: tiles
//                        of W and of the batch rows X streamed into a 3- or
//                        4-stage LDS ring by DMA, W fragments as MFMA A operands and
//                        X fragments as B operands, the four waves of a
//                        work-group on four quarters of each tile's k range
//                        summed through LDS at the end; fp32 X enters the
//                        bf16 MFMA as a high and a low bf16 part
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
// (a head, or 0), row block blockIdx.x (32*RB rows of W) and k group
// blockIdx.y:
//   Y[b][n] = sum_{k in the k group} X[b][k] W[n][k]
//   X(b, k) = x[x_g*g + b*x_ld + k]   (bf16 or fp32),  b < nb (<= 64)
//   W(n, k) = w[w_g*g + n*w_ld + k]   (bf16, k contiguous)
// The k group is kspan long, in tiles of KT.  Both operands of a tile stream
// into an LDS ring of ST stages by DMA (global_load_lds, 16 bytes per lane,
// issued in inline asm so that every wait on them is an explicit vmcnt): the
// W tile (32*RB rows x KT) and the X tile (XR rows: 16, 32 or 64, enough for
// nb; rows past nb repeat row nb - 1, and their columns are dropped).  The
// 32 MFMA columns of a batch block read X row (32*j + lane%32) % XR, so with
// XR = 16 the upper 16 columns repeat the lower ones.  Within a row, 16-byte
// chunk c sits at slot c ^ swz(row): the 16 lanes of a fragment read (16
// consecutive rows at one chunk) then hit 16 different 16-byte bank groups
// (swz = row & 15 for rows of 16 or more chunks; (row >> 1) & 7 for 8-chunk
// rows, two to a 256-byte bank line).  Wave w takes the k-steps
// w*KT/64 .. of each tile: C^T[n][b] += W[n][k] X[b][k] with W fragments as A
// and X fragments as B (fp32 X enters the bf16 MFMA as a high and a low bf16
// part).  After the k loop the waves add their blocks through LDS in a fixed
// order, and the sum goes to
//   y[y_g*g + b*y_ld + n]   (bf16, one rounding; to_part == 0), or
//   part[(k group * nb + b) * n_total + n]   (fp32 partial; to_part == 1).
// ---------------------------------------------------------------------------

struct WsArgs {
  const void* x;
  const u16* w;
  void* y;        // bf16 output (to_part == 0)
  float* part;    // fp32 partials per k group (to_part == 1)
  int64_t x_g, x_ld, w_g, w_ld, y_g, y_ld;
  int nb, n_total, kspan, kgroups, to_part;
};

template <typename XT, int NB, int RB, int KT, int XR, int ST>
struct DsShape {
  static constexpr int WROWS = 32 * RB;
  static constexpr int XROWS = 32 * NB;                 // MFMA batch columns
  static constexpr int WCH = KT / 8;                    // 16-byte chunks of a W row in a tile
  static constexpr int XROWB = KT * (int)sizeof(XT);    // bytes of an X row in a tile
  static constexpr int XCH = XROWB / 16;
  static constexpr int WBYTES = WROWS * KT * 2;
  static constexpr int XBYTES = XR * XROWB;
  static constexpr int STAGE = WBYTES + XBYTES;
  static constexpr int WDMA = WBYTES / (256 * 16);      // DMA instructions per thread and tile
  static constexpr int XDMA = XBYTES / (256 * 16);
  static constexpr int PER_TILE = WDMA + XDMA;
  static constexpr int KSTEPS = KT / 64;                // k-steps of 16 per wave and tile
  static constexpr int RED = 4 * WROWS * 33 * 4;  // one batch block of the waves' partial sums
  static constexpr int LDS = ST * STAGE > RED ? ST * STAGE : RED;
  static_assert(KT % 64 == 0 && XR <= XROWS && XR >= 16, "shape");
  static_assert(WBYTES % (256 * 16) == 0 && XBYTES % (256 * 16) == 0, "whole DMA instructions");
  static_assert(WCH >= 8 && XCH >= 8, "rows of at least 8 chunks");
  static_assert(PER_TILE * (ST - 2) <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// slot of 16-byte chunk c of a row of ch chunks
template <int CH>
__device__ __forceinline__ int ds_slot(int c, int row) {
  return CH >= 16 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}

// One 16-byte-per-lane LDS DMA: lane l copies 16 bytes at src to LDS byte
// lds + 16*l (lds wave-uniform).  m0 carries the LDS address and is restored.
__device__ __forceinline__ void dma16(const void* src, int lds) {
  uint32_t save;
  asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[a], off\n\t"
               "s_mov_b32 m0, %[sv]"
               : [sv] "=&s"(save)
               : [a] "v"(src), [l] "s"(lds)
               : "memory");
}

// tile t has landed once at most `younger` later tiles of PER DMA
// instructions each are in flight; then every wave meets at the barrier
template <int PER>
__device__ __forceinline__ void ds_wait(int younger) {
  if (younger >= 2) wait_vm_then_barrier<2 * PER>();
  else if (younger == 1) wait_vm_then_barrier<PER>();
  else wait_vm_then_barrier<0>();
}

// X fragment of row r (its LDS bytes at row): bf16 X is chunk c (8 values);
// fp32 X is chunks c and c + 1 (8 values), split into high and low bf16 parts
template <typename XT, int XCH>
__device__ __forceinline__ void read_x(const LDS_AS char* row, int r, int c, i16x8& hi, i16x8& lo) {
  if constexpr (sizeof(XT) == 2) {
    hi = *(const LDS_AS i16x8*)(row + 16 * ds_slot<XCH>(c, r));
    lo = hi;  // (unused)
  } else {
    const f32x4 v0 = *(const LDS_AS f32x4*)(row + 16 * ds_slot<XCH>(c, r));
    const f32x4 v1 = *(const LDS_AS f32x4*)(row + 16 * ds_slot<XCH>(c + 1, r));
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float hv = round_bf16_finite(v[e]);
      hi[e] = (short)(__float_as_uint(hv) >> 16);
      lo[e] = (short)f2bf(v[e] - hv);
    }
  }
}

template <typename XT, int NB, int RB, int KT, int XR, int ST>
__global__ __launch_bounds__(256) void wstream_kernel(WsArgs p) {
  using S = DsShape<XT, NB, RB, KT, XR, ST>;
  constexpr bool SPLIT = sizeof(XT) == 4;  // fp32 X: high and low bf16 parts
  __shared__ __attribute__((aligned(1024))) char ring[S::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.z;
  const int n0 = blockIdx.x * S::WROWS;
  const int64_t kbeg = (int64_t)blockIdx.y * p.kspan;
  const int ntiles = p.kspan / KT;
  const int lds0 = (int)(uintptr_t)(LDS_AS char*)ring;

  // DMA sources.  Instruction i of thread t fills physical chunk q = 256*i + t
  // of the W (then X) part of a stage: row q / chunks-per-row, slot q % chunks-
  // per-row, which holds the row's chunk whose slot is that (the swizzle is an
  // involution).
  const char* wsrc[S::WDMA];
  const char* xsrc[S::XDMA];
  {
    const char* wb = (const char*)(p.w + g * p.w_g + (int64_t)n0 * p.w_ld + kbeg);
#pragma unroll
    for (int i = 0; i < S::WDMA; ++i) {
      const int q = 256 * i + tid, r = q / S::WCH, sl = q % S::WCH;
      wsrc[i] = wb + (int64_t)r * p.w_ld * 2 + 16 * ds_slot<S::WCH>(sl, r);
    }
    const char* xb = (const char*)((const XT*)p.x + g * p.x_g + kbeg);
#pragma unroll
    for (int i = 0; i < S::XDMA; ++i) {
      const int q = 256 * i + tid, r = q / S::XCH, sl = q % S::XCH;
      const int rr = r < p.nb ? r : p.nb - 1;
      xsrc[i] = xb + (int64_t)rr * p.x_ld * (int64_t)sizeof(XT) + 16 * ds_slot<S::XCH>(sl, r);
    }
  }
  auto issue = [&](int tile, int stage) {
    const int base = lds0 + stage * S::STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < S::WDMA; ++i) dma16(wsrc[i] + (int64_t)tile * (KT * 2), base + 4096 * i);
#pragma unroll
    for (int i = 0; i < S::XDMA; ++i)
      dma16(xsrc[i] + (int64_t)tile * S::XROWB, base + S::WBYTES + 4096 * i);
  };

  f32x16 acc[RB][NB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = zero16();

  // fragment addressing: A (W) row 32*i + lane%32, B (X) row (32*j +
  // lane%32) % XR; k-step u of this wave: k = 16*(KSTEPS*wave + u) +
  // 8*(lane/32) .. +7
  const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (t < ntiles) issue(t, t);
  for (int t = 0; t < ntiles; ++t) {
    // tile t has landed in every wave (later ones may be in flight), and every
    // wave is done with tile t - 1, whose stage the copy of t + ST - 1 takes
    const int younger = min(ST - 2, ntiles - 1 - t);
    ds_wait<S::PER_TILE>(younger);
    if (t + ST - 1 < ntiles) issue(t + ST - 1, (t + ST - 1) % ST);
    const LDS_AS char* st = (const LDS_AS char*)ring + (t % ST) * S::STAGE;
#pragma unroll
    for (int u = 0; u < S::KSTEPS; ++u) {
      const int cw = 2 * (S::KSTEPS * wave + u) + hf;  // W chunk (8 bf16) of this lane
      i16x8 wa[RB], xh[NB], xl[NB];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        wa[i] = *(const LDS_AS i16x8*)(st + (32 * i + l32) * (KT * 2) + 16 * ds_slot<S::WCH>(cw, l32));
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int xr = (32 * j + l32) % XR;
        read_x<XT, S::XCH>(st + S::WBYTES + xr * S::XROWB, xr, SPLIT ? 2 * cw : cw, xh[j], xl[j]);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[i][j] = Mma<u16>::mma(wa[i], xh[j], acc[i][j]);
          if constexpr (SPLIT) acc[i][j] = Mma<u16>::mma(wa[i], xl[j], acc[i][j]);
        }
    }
  }
  // The waves' partial sums go through LDS one 32-column batch block at a
  // time (C^T[n][b]: lane holds batch column 32*j + lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 of row block i), added in a fixed order.
  float* red = (float*)ring;  // [wave][row][column], rows padded to 33
  constexpr int RS = 33;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    __syncthreads();  // every wave is done with the ring (or with the previous block's sums)
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red[(wave * S::WROWS + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3)) * RS + l32] = acc[i][j][r];
    __syncthreads();
    for (int e = tid; e < S::WROWS * 32; e += 256) {
      const int bc = e / S::WROWS, n = e % S::WROWS;  // consecutive threads on consecutive rows n
      const int bcol = 32 * j + bc;
      if (bcol >= p.nb) continue;
      const float s = ((red[(0 * S::WROWS + n) * RS + bc] + red[(1 * S::WROWS + n) * RS + bc]) +
                       red[(2 * S::WROWS + n) * RS + bc]) + red[(3 * S::WROWS + n) * RS + bc];
      if (!p.to_part) {
        ((u16*)p.y)[g * p.y_g + (int64_t)bcol * p.y_ld + n0 + n] = f2bf(s);
      } else {
        p.part[((int64_t)blockIdx.y * p.nb + bcol) * p.n_total + n0 + n] = s;
      }
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

// Work-group shape of a product over n_rows rows of W per group (groups of
// them) and K of k, for a batch slice of nb rows: 32*rb rows per work-group
// (rb in 8, 5, 4, 2; 256 rows only with at most 32 batch rows), tiles of 64
// k (128 for rb = 2), and (split_k) a power-of-two count of k groups of at
// least 16 tiles.  The plan with the least estimated time wins: rounds of
// work-groups over the 256 compute units of MI355X times each one's weight
// bytes plus a fixed cost of about 150 KB for filling the ring and adding the
// waves' sums (ties: fewer work-groups).
struct WsPlan {
  int rb, kt, kg;
};
WsPlan ws_plan(int nb, int n_rows, int64_t K, int groups, bool split_k) {
  constexpr int64_t kCus = 256, kFixed = 150 * 1024;
  WsPlan best{2, 128, 1};
  int64_t best_cost = INT64_MAX, best_wgs = INT64_MAX;
  for (int rb : {8, 5, 4, 2}) {
    const int rows = 32 * rb, kt = rb >= 4 ? 64 : 128;
    if ((rb == 8 && nb > 32) || n_rows % rows != 0 || K % kt != 0) continue;
    const int64_t blocks = (int64_t)(n_rows / rows) * groups;
    for (int64_t kg = 1; K % (kg * kt) == 0; kg *= 2) {
      const int64_t tiles = K / kg / kt;
      if (kg > 1 && (!split_k || tiles < 16)) break;
      const int64_t wgs = blocks * kg;
      const int64_t cost = (wgs + kCus - 1) / kCus * (rows * (K / kg) * 2 + kFixed);
      if (cost < best_cost || (cost == best_cost && wgs < best_wgs)) {
        best_cost = cost, best_wgs = wgs;
        best = {rb, kt, (int)kg};
      }
    }
  }
  return best;
}

// The kernel of a shape: X tiles of XR rows (at least one whole DMA
// instruction), a 4-stage ring where 4 stages fit 144 KB, else 3.
template <typename XT, int NB, int RB, int XR>
void launch_ws(const WsArgs& a, dim3 grid, hipStream_t stream) {
  constexpr int KT = RB >= 4 ? 64 : 128;
  constexpr int XRR = (XR * KT * (int)sizeof(XT)) % 4096 == 0 ? XR : 2 * XR;
  constexpr int STAGE = 32 * RB * KT * 2 + XRR * KT * (int)sizeof(XT);
  constexpr int ST = 4 * STAGE <= 144 * 1024 ? 4 : 3;
  hipLaunchKernelGGL((wstream_kernel<XT, NB, RB, KT, XRR, ST>), grid, dim3(256), 0, stream, a);
}

template <typename XT, int NB, int XR>
void launch_ws_rb(const WsArgs& a, int rb, dim3 grid, hipStream_t stream) {
  if constexpr (NB == 1) {
    if (rb == 8) return launch_ws<XT, NB, 8, XR>(a, grid, stream);
  }
  if (rb == 5) return launch_ws<XT, NB, 5, XR>(a, grid, stream);
  if (rb == 4) return launch_ws<XT, NB, 4, XR>(a, grid, stream);
  launch_ws<XT, NB, 2, XR>(a, grid, stream);
}

template <typename XT>
hipError_t launch_wstream(const WsArgs& a, const WsPlan& pl, int n_rows, int groups, hipStream_t stream) {
  const dim3 grid((unsigned)(n_rows / (32 * pl.rb)), (unsigned)a.kgroups, (unsigned)groups);
  if (a.nb <= 16) {
    launch_ws_rb<XT, 1, 16>(a, pl.rb, grid, stream);
  } else if (a.nb <= 32) {
    launch_ws_rb<XT, 1, 32>(a, pl.rb, grid, stream);
  } else {
    launch_ws_rb<XT, 2, 64>(a, pl.rb, grid, stream);
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
    const WsPlan pl = ws_plan(a.nb, r, dcq, H, false);
    a.n_total = r, a.kspan = dcq, a.kgroups = 1, a.to_part = 0;
    hipError_t e = launch_wstream<u16>(a, pl, r, H, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Split-k plan of the folded output product for a batch slice of nb rows
int out_folded_kgroups(int nb, int d_model, int64_t K) { return ws_plan(nb, d_model, K, 1, true).kg; }

// fp32 partials of one batch slice (up to 64 sequences), reused slice by
// slice: the larger of the first slice's and the last (partial) slice's
size_t out_folded_workspace_bytes(int B, int d_model, int64_t K) {
  const int nb0 = B < 64 ? B : 64, nbl = B % 64;
  size_t floats = (size_t)out_folded_kgroups(nb0, d_model, K) * nb0;
  if (nbl != 0) {
    const size_t fl = (size_t)out_folded_kgroups(nbl, d_model, K) * nbl;
    floats = fl > floats ? fl : floats;
  }
  return floats * d_model * sizeof(float);
}

// y[b][m] = sum_k w_ov[m][k] o_lat[b][k], k < K = H*r, fp32 out
hipError_t launch_out_folded(int B, int d_model, int64_t K, const float* o_lat, const void* w_ov, float* y,
                             float* workspace, hipStream_t stream) {
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int nb = B - b0 < 64 ? B - b0 : 64;
    const WsPlan pl = ws_plan(nb, d_model, K, 1, true);
    const int kg = pl.kg;
    WsArgs a{};
    a.x = o_lat + (int64_t)b0 * K;
    a.w = (const u16*)w_ov;
    a.y = nullptr;
    a.part = workspace;
    a.x_g = 0, a.x_ld = K, a.w_g = 0, a.w_ld = K, a.y_g = 0, a.y_ld = d_model;
    a.nb = nb, a.n_total = d_model, a.kspan = (int)(K / kg), a.kgroups = kg, a.to_part = 1;
    hipError_t e = launch_wstream<float>(a, pl, d_model, 1, stream);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)nb * d_model;
    hipLaunchKernelGGL(wstream_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, workspace,
                       kg, nb, d_model, y + (int64_t)b0 * d_model, (int64_t)d_model);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla_detail
