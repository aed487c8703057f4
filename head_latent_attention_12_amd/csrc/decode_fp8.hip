// Split-KV decode over an fp8 latent cache (gfx950 / CDNA4).
//
// The latent cache can be stored in FP8 to shrink it further ("MLA from
// scratch", the closing list of what a production implementation adds).  The
// pages fix no format, so this library takes:
//   row (640 bytes) = 512 OCP E4M3FN codes of c_kv / s_row, then the 64 bf16
//                     values of the rotated RoPE key (kept exact: the position
//                     key is small and the pages cache it as is)
//   s_row           = a power of two per row (fp32, separate array): the
//                     smallest 2^e with max|c_kv| <= 448 * 2^e, e in [-116, 63]
// Dequantised values code * s_row are exact in bf16, so the kernel computes
// the bf16 decode of the dequantised cache: scores and P*V run on the bf16
// MFMA with fp32 accumulation, the fp8 operands widened in registers.
//
// Work-group = (sequence, split), 4 waves x 32 heads, as the bf16 kernel.
// Per 32-row tile (7-stage LDS ring filled by DMA, no register staging):
//   S^T[t][h] = sum_k deq(cache[t][k]) q_lat[h][k]: A = cache row t (8 codes
//     per lane, ds_read_b64, widened with the row's scale), B = q_lat^T (the
//     latent part held in registers, the RoPE part read from LDS); the 64 RoPE
//     columns of the row are bf16 already (ds_read_b128)
//   online softmax per head (one head per lane, as in the bf16 kernel)
//   O^T[c][h] += sum_t code[t][c] (P[h][t] s_t): A = codes of column c over 8
//     rows (ds_read_b64_tr_b8), widened unscaled; B = P^T with each row's
//     scale folded in (exact: powers of two)
// Code reads run one group of 4 k-steps (P*V: 2 column blocks) ahead of the
// widening and the MFMAs.  LDS bytes per tile and wave are half those of the
// bf16 kernel; the MFMA work is the same.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla.h"
#include "mla_common.h"

namespace {

constexpr int kH = 128, kR = 512, kDR = 64, kW = kR + kDR;
constexpr int kRowB = kR + 2 * kDR;           // 640 bytes per cache row
constexpr int kNch = kRowB / 16;              // 40 chunks of 16 bytes
constexpr int kTile = 32;                     // rows per tile
constexpr int kTileB = kTile * kRowB;         // 20480
constexpr int kStages = 7;                    // ring depth (6 tiles in flight)
constexpr int kNW = 4;                        // waves
constexpr int kDpw = kTile * kNch / 64 / kNW;  // 5 chunk copies per wave and tile
constexpr int kOps = kDpw + 1;                // + one copy of the tile's row scales
constexpr int kKS = kW / 16;                  // 36 k-steps of the score product
constexpr int kCB = kR / 32;                  // 16 column blocks of the output
static_assert(kTile * kNch % (64 * kNW) == 0, "tile must split evenly over the waves");
static_assert(kOps * (kStages - 2) <= 63, "vmcnt range");
static_assert(kNW * 32 * kR * 2 <= kStages * kTileB, "the epilogue stages the bf16 partials in the ring");

// Slot of logical 16-byte chunk c in LDS row t.  The 32 code chunks XOR their
// low two bits with (t >> 1) & 3, the 8 RoPE chunks with (t >> 1) & 7, each
// inside its own range (rows t and t + 1 start 32 banks apart).  A 2-bit XOR
// keeps every code read at one of four per-lane bases plus an immediate
// offset (no address arithmetic per read), for 2-way bank conflicts on the
// code reads.  An XOR is its own inverse.
__device__ __forceinline__ int f8_slot(int t, int c) {
  return c < 32 ? (c ^ ((t >> 1) & 3)) : (32 + ((c - 32) ^ ((t >> 1) & 7)));
}

// Eight E4M3 codes (lo: bytes 0-3, hi: bytes 4-7) times a power-of-two scale,
// as eight bf16 values in byte order (exact).
__device__ __forceinline__ i16x8 widen8(uint32_t lo, uint32_t hi, float s) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, true);
  return __builtin_bit_cast(i16x8, (u32x4){__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                          __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)});
}

// One tile's DMA for this wave: five 1 KB chunk copies (lane l of copy n
// moves 16 bytes from tb + off[n] to LDS ldst + 1024 n + 16 l) and one copy of
// 64 row scales (lane l: 4 bytes from sb + soff to LDS lsc + 4 l).  Issued from
// inline asm, so the compiler does not wait for the copies before every LDS
// read; each wait on them is explicit (wait_vm_then_barrier).  m0, the DMA's
// LDS base, is saved and restored.
__device__ __forceinline__ void dma_tile(uint64_t tb, uint64_t sb, int ldst, int lsc, const uint32_t (&off)[kDpw],
                                         uint32_t soff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[l]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o0], %[tb]\n\t"
      "s_add_u32 m0, %[l], 1024\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o1], %[tb]\n\t"
      "s_add_u32 m0, %[l], 2048\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o2], %[tb]\n\t"
      "s_add_u32 m0, %[l], 3072\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o3], %[tb]\n\t"
      "s_add_u32 m0, %[l], 4096\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o4], %[tb]\n\t"
      "s_mov_b32 m0, %[ls]\n\ts_nop 0\n\tglobal_load_lds_dword %[so], %[sb]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(save)
      : [tb] "s"(uniform_u64(tb)), [sb] "s"(uniform_u64(sb)), [l] "s"(__builtin_amdgcn_readfirstlane(ldst)),
        [ls] "s"(__builtin_amdgcn_readfirstlane(lsc)), [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]),
        [o3] "v"(off[3]), [o4] "v"(off[4]), [so] "v"(soff)
      : "memory", "scc");
}

// wait until at most `ahead` tiles of this wave's copies are in flight, then
// a work-group barrier
__device__ __forceinline__ void wait_tiles_then_barrier(int ahead) {
  switch (ahead) {
    case 0: wait_vm_then_barrier<0>(); break;
    case 1: wait_vm_then_barrier<kOps>(); break;
    case 2: wait_vm_then_barrier<2 * kOps>(); break;
    case 3: wait_vm_then_barrier<3 * kOps>(); break;
    case 4: wait_vm_then_barrier<4 * kOps>(); break;
    default: wait_vm_then_barrier<5 * kOps>(); break;
  }
}

template <bool PAGED>
__global__ __launch_bounds__(kNW * 64, 1) void decode_latent_fp8_kernel(
    const u16* __restrict__ q_lat, const uint8_t* __restrict__ cache, const float* __restrict__ scales, CacheMap cm,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int32_t batch, int32_t num_splits,
    int32_t chunk, u16* __restrict__ o_part, float* __restrict__ lse_part, float scale_log2) {
  using M = Mma<u16>;
  static_assert(kStages - 2 <= 5, "wait_tiles_then_barrier covers up to 5 tiles ahead");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kTileB];
  // the tile's 32 row scales, twice (lanes 32-63 of a scale copy repeat rows
  // 0-31); every wave copies the same bytes, so each wave's own wait covers them
  __shared__ __attribute__((aligned(16))) float scl[kStages][64];
  // RoPE part of q_lat for the work-group's heads: chunk c of head i's 128 bytes
  // at slot c ^ ((i >> 1) & 7) (reads by 32 heads hit distinct bank groups)
  __shared__ __attribute__((aligned(16))) char qr_lds[kH * 2 * kDR];
  __shared__ int redo_stamp[2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  DecodeItem it;
  if (!decode_item<PAGED, 1>(seq_lens, cm, batch, num_splits, chunk, it)) return;
  const int b = it.b, s = it.s, n_b = it.n_b, seq_len = it.seq_len;
  const int head = wave * 32 + l32;

  const int r0 = s * chunk;
  const int r1 = min(r0 + chunk, seq_len);
  float* lse_out = lse_part + ((int64_t)b * num_splits + s) * kH;
  if (s == 0) {
    for (int e = n_b * kH + (int)threadIdx.x; e < num_splits * kH; e += kNW * 64)
      lse_part[(int64_t)b * num_splits * kH + e] = -INFINITY;
  }
  if (r0 >= r1) {  // only with seq_lens[b] < 1 (inconsistent metadata): nothing to attend
    if (hf == 0) lse_out[head] = -INFINITY;
    return;
  }
  const int ntiles = (r1 - r0 + kTile - 1) / kTile;
  // Packed: the split's absolute rows, clamped into the cache.  Paged: a tile
  // lies in one page (chunk and page size are multiples of 32).
  int64_t row_lo = 0;
  int last_rel;  // last valid row relative to the split's first
  if constexpr (!PAGED) {
    int64_t hi;
    row_lo = it.row_off + r0;
    hi = it.row_off + r1 - 1;
    row_lo = row_lo < 0 ? 0 : (row_lo > cm.total_rows - 1 ? cm.total_rows - 1 : row_lo);
    hi = hi < row_lo ? row_lo : (hi > cm.total_rows - 1 ? cm.total_rows - 1 : hi);
    last_rel = (int)(hi - row_lo);
  } else {
    last_rel = r1 - 1 - r0;
  }
  // cache row of the tile's first row; rel0 = that row relative to the
  // split's first (a packed split clamped at the cache end can have tiles that
  // start past its last valid row: they start at that row instead, so that
  // every copy offset below is non-negative and inside the cache)
  auto tile_row = [&](int tile, int rel0) -> int64_t {
    if constexpr (PAGED) return cm.paged_row(b, r0 + tile * kTile, block_table);
    else return row_lo + rel0;
  };

  // DMA lanes: copy n of this wave fills physical chunk p = (wave * kDpw + n)
  // * 64 + lane of the stage = row p / 40, slot p % 40, which holds logical
  // chunk f8_slot(row, slot) (recomputed per tile rather than kept live).
  const int lds_base = (int)(uintptr_t)((LDS_AS char*)smem);
  auto issue_tile = [&](int tile, int stage) {
    // opaque copies: keep the compiler from hoisting every prologue tile's
    // addresses out of the pass loop (they would stay live, and spill)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    asm volatile("" : "+s"(tile));
    const int rel0 = min(tile * kTile, last_rel);
    const int vmax = min(kTile - 1, last_rel - rel0);  // (>= 0) rows past it repeat the last valid one
    uint32_t off[kDpw];
#pragma unroll
    for (int n = 0; n < kDpw; ++n) {
      const int p = (wave * kDpw + n) * 64 + ln, t = p / kNch;
      off[n] = (uint32_t)(min(t, vmax) * kRowB + 16 * f8_slot(t, p - t * kNch));
    }
    const int64_t row0 = tile_row(tile, rel0);
    dma_tile((uint64_t)(cache + row0 * kRowB), (uint64_t)(scales + row0),
             lds_base + stage * kTileB + wave * kDpw * 1024,
             (int)(uintptr_t)((LDS_AS float*)&scl[stage][0]), off, (uint32_t)(4 * min(ln & 31, vmax)));
  };

  // q_lat^T fragments (B operand of the scores), one head per lane: k-step kk
  // holds columns 16 kk + 8 hf .. +7; the 32 latent k-steps stay in
  // registers, the 4 RoPE ones go to LDS (registers are the limit: the 32 x 512
  // output block takes all 256 AGPRs).  Loaded before any tile copy and used at
  // once, so that the compiler's wait for them drains nothing else.
  constexpr int kKL = kR / 16;  // 32 latent k-steps
  M::Frag qf[kKL];
  {
    const u16* qrow = q_lat + ((int64_t)b * kH + head) * kW + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < kKL; ++kk) qf[kk] = *(const i16x8*)(qrow + 16 * kk);
    i16x8 qr[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) qr[c4] = *(const i16x8*)(qrow - 8 * hf + kR + 8 * (2 * c4 + hf));
#pragma unroll
    for (int kk = 0; kk < kKL; ++kk) asm volatile("" ::"v"(qf[kk]));
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int c = 2 * c4 + hf;
      *(LDS_AS i16x8*)((LDS_AS char*)qr_lds + head * 128 + 16 * (c ^ ((head >> 1) & 7))) = qr[c4];
    }
  }

  // LDS byte offsets inside a stage.  Scores: row l32, code chunk kk, half hf;
  // RoPE chunk 32 + 2 (kk - 32) + hf.  P*V transpose reads (16-lane group G,
  // m = lane % 16): lanes 2j and 2j+1 of a group address row t_j, bytes
  // 8 (m & 1) .. +7 of code chunk 2 cb + (G & 1); the read hands lane m byte m
  // of that chunk from each of the 8 rows, i.e. column 32 cb + lane % 32.  The
  // rows t_j = 16 kh + 8 (j >> 2) + 4 hf + (j & 3) are the ones whose weights
  // this lane holds in accumulator registers 8 kh + j.
  // code chunk 4 g + j of row t sits at 64 g + 16 (j ^ ((t >> 1) & 3))
  const int g_l32 = (l32 >> 1) & 7;  // (the RoPE swizzle; its low two bits are the code swizzle)
  int s_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_base[j] = l32 * kRowB + 8 * hf + 16 * (j ^ (g_l32 & 3));
  int tr_base[2][2];  // [kh][cb & 1]: chunk 2 cb + (G & 1) = 4 (cb >> 1) + (2 (cb & 1) + (G & 1))
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int j = (lane & 15) >> 1;
    const int t = 16 * kh + 8 * (j >> 2) + 4 * hf + (j & 3);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      tr_base[kh][par] = t * kRowB + 8 * (lane & 1) + 16 * ((2 * par + ((lane >> 4) & 1)) ^ ((t >> 1) & 3));
  }

  f32x16 o[kCB];
  float m_ref = -INFINITY;   // exponent reference of this lane's head (log2 units)
  float m_seen = -INFINITY;  // largest score seen so far
  float l_sum = 0.f;
  if (threadIdx.x < 2) redo_stamp[threadIdx.x] = -1;  // ordered by the first barrier below

  // pass 0: normal; pass 1: scores only, for the exact max (after an
  // overflow); pass 2: final pass with that max as the reference
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) o[cb] = zero16();
    l_sum = 0.f;
#pragma unroll
    for (int k = 0; k < kStages - 1; ++k)
      if (k < ntiles) issue_tile(k, k);
    bool redo = false;
    int step = 0;  // block-uniform iteration stamp within the pass
    for (int i = 0; i < ntiles; ++i) {
      wait_tiles_then_barrier(min(kStages - 2, ntiles - 1 - i));
      if (pass == 0 && i > 0 && redo_stamp[(step - 1) & 1] == step - 1) {  // the previous tile overflowed
        redo = true;
        break;
      }
      // tile i + 6 into the stage of tile i - 1 (every wave is past it)
      if (i + kStages - 1 < ntiles) issue_tile(i + kStages - 1, (i + kStages - 1) % kStages);
      const int stage = i % kStages;
      const char* tl = smem + stage * kTileB;
      const int tl_off = (int)(uintptr_t)((LDS_AS char*)tl);
      const float* sc = &scl[stage][0];
      ++step;

      // scores: the code reads run one group of 4 k-steps ahead of the
      // widening and the MFMAs (double-buffered raw operands), so that LDS
      // latency overlaps the matrix work
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
      f32x16 sacc = zero16();
      const float rs = sc[l32];
      auto srd = [&](int kk) -> u32x2 {
        return *(const LDS_AS u32x2*)((LDS_AS char*)(uintptr_t)(tl_off + s_base[kk & 3]) + 64 * (kk >> 2));
      };
      u32x2 sraw[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sraw[0][j] = srd(j);
#pragma unroll
      for (int g = 0; g < kKL / 4; ++g) {
        if (g + 1 < kKL / 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) sraw[(g + 1) & 1][j] = srd(4 * (g + 1) + j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc = M::mma(widen8(sraw[g & 1][j].x, sraw[g & 1][j].y, rs), qf[4 * g + j], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kk = kKL; kk < kKS; ++kk) {
        const int c = 2 * (kk - kKL) + hf;
        const i16x8 a = *(const LDS_AS i16x8*)((LDS_AS char*)tl + l32 * kRowB + 16 * (32 + (c ^ g_l32)));
        const i16x8 q = *(const LDS_AS i16x8*)((LDS_AS char*)qr_lds + head * 128 + 16 * (c ^ ((head >> 1) & 7)));
        sacc = M::mma(a, q, sacc);
      }
      // the first P*V operands, read while the softmax runs
      auto trd = [&](int cb, int kh) -> i32x2 {
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS_AS i32x2*)((LDS_AS char*)(uintptr_t)(tl_off + tr_base[kh][cb & 1]) + 64 * (cb >> 1)));
      };
      i32x2 traw[2][4];
      if (pass != 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) traw[0][j] = trd(j >> 1, j & 1);
      }
      // rows past the split end get -inf; the tile's max in log2 units
      const int valid = r1 - (r0 + i * kTile);
      if (valid < kTile) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 8 * (r >> 2) + 4 * hf + (r & 3);
          if (t >= valid) sacc[r] = -INFINITY;
        }
      }
      float mx = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      mx = fmaxf(mx, xor32(mx, [](float a, float c) { return fmaxf(a, c); })) * scale_log2;
      m_seen = fmaxf(m_seen, mx);
      if (pass == 1) continue;  // max scan only
      if (m_ref == -INFINITY) m_ref = mx;
      if (pass == 0 && __any(mx > m_ref + kRefSlack)) {
        if (lane == 0) redo_stamp[(step - 1) & 1] = step - 1;
      }

      // weights p = 2^(s * scale - ref); B operand = p * s_t rounded to bf16
      // (= bf16(p) * s_t: the scale is a power of two)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      uint32_t pk[8];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 st = *(const LDS_AS f32x4*)((const LDS_AS float*)sc + 8 * a + 4 * hf);
        float p[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          p[c] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * a + c], scale_log2, -m_ref));
          l_sum += p[c];
        }
        pk[2 * a] = cvt_pk_bf16(p[0] * st[0], p[1] * st[1]);
        pk[2 * a + 1] = cvt_pk_bf16(p[2] * st[2], p[3] * st[3]);
      }
      const i16x8 pb0 = __builtin_bit_cast(i16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]});
      const i16x8 pb1 = __builtin_bit_cast(i16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]});
      // O^T += codes^T (P s)^T, reads one group of 2 column blocks ahead
#pragma unroll
      for (int g = 0; g < kCB / 2; ++g) {
        if (g + 1 < kCB / 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) traw[(g + 1) & 1][j] = trd(2 * (g + 1) + (j >> 1), j & 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cb = 2 * g + (j >> 1);
          const i32x2 a = traw[g & 1][j];
          o[cb] = M::mma(widen8((uint32_t)a.x, (uint32_t)a.y, 1.0f), (j & 1) ? pb1 : pb0, o[cb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (pass == 0 && !redo) {  // the last tile may have overflowed too
      wait_vm_then_barrier<0>();
      redo = redo_stamp[(step - 1) & 1] == step - 1;
    }
    if (pass != 1 && !redo) break;
    wait_vm_then_barrier<0>();  // every copy has landed and every wave is here: refill from tile 0
    if (pass == 1) m_ref = m_seen;  // exact max of the split: p <= 1 in the final pass
  }

  // o_part of split (b, s): [H][R] bf16 rows, staged through LDS (the ring is
  // free now) so that each row goes out as coalesced 16-byte stores: 16-byte
  // chunk k of row t at slot k ^ (t & 15).
  const float l_tot = xor32(l_sum, [](float a, float c) { return a + c; });
  const float inv = 1.f / l_tot;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __syncthreads();  // every wave is done with the ring
  LDS_AS char* wrows = (LDS_AS char*)smem + wave * 32 * (kR * 2);
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 4 * cb + q;
      *(LDS_AS u32x2*)(wrows + l32 * (kR * 2) + 16 * (k ^ (l32 & 15)) + 8 * hf) =
          u32x2{cvt_pk_bf16(o[cb][4 * q] * inv, o[cb][4 * q + 1] * inv),
                cvt_pk_bf16(o[cb][4 * q + 2] * inv, o[cb][4 * q + 3] * inv)};
    }
  }
  __syncthreads();
  u16* op = o_part + (((int64_t)b * num_splits + s) * kH + wave * 32) * kR + 8 * lane;
#pragma unroll 8
  for (int t = 0; t < 32; ++t) {
    const u32x4 v = *(const LDS_AS u32x4*)(wrows + t * (kR * 2) + 16 * (lane ^ (t & 15)));
    *(u32x4*)(op + (int64_t)t * kR) = v;
  }
  if (hf == 0) lse_out[head] = (m_ref + __log2f(l_tot)) * kLn2;
}

}  // namespace

// Internal launcher, called by the C-ABI entry points in mla.hip after they
// have validated the arguments (dims are the bf16 instance H 128, r 512,
// d_rope 64).
hipError_t mla_launch_decode_fp8(const void* q_lat, const void* cache, const float* scales,
                                 const mla_detail::CacheMap& cm,
                                 const int32_t* seq_lens, int32_t batch, int32_t num_splits, int32_t chunk,
                                 void* o_part, float* lse_part, float scale_log2, hipStream_t stream) {
  const int64_t blocks = ((int64_t)batch * num_splits + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (cm.block_table != nullptr) {
    hipLaunchKernelGGL((decode_latent_fp8_kernel<true>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream,
                       (const u16*)q_lat, (const uint8_t*)cache, scales, cm, cm.block_table, seq_lens, batch,
                       num_splits, chunk, (u16*)o_part, lse_part, scale_log2);
  } else {
    hipLaunchKernelGGL((decode_latent_fp8_kernel<false>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream,
                       (const u16*)q_lat, (const uint8_t*)cache, scales, cm, nullptr, seq_lens, batch, num_splits,
                       chunk, (u16*)o_part, lse_part, scale_log2);
  }
  return hipGetLastError();
}
