// Absorbed Multi-head Latent Attention decode for MI355X (gfx950 / CDNA4).
//
// Kernels behind the C ABI declared in include/mla.h:
//   absorb_q_kernel          q~ = W_UK^T q_nope          (32x32 MFMA, W_UK staged in LDS; fp32)
//   absorb_q_bf16_kernel     the same for bf16, weight tile and queries copied to LDS by DMA
//   rope_append_kernel       RoPE(q_rope), append [c_kv_new | RoPE(k_rope_new)]
//   absorb_rope_bf16_kernel  the two above in one launch (the absorption blocks do the RoPE work);
//                            appends bf16 rows, or fp8 rows (E4M3 codes + a power-of-two row scale)
//   decode_latent_kernel     split-KV flash decode over the latent cache (32x32 MFMA), packed or
//                            paged cache
//   combine_kernel           log-sum-exp merge of the splits
//   up_v_*_kernel            out = W_UV o_lat             (32x32 MFMA)
//   combine_up_v_*_kernel    the merge formed where W_UV consumes it (one launch)
//   kv_down_*_kernel         c_kv_new, k_rope_new from the hidden state (W_DKV + RMSNorm, W_KR)
// The decode kernel over an fp8 cache is in decode_fp8.hip; the device helpers
// both files use are in mla_common.h.
//
// Sources (page title, section): "DeepSeek MLA, Built From the Paper" section 3
// (absorption identity) and section 2 (decoupled RoPE key shared by the heads);
// "MLA from scratch" (MLAAttention weight shapes, decode-time cache append,
// absorbing projections); "Build a DeepSeek Model (From Scratch)" chapter 3
// figure captions (RoPE pairs, content score plus position score);
// "Multi-head latent attention" (octlm: latent plus shared rotated RoPE key).
//
// MFMA operand layouts used below (v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2f32, wave64):
//   A[m][k]: lane i holds row m = i%32 and KPL consecutive k starting at KPL*(i/32)
//   B[k][n]: lane i holds column n = i%32 and the same k slots
//   C[m][n]: lane i, accumulator r holds row 8*(r/4) + 4*(i/32) + r%4, column i%32
// Only the pairing of k slots between A and B matters for a dot product, so a
// kernel may assign any set of k indices to a lane's slots as long as both
// operands use the same assignment.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "mla.h"

#include "decode_asm.inc"  // hand-scheduled inner blocks of the bf16 decode tile
#include "mla_common.h"

namespace {

// ---------------------------------------------------------------------------
// Row-major LDS tiles with 16-byte chunks XOR-swizzled within groups of 8.
// The LDS has 64 four-byte banks and serves a b128 read 16 lanes at a time;
// a 1152-byte cache row is 288 banks, so odd rows start 32 banks later than
// even ones.  Row t XORs its chunk slot with 4*((t>>1)&1) + ((t>>2)&3): the
// 8 even and the 8 odd rows of a 16-row block then hold one logical chunk in
// 8 distinct slots, so a b128 read of that chunk over 16 rows touches 16
// distinct 4-bank groups, and a transpose read of 4 aligned chunks over 4
// aligned rows (the two even rows differ in bit 2 of the XOR) does too.
// ---------------------------------------------------------------------------

template <int NCH>
__device__ __forceinline__ int swz_chunk(int t, int c) {
  if constexpr (NCH % 8 == 0) {
    return c ^ ((((t >> 1) & 1) << 2) | ((t >> 2) & 3));
  } else {
    return c;
  }
}

template <int ROWB, int NCH>
__device__ __forceinline__ int tile_off(int t, int byte_in_row) {
  return t * ROWB + 16 * swz_chunk<NCH>(t, byte_in_row >> 4) + (byte_in_row & 15);
}

// B/A operand "column of 8 rows" for bf16 via two ds_read_b64_tr_b16: lane i
// (16-lane group G = i/16, m = i%16) receives column col0 + 16*(G%2) + m of
// rows rowA..rowA+3 (slots 0-3) and rowB..rowB+3 (slots 4-7).  Within a
// 16-lane group, source lane 4j+q supplies the 8 bytes at row (base + j),
// columns 4q..4q+3; lane m then receives element m%4 from lanes 4j + m/4.
template <int ROWB, int NCH>
__device__ __forceinline__ i16x8 load_col8_tr(const char* tile, int col0, int rowA, int rowB, int lane) {
  const int m = lane & 15;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (m & 3);
  const int ra = rowA + (m >> 2), rb = rowB + (m >> 2);
  LDS_AS char* base = (LDS_AS char*)tile;
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + tile_off<ROWB, NCH>(ra, 2 * col)));
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(base + tile_off<ROWB, NCH>(rb, 2 * col)));
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The bf16 decode tile runs its two inner phases as hand-scheduled asm blocks
// (decode_asm.inc): the 32x512 fp32 output block lives in AGPRs and the q
// fragments in VGPRs, which the register allocator does not find on its own,
// and LDS reads are pipelined ahead of the MFMAs they feed.  The compiler
// cannot see those MFMAs, so acc_fence() supplies the wait states around the
// accumulators: after zeroing them and before reading them back (24 cycles,
// above the 12 a VALU/AGPR read of an 8-pass 32x32x16 result needs).
template <int CB>
__device__ __forceinline__ void acc_fence(f32x16 (&o)[CB]) {
  static_assert(CB == 16, "acc_fence is written for 16 accumulator blocks");
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                 "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));
}


// Nine 1 KB LDS DMA copies (16 bytes per lane): lane l of copy n moves 16
// bytes from sbase + off[n] to LDS byte ldst + 1024*n + 16*l.  Issued from
// inline asm: the compiler cannot tell which LDS bytes a DMA writes and would
// otherwise wait for every copy in flight (vmcnt(0)) before any later LDS
// read; each wait on these copies is explicit instead (wait_vm_then_barrier).
// m0, which the DMA uses as its LDS base, is saved and restored.
#define MLA_DMA9_BODY(ADDR)                                                                                       \
  "s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o0], " ADDR "\n\t"          \
  "s_add_u32 m0, %[l], 1024\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o1], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 2048\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o2], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 3072\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o3], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 4096\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o4], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 5120\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o5], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 6144\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o6], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 7168\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o7], " ADDR "\n\t"                              \
  "s_add_u32 m0, %[l], 8192\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o8], " ADDR "\n\t"                              \
  "s_mov_b32 m0, %[sv]"

// from a uniform base plus 32-bit lane offsets
__device__ __forceinline__ void lds_dma9(uint64_t sbase, int ldst, const uint32_t (&off)[9]) {
  uint32_t save;
  asm volatile(MLA_DMA9_BODY("%[tb]")
               : [sv] "=&s"(save)
               : [tb] "s"(uniform_u64(sbase)), [l] "s"(__builtin_amdgcn_readfirstlane(ldst)), [o0] "v"(off[0]),
                 [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]), [o4] "v"(off[4]), [o5] "v"(off[5]),
                 [o6] "v"(off[6]), [o7] "v"(off[7]), [o8] "v"(off[8])
               : "memory", "scc");
}

// from per-lane 64-bit addresses
__device__ __forceinline__ void lds_dma9(int ldst, const uint64_t (&addr)[9]) {
  uint32_t save;
  asm volatile(MLA_DMA9_BODY("off")
               : [sv] "=&s"(save)
               : [l] "s"(__builtin_amdgcn_readfirstlane(ldst)), [o0] "v"(addr[0]), [o1] "v"(addr[1]),
                 [o2] "v"(addr[2]), [o3] "v"(addr[3]), [o4] "v"(addr[4]), [o5] "v"(addr[5]), [o6] "v"(addr[6]),
                 [o7] "v"(addr[7]), [o8] "v"(addr[8])
               : "memory", "scc");
}


// ---------------------------------------------------------------------------
// K3: split-KV attention over the latent cache.
//
// One work-group per (sequence b, split s, head group g); NW waves, wave w
// owns 32 heads.  Rows stream HBM -> LDS in 32-row tiles through a 4-stage
// ring filled by global_load_lds (no register staging).  Per tile and wave:
//   S^T[t][h] = sum_k cache[t][k] q_lat[h][k]       (A = cache rows, B = q_lat^T
//                                                    held in registers)
//   online softmax over t per head (the accumulator layout puts one head per
//   lane, so max/sum need only lane-local work plus one xor-32 exchange)
//   O^T[c][h] += sum_t cache[t][c] P[h][t]           (A = cache^T via transpose
//                                                    reads, B = P^T straight
//                                                    from the S^T accumulators)
// ---------------------------------------------------------------------------

template <typename T, int H, int R, int DR, int NW>
struct DecodeShape {
  static constexpr int W = R + DR;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int ROWB = W * ES;
  static constexpr int NCH = ROWB / 16;
  static constexpr int TILE = 32;
  static constexpr int STAGES = 4;
  static constexpr int TILE_BYTES = TILE * ROWB;
  static constexpr int DMA_PER_TILE = TILE * NCH / 64;
  static constexpr int DMA_PER_WAVE = DMA_PER_TILE / NW;
  static constexpr int KS = W / Mma<T>::KSTEP;
  static constexpr int CB = R / 32;
  static constexpr int HEADS_PER_GROUP = 32 * NW;
  static constexpr int GROUPS = (H + HEADS_PER_GROUP - 1) / HEADS_PER_GROUP;
  static_assert(ROWB % 16 == 0, "cache row must be a whole number of 16-byte chunks");
  static_assert((TILE * NCH) % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(W % Mma<T>::KSTEP == 0 && R % 32 == 0, "shape");
  static_assert(DMA_PER_WAVE * 2 <= 63, "vmcnt range");
  static_assert(STAGES * TILE_BYTES <= 160 * 1024, "LDS");
};

template <typename T, int H, int R, int DR, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64, 1) void decode_latent_kernel(
    const T* __restrict__ q_lat, const T* __restrict__ cache, CacheMap cm, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int32_t batch, int32_t num_splits, int32_t chunk, T* __restrict__ o_part,
    float* __restrict__ lse_part, float scale_log2) {
  using S = DecodeShape<T, H, R, DR, NW>;
  using M = Mma<T>;
  constexpr int W = S::W, ROWB = S::ROWB, NCH = S::NCH, TILE = S::TILE, STAGES = S::STAGES;
  constexpr int DPW = S::DMA_PER_WAVE, KS = S::KS, CB = S::CB, TB = S::TILE_BYTES;
  constexpr bool BF16 = sizeof(T) == 2;
  static_assert(!BF16 || (ROWB == 1152 && KS == 36 && CB == 16 && DPW == 9), "asm blocks are generated for 576-wide rows, r = 512, 4 waves");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * TB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (LDS DMA base)
  const int hf = lane >> 5, l32 = lane & 31;
  // every kernel argument, fetched in one batch at entry (otherwise the
  // compiler loads them in dependent rounds between the work lookup's steps)
  asm volatile("" ::"s"(q_lat), "s"(cache), "s"(cm.row_offsets), "s"(cm.total_rows), "s"(cm.total_pages),
               "s"(cm.bt_stride), "s"(cm.page_shift), "s"(block_table), "s"(seq_lens), "s"(batch), "s"(num_splits),
               "s"(chunk), "s"(o_part), "s"(lse_part), "s"(scale_log2));
  DecodeItem it;
  if (!decode_item<PAGED, S::GROUPS>(seq_lens, cm, batch, num_splits, chunk, it)) return;
  const int b = it.b, s = it.s, n_b = it.n_b, seq_len = it.seq_len;
  const int64_t row_off = it.row_off;
  const int g = 0;  // one head group per work item (GROUPS == 1 here)
  static_assert(S::GROUPS == 1, "one work-group covers all heads");
  const int head = g * S::HEADS_PER_GROUP + wave * 32 + l32;
  const bool head_ok = head < H;

  const int r0 = s * chunk;
  const int r1 = min(r0 + chunk, seq_len);
  float* lse_out = lse_part + ((int64_t)b * num_splits + s) * H;
  if (s == 0) {
    for (int e = n_b * H + (int)threadIdx.x; e < num_splits * H; e += NW * 64)
      lse_part[(int64_t)b * num_splits * H + e] = -INFINITY;
  }
  if (r0 >= r1) {  // only with seq_lens[b] < 1 (inconsistent metadata): nothing to attend
    if (hf == 0 && head_ok) lse_out[head] = -INFINITY;
    return;
  }
  const int ntiles = (r1 - r0 + TILE - 1) / TILE;
  // Packed: the split's absolute cache rows, clamped into the cache
  // (inconsistent metadata can then only produce wrong numbers, never a stray
  // access).  Paged: every 32-row tile lies in one page (chunk and page size
  // are multiples of 32); its rows are looked up per tile.
  const char* split_base = nullptr;
  int last_rel;  // last valid row relative to the split's first
  if constexpr (!PAGED) {
    int64_t row_lo = row_off + r0, row_hi = row_off + r1 - 1;
    row_lo = row_lo < 0 ? 0 : (row_lo > cm.total_rows - 1 ? cm.total_rows - 1 : row_lo);
    row_hi = row_hi < row_lo ? row_lo : (row_hi > cm.total_rows - 1 ? cm.total_rows - 1 : row_hi);
    split_base = (const char*)cache + row_lo * ROWB;
    last_rel = (int)(row_hi - row_lo);
  } else {
    last_rel = r1 - 1 - r0;
  }
  // Paged: the page ids of the split's first 64 pages, one per lane (loaded
  // once, clamped as in CacheMap::paged_row), so that a tile's page comes from
  // a lane read instead of a memory access inside the tile loop; a split
  // reaching past 64 pages reads the block table for the tiles beyond.
  const int pg_first = PAGED ? (r0 >> cm.page_shift) : 0;
  int pg_lane = 0;
  if constexpr (PAGED) {
    int pi = pg_first + lane;
    pi = pi < 0 ? 0 : (pi >= cm.bt_stride ? cm.bt_stride - 1 : pi);
    const int64_t pg = block_table[(int64_t)b * cm.bt_stride + pi];
    pg_lane = (int)(pg < 0 ? 0 : (pg >= cm.total_pages ? cm.total_pages - 1 : pg));
  }
  // first byte of the split's tile `tile` (32 consecutive cache rows)
  auto tile_ptr = [&](int tile) -> const char* {
    if constexpr (PAGED) {
      const int t = r0 + tile * TILE;
      const int rel = (t >> cm.page_shift) - pg_first;
      int64_t pg;
      if (rel < 64) {
        pg = __builtin_amdgcn_readlane(pg_lane, rel);
      } else {  // one scalar read of the block table (loaded and waited for in one asm statement)
        int pi = t >> cm.page_shift;
        pi = pi < 0 ? 0 : (pi >= cm.bt_stride ? cm.bt_stride - 1 : pi);
        const uint64_t addr = uniform_u64((uint64_t)(block_table + (int64_t)b * cm.bt_stride + pi));
        int v;
        asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(addr) : "memory");
        pg = v < 0 ? 0 : (v >= cm.total_pages ? cm.total_pages - 1 : v);
      }
      return (const char*)cache + ((pg << cm.page_shift) + (t & ((1 << cm.page_shift) - 1))) * ROWB;
    } else {
      return split_base + (int64_t)tile * TILE * ROWB;
    }
  };

  // DMA: wave instruction n of a tile fills LDS bytes [gi*1024, gi*1024 + 1024)
  // of the stage (gi = wave*DPW + n); lane l writes 16 bytes at gi*1024 + 16*l,
  // which is physical chunk p = gi*64 + l = row t, swizzled slot p % NCH.  A
  // full tile is 32 consecutive cache rows, so the source is the tile base plus
  // 16 * (p ^ swz(t)) (the swizzle only flips the low 3 bits, and NCH % 8 == 0),
  // the same lane offsets for every tile: they are computed once.  Only the
  // last, partial tile clamps its rows.
  uint32_t dma_off[DPW];
#pragma unroll
  for (int n = 0; n < DPW; ++n) {
    const int p = (wave * DPW + n) * 64 + lane;
    dma_off[n] = (uint32_t)(16 * (p ^ swz_chunk<NCH>(p / NCH, 0)));
  }
  // 32 consecutive 1152-byte rows at tbase into a stage
  auto issue_rows = [&](const char* tbase, int stage) {
    LDS_AS char* dst = (LDS_AS char*)smem + stage * TB + wave * DPW * 1024;
    if constexpr (BF16) {
      lds_dma9((uint64_t)tbase, (int)(uintptr_t)dst, dma_off);
    } else {
#pragma unroll
      for (int n = 0; n < DPW; ++n) {
        uint32_t off = dma_off[n];
        asm volatile("" : "+v"(off));  // keeps the 64-bit address sums from being hoisted out of the loop
        __builtin_amdgcn_global_load_lds(tbase + off, dst + n * 1024, 16, 0, 0);
      }
    }
  };
  auto issue_tile = [&](int tile, int stage) {
    const int rel0 = tile * TILE;
    LDS_AS char* dst = (LDS_AS char*)smem + stage * TB + wave * DPW * 1024;
    const char* tbase = tile_ptr(tile);
    if (rel0 + TILE - 1 <= last_rel) {
      issue_rows(tbase, stage);
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));  // recomputed here, not kept live
      if constexpr (BF16) {
        uint64_t addr[DPW];
#pragma unroll
        for (int n = 0; n < DPW; ++n) {
          const int p = (wave * DPW + n) * 64 + ln;
          const int t = p / NCH;
          const int rel = min(rel0 + t, last_rel);
          addr[n] = (uint64_t)(tbase + (int64_t)(rel - rel0) * ROWB + 16 * swz_chunk<NCH>(t, p - t * NCH));
        }
        lds_dma9((int)(uintptr_t)dst, addr);
      } else {
#pragma unroll
        for (int n = 0; n < DPW; ++n) {
          const int p = (wave * DPW + n) * 64 + ln;
          const int t = p / NCH;
          const int rel = min(rel0 + t, last_rel);
          const char* src = tbase + (int64_t)(rel - rel0) * ROWB + 16 * swz_chunk<NCH>(t, p - t * NCH);
          __builtin_amdgcn_global_load_lds(src, dst + n * 1024, 16, 0, 0);
        }
      }
    }
  };

  // Tile t lives in stage stg(t).  The bf16 prologue stages q_lat through
  // stages 0 and 1 while tiles 0 and 1 land in stages 2 and 3, hence the shift.
  constexpr int SOFF = BF16 ? 2 : 0;
  auto stg = [](int t) { return (t + SOFF) % STAGES; };

  typename M::Frag qf[KS];  // q_lat^T fragments (B operand of the score product), one head per lane
  if constexpr (!BF16) {
#pragma unroll
    for (int k = 0; k < STAGES - 1; ++k)
      if (k < ntiles) issue_tile(k, k);
    const T* qrow = q_lat + ((int64_t)b * H + (head_ok ? head : 0)) * W;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float v = qrow[kk * 2 + hf];
      qf[kk] = head_ok ? v : 0.f;
    }
  }

  // Lane base offsets inside a stage.  Scores (bf16): row l32, logical chunk
  // 2*kk + hf; the swizzle only permutes the low 3 bits, so chunk 8a + x sits at
  // 16*(8a + (x ^ swz)) and four bases (kk % 4) plus immediates cover all kk.
  // Transpose reads: the swizzle of rows 16*ks + 8*sel + 4*hf + j does not
  // depend on ks, and logical chunk 4*cb + 2*cg + q/2 needs only the parity
  // of cb, so four bases (sel, parity of cb) cover all 2*CB*2 reads.
  const int lds_base = (int)(uintptr_t)((LDS_AS char*)smem);  // byte address of the ring in LDS
  int s_base[4];
  int tr_base[4];
  if constexpr (BF16) {
    const int sw = swz_chunk<NCH>(l32, 0) ^ 0;  // swizzle value of row l32
#pragma unroll
    for (int q = 0; q < 4; ++q) s_base[q] = l32 * ROWB + 16 * ((2 * q + hf) ^ sw);
    const int m = lane & 15, cg = (lane >> 4) & 1;
#pragma unroll
    for (int sel = 0; sel < 2; ++sel) {
      const int trow = 8 * sel + 4 * hf + (m >> 2);
      const int tsw = swz_chunk<NCH>(trow, 0);
#pragma unroll
      for (int par = 0; par < 2; ++par)
        tr_base[2 * sel + par] = trow * ROWB + 16 * ((4 * par + 2 * cg + ((m & 3) >> 1)) ^ tsw) + 8 * (m & 1);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) s_base[q] = tr_base[q] = 0;
  }

  if constexpr (BF16) {
    // q_lat[b] is 128 rows of 1152 bytes, like four cache tiles, copied with
    // the tiles' coalesced DMA in two halves through stages 0 and 1 (heads
    // 32g.. of half h into stage g, read by wave 2h + g with the score-phase
    // addressing) while tiles 0 and 1 stream into stages 2 and 3.
    static_assert(H == STAGES * 32 && W * S::ES == ROWB, "q_lat of one sequence fills the ring");
    const char* qbase = (const char*)(q_lat + (int64_t)b * H * W);
    issue_rows(qbase, 0);
    issue_rows(qbase + TB, 1);
    if (ntiles > 0) issue_tile(0, stg(0));
    if (ntiles > 1) issue_tile(1, stg(1));
    if (ntiles > 1) wait_vm_then_barrier<2 * DPW>();  // the first half has landed (the tiles may not)
    else wait_vm_then_barrier<DPW>();
    auto read_q = [&](int stage) {
      const char* mine = smem + stage * TB;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qf[kk] = *(const i16x8*)(mine + s_base[kk & 3] + 128 * (kk >> 2));
    };
    if (wave < 2) read_q(wave);
    wait_vm_then_barrier<2 * DPW>();  // stages 0 and 1 are read (lgkmcnt(0) in the barrier)
    issue_rows(qbase + 2 * TB, 0);
    issue_rows(qbase + 3 * TB, 1);
    wait_vm_then_barrier<0>();
    if (wave >= 2) read_q(wave - 2);
    wait_vm_then_barrier<0>();  // every wave holds its fragments: stages 0 and 1 are free
    if (ntiles > 2) issue_tile(2, stg(2));
  }

  __shared__ int redo_stamp[2];  // fp32 path: iteration stamp of an overflowed tile
  __shared__ int redo_flag;      // bf16 path: some wave overflowed in pass 0
  if (threadIdx.x < 2) redo_stamp[threadIdx.x] = -1;  // ordered by the first barrier below
  if (threadIdx.x == 0) redo_flag = 0;

  f32x16 o[CB];
  float m_ref = -INFINITY;   // exponent reference of this lane's head (log2 units)
  float m_seen = -INFINITY;  // largest score seen so far
  float l_sum = 0.f;

  // scores S^T[t][h] of the tile in a stage: lane row t = l32 of the A operand
  auto score_tile = [&](int stage_off) -> f32x16 {
    f32x16 sacc;
    if constexpr (BF16) {
      const int sb0 = lds_base + stage_off + s_base[0], sb1 = lds_base + stage_off + s_base[1];
      const int sb2 = lds_base + stage_off + s_base[2], sb3 = lds_base + stage_off + s_base[3];
      asm volatile(MLA_ASM_SCORE_BLOCK0
                   : [acc] "=&v"(sacc)
                   : [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]),
                     [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]),
                     [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]),
                     [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]),
                     [b0] "v"(sb0), [b1] "v"(sb1), [b2] "v"(sb2), [b3] "v"(sb3)
                   : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",
                     "v251", "v252", "v253", "v254", "v255", "memory");  // keeps the tile DMA issue above
      asm volatile(MLA_ASM_SCORE_BLOCK1
                   : [acc] "+v"(sacc)
                   : [q0] "v"(qf[18]), [q1] "v"(qf[19]), [q2] "v"(qf[20]), [q3] "v"(qf[21]), [q4] "v"(qf[22]),
                     [q5] "v"(qf[23]), [q6] "v"(qf[24]), [q7] "v"(qf[25]), [q8] "v"(qf[26]), [q9] "v"(qf[27]),
                     [q10] "v"(qf[28]), [q11] "v"(qf[29]), [q12] "v"(qf[30]), [q13] "v"(qf[31]),
                     [q14] "v"(qf[32]), [q15] "v"(qf[33]), [q16] "v"(qf[34]), [q17] "v"(qf[35]),
                     [b0] "v"(sb0), [b1] "v"(sb1), [b2] "v"(sb2), [b3] "v"(sb3)
                   : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",
                     "v251", "v252", "v253", "v254", "v255");
    } else {
      const char* tile = smem + stage_off;
      sacc = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const float a = *(const float*)(tile + tile_off<ROWB, NCH>(l32, (kk * 2 + hf) * 4));
        sacc = M::mma(a, qf[kk], sacc);
      }
    }
    return sacc;
  };

  // Rows past the split end (only in its last tile) get -inf; returns the
  // tile's max score of this lane's head in log2 units.
  auto tile_max = [&](f32x16& sacc, int valid) -> float {
    if (valid < TILE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 8 * (r >> 2) + 4 * hf + (r & 3);
        if (t >= valid) sacc[r] = -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    return fmaxf(mx, xor32(mx, [](float a, float c) { return fmaxf(a, c); })) * scale_log2;
  };

  // pass 0: normal; pass 1: scores only, to get the exact max (after an
  // overflow); pass 2: final pass with that max as the reference
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] = zero16();
    if constexpr (BF16) acc_fence(o);
    l_sum = 0.f;
    if (pass > 0) {
#pragma unroll
      for (int k = 0; k < STAGES - 1; ++k)
        if (k < ntiles) issue_tile(k, stg(k));
    }
    bool redo = false;
    if (BF16 && pass != 1) {
      if constexpr (BF16) {  // (only the bf16 instance has the pipelined loop)
        // Software-pipelined tile loop.  Iteration i is one asm block: the
        // softmax of tile i (its scores held in sv) runs on the VALU between
        // the score MFMAs of tile i+1, then P*V of tile i, whose weights the
        // block keeps in fixed registers.  Tile 0's scores come first.  A stage
        // is refilled (tile i+3 into the stage of tile i-1) once every wave has
        // passed the barrier of iteration i.  An overflow (pass 0) is only
        // recorded; the pass runs to its end and the work-group then decides
        // on a redo.
        if (ntiles >= 3) wait_vm_then_barrier<2 * DPW>();
        else if (ntiles == 2) wait_vm_then_barrier<DPW>();
        else wait_vm_then_barrier<0>();
        bool ovf = false;  // wave-uniform: some weight of the pass reached 2^kRefSlack
        // scores of the tile whose softmax the next block computes (register r of
        // the tile's score accumulator)
        float sv0, sv1, sv2, sv3, sv4, sv5, sv6, sv7, sv8, sv9, sv10, sv11, sv12, sv13, sv14, sv15;
        {
          // tile 0's scores (masked past the split end) set the exponent
          // reference and are the first block's softmax input
          f32x16 sacc = score_tile(stg(0) * TB);
          const float mx = tile_max(sacc, r1 - r0);
          if (m_ref == -INFINITY) m_ref = mx;
          sv0 = sacc[0], sv1 = sacc[1], sv2 = sacc[2], sv3 = sacc[3], sv4 = sacc[4], sv5 = sacc[5];
          sv6 = sacc[6], sv7 = sacc[7], sv8 = sacc[8], sv9 = sacc[9], sv10 = sacc[10], sv11 = sacc[11];
          sv12 = sacc[12], sv13 = sacc[13], sv14 = sacc[14], sv15 = sacc[15];
        }
  // operands of the fused block (both forms)
#define MLA_FUSED_OPERANDS \
                       : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]), \
                         [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]), \
                         [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]), \
                         [o14] "+a"(o[14]), [o15] "+a"(o[15]), \
                         [l] "+v"(l_sum), [m0save] "=&s"(m0save), [s0] "+v"(sv0), [s1] "+v"(sv1), \
                         [s2] "+v"(sv2), [s3] "+v"(sv3), [s4] "+v"(sv4), [s5] "+v"(sv5), [s6] "+v"(sv6), \
                         [s7] "+v"(sv7), [s8] "+v"(sv8), [s9] "+v"(sv9), [s10] "+v"(sv10), [s11] "+v"(sv11), \
                         [s12] "+v"(sv12), [s13] "+v"(sv13), [s14] "+v"(sv14), [s15] "+v"(sv15) \
                       : [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]), \
                         [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]), \
                         [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]), \
                         [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]), \
                         [q18] "v"(qf[18]), [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]), \
                         [q22] "v"(qf[22]), [q23] "v"(qf[23]), [q24] "v"(qf[24]), [q25] "v"(qf[25]), \
                         [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]), \
                         [q30] "v"(qf[30]), [q31] "v"(qf[31]), [q32] "v"(qf[32]), [q33] "v"(qf[33]), \
                         [q34] "v"(qf[34]), [q35] "v"(qf[35]), [b0] "v"(sb0), \
                         [b1] "v"(sb1), [b2] "v"(sb2), [b3] "v"(sb3), [t0] "v"(tb0), [t1] "v"(tb1), \
                         [t2] "v"(tb2), [t3] "v"(tb3), [mref] "v"(m_ref), [sc] "s"(scale_log2), [valid] "s"(valid), [nx] "s"(nx), \
                         [dma] "s"(dma), [ldst] "s"(ldst), [tbase] "s"(tb_s), [d0] "v"(dma_off[0]), \
                         [d1] "v"(dma_off[1]), [d2] "v"(dma_off[2]), [d3] "v"(dma_off[3]), [d4] "v"(dma_off[4]), \
                         [d5] "v"(dma_off[5]), [d6] "v"(dma_off[6]), [d7] "v"(dma_off[7]), [d8] "v"(dma_off[8]) \
                       : "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206", \
                         "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", \
                         "v220", "v221", "v222", "v223", "v240", "v241", "v242", "v243", \
                         "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", \
                         "v255", "vcc", "scc", "memory"
        // One pipelined iteration: the scores of tile i+1 (skipped when nx = 0,
        // at the split's last tile) with the softmax of tile i (scores in sv)
        // interleaved, then P*V of tile i; (dma = 1) the copy
        // of the full tile at tb_s into the LDS bytes at ldst, spread over the
        // score MFMAs.  valid = rows of tile i before the split end (the general
        // block masks the rest when it is below 32).
        auto iterate = [&](bool steady, int i, int dma, int ldst, uint64_t tb_s, int nx, int valid) {
          const int cur = lds_base + stg(i) * TB;
          const int nxt = lds_base + stg(i + 1) * TB;
          const int tb0 = cur + tr_base[0], tb1 = cur + tr_base[1], tb2 = cur + tr_base[2], tb3 = cur + tr_base[3];
          const int sb0 = nxt + s_base[0], sb1 = nxt + s_base[1], sb2 = nxt + s_base[2], sb3 = nxt + s_base[3];
          uint32_t m0save;
          if (steady) {
            asm volatile(MLA_ASM_FUSED_BLOCK_STEADY MLA_FUSED_OPERANDS);
          } else {
            asm volatile(MLA_ASM_FUSED_BLOCK MLA_FUSED_OPERANDS);
          }
        };
        // Steady state, free of per-tile branches: tiles i .. i+3 exist and are
        // full (nfull counts the split's full tiles).
        const int nfull = (last_rel + 1) / TILE;
        const uint64_t split_s = uniform_u64((uint64_t)split_base);
        const int ldst_w = lds_base + wave * DPW * 1024;
        int i = 0;
        for (; i + STAGES - 1 < nfull; ++i) {
          wait_vm_then_barrier<DPW>();  // tile i+1 has landed, every wave has finished iteration i-1
          const int t3 = i + STAGES - 1;
          // paged: one scalar read of the block table per tile (16 page ids
          // share a scalar-cache line)
          const uint64_t tb = PAGED ? uniform_u64((uint64_t)tile_ptr(t3)) : split_s + (uint64_t)t3 * (TILE * ROWB);
          iterate(true, i, 1, ldst_w + stg(t3) * TB, tb, 1, TILE);
        }
        // the last STAGES - 1 iterations (and every iteration of a short split)
        for (; i < ntiles; ++i) {
          // tile i+1 has landed (tile i+2 may still be in flight) and every wave
          // has finished iteration i-1
          if (i + 2 < ntiles) wait_vm_then_barrier<DPW>();
          else wait_vm_then_barrier<0>();
          // tile i+3 into the stage of tile i-1: a full tile is copied inside
          // the block, a partial one here
          const int t3 = i + STAGES - 1;
          int dma = 0, ldst = 0;
          uint64_t tbase = (uint64_t)split_base;
          if (t3 < ntiles) {
            if (t3 * TILE + TILE - 1 <= last_rel) {
              dma = 1;
              tbase = (uint64_t)tile_ptr(t3);
              ldst = ldst_w + stg(t3) * TB;
            } else {
              issue_tile(t3, stg(t3));
            }
          }
          const int nx = __builtin_amdgcn_readfirstlane((i + 1 < ntiles) ? 1 : 0);
          const int valid = __builtin_amdgcn_readfirstlane(r1 - (r0 + i * TILE));
          dma = __builtin_amdgcn_readfirstlane(dma);
          ldst = __builtin_amdgcn_readfirstlane(ldst);
          const uint64_t tb_s = uniform_u64(tbase);
          iterate(false, i, dma, ldst, tb_s, nx, valid);
        }
        ovf = __any(!(l_sum < 0x1p64f));  // 2^kRefSlack
#undef MLA_FUSED_OPERANDS
        if (pass == 0) {  // redo if any wave overflowed
          if (ovf && lane == 0) redo_flag = 1;
          wait_vm_then_barrier<0>();
          redo = redo_flag != 0;
        }
      }
    } else {
      // One tile per iteration: scores, softmax, P*V (fp32), or scores only
      // (the max scan of pass 1).  An overflow stamped for a tile is seen by
      // every wave at the next barrier.
      int step = 0;  // block-uniform iteration stamp within the pass
      for (int it = 0; it < ntiles; ++it) {
        const int ahead = min(STAGES - 2, ntiles - 1 - it);
        if (ahead >= 2) wait_vm_then_barrier<2 * DPW>();
        else if (ahead == 1) wait_vm_then_barrier<DPW>();
        else wait_vm_then_barrier<0>();
        if (pass == 0 && it > 0 && redo_stamp[(step - 1) & 1] == step - 1) {  // previous tile overflowed
          redo = true;
          break;
        }
        if (it + STAGES - 1 < ntiles) issue_tile(it + STAGES - 1, stg(it + STAGES - 1));
        const int stage_off = stg(it) * TB;
        ++step;
        f32x16 sacc = score_tile(stage_off);
        const float mx = tile_max(sacc, r1 - (r0 + it * TILE));
        m_seen = fmaxf(m_seen, mx);
        if (BF16 || pass == 1) continue;  // max scan only (bf16 reaches here in pass 1 only)
        if (m_ref == -INFINITY) m_ref = mx;
        if (pass == 0 && __any(mx > m_ref + kRefSlack)) {
          if (lane == 0) redo_stamp[(step - 1) & 1] = step - 1;
        }
        // fp32: p = 2^(s*scale - ref); O^T[c][h] += cache^T P^T
        const char* tile = smem + stage_off;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -m_ref));
          l_sum += sacc[r];
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = 8 * (r >> 2) + 4 * hf + (r & 3);
            const float a = *(const float*)(tile + tile_off<ROWB, NCH>(t, (32 * cb + l32) * 4));
            o[cb] = M::mma(a, sacc[r], o[cb]);
          }
        }
      }
      if (!BF16 && pass == 0 && !redo) {  // the last tile may have overflowed too
        wait_vm_then_barrier<0>();
        redo = redo_stamp[(step - 1) & 1] == step - 1;
      }
    }
    if constexpr (BF16) acc_fence(o);  // last MFMA -> readout / re-zeroing
    if (pass != 1 && !redo) break;
    // every wave is here and its loads have landed: refill the ring from tile 0
    wait_vm_then_barrier<0>();
    if (pass == 1) m_ref = m_seen;  // exact max of the split: p <= 1 in the final pass
  }

  // o_part of split (b, s) is [H][R] in the storage dtype: one contiguous row
  // per head, which its consumers read whole.  A lane holds columns
  // 32*cb + 8*q + 4*hf + (0..3) of its head, so the bf16 block goes through
  // LDS (the ring is free now): each wave writes its 32 heads x R as rows of
  // R*2 bytes, 16-byte chunk k of row t at slot k ^ (t & 15), then stores the
  // rows with one coalesced 16-byte access per lane.  bf16 partials are the
  // fp32 softmax-weighted means rounded once (relative error <= 2^-9).
  const float l_tot = xor32(l_sum, [](float a, float b) { return a + b; });
  const float inv = 1.f / l_tot;
  if constexpr (BF16) {
    static_assert(R * 2 == 1024 && 4 * 32 * R * 2 <= STAGES * TB, "one 1 KB row per lane-chunk, 4 waves in the ring");
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __syncthreads();  // every wave is done with the ring
    LDS_AS char* wrows = (LDS_AS char*)smem + wave * 32 * (R * 2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = 4 * cb + q;  // 16-byte chunk of the row; this lane's half is hf
        *(LDS_AS u32x2*)(wrows + l32 * (R * 2) + 16 * (k ^ (l32 & 15)) + 8 * hf) =
            u32x2{cvt_pk_bf16(o[cb][4 * q] * inv, o[cb][4 * q + 1] * inv),
                  cvt_pk_bf16(o[cb][4 * q + 2] * inv, o[cb][4 * q + 3] * inv)};
      }
    }
    __syncthreads();  // (the rows of a wave are written and read by that wave only)
    // System-scope stores (sc0 sc1) write the partial rows through the XCD's
    // L2 instead of leaving up to its whole capacity dirty for the writeback
    // that ends the kernel; the merge that reads them runs next either way.
    T* op = o_part + (((int64_t)b * num_splits + s) * H + wave * 32) * R + 8 * lane;
#pragma unroll 8
    for (int t = 0; t < 32; ++t) {
      const u32x4 v = *(const LDS_AS u32x4*)(wrows + t * (R * 2) + 16 * (lane ^ (t & 15)));
      asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(op + (int64_t)t * R), "v"(v) : "memory");
    }
    if (hf == 0) lse_out[head] = (m_ref + __log2f(l_tot)) * kLn2;
  } else if (head_ok) {
    T* op = o_part + (((int64_t)b * num_splits + s) * H + head) * R + 4 * hf;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(op + 32 * cb + 8 * q) = f32x4{o[cb][4 * q] * inv, o[cb][4 * q + 1] * inv,
                                                 o[cb][4 * q + 2] * inv, o[cb][4 * q + 3] * inv};
    }
    if (hf == 0) lse_out[head] = (m_ref + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// K4: merge the splits.  The partials of split (b, s) are [H][R], so octet P
// (8 contiguous values: columns 8*(P % (R/8)) .. +7 of head P / (R/8)) is one
// 16-byte (bf16) or 32-byte (fp32) load.  A work-group of 256 threads is SG
// split groups x TQ = 256/SG threads; thread t of a group takes octet
// (block*TQ + t) of every SG-th split, eight splits per step with the loads
// issued together, keeping a running maximum of the log-sum-exps (sums
// rescaled when it grows).  The groups are merged through LDS the same way.
// SG grows with the split count so that a thread sees about eight.
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxGroups = 16;

// Eight consecutive values of a partial: the raw load is kept apart from the
// unpacking to two fp32 quads, so that all of a step's loads are in flight
// before the first is used.
template <typename PT> struct Oct;
template <> struct Oct<float> {
  typedef f32x4 Raw[2];
  static __device__ __forceinline__ void zero(Raw& r) { r[0] = r[1] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  static __device__ __forceinline__ void load(const float* p, Raw& r) {
    r[0] = *(const f32x4*)p;
    r[1] = *(const f32x4*)(p + 4);
  }
  static __device__ __forceinline__ void unpack(const Raw& r, f32x4& a, f32x4& b) {
    a = r[0];
    b = r[1];
  }
};
template <> struct Oct<u16> {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef u32x4 Raw;
  static __device__ __forceinline__ void zero(Raw& r) { r = u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ void load(const u16* p, Raw& r) { r = *(const u32x4*)p; }
  static __device__ __forceinline__ void unpack(const Raw& v, f32x4& a, f32x4& b) {
    a = f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
              __uint_as_float(v[1] & 0xffff0000u)};
    b = f32x4{__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xffff0000u), __uint_as_float(v[3] << 16),
              __uint_as_float(v[3] & 0xffff0000u)};
  }
};

template <int R, typename PT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const PT* __restrict__ o_part,
                                                                  const float* __restrict__ lse_part,
                                                                  int num_splits, int H, int SG,
                                                                  float* __restrict__ o_lat,
                                                                  float* __restrict__ lse_out) {
  constexpr int U = 8;
  __shared__ f32x4 part[kCombineThreads][2];
  __shared__ float wpart[kCombineThreads], mpart[kCombineThreads];
  const int TQ = (int)blockDim.x / SG;
  const int octs = (R / 8) * H;                 // octets per split
  const int blocks_per_b = octs / TQ;
  const int b = (int)blockIdx.x / blocks_per_b;
  const int t = (int)threadIdx.x % TQ, sg = (int)threadIdx.x / TQ;
  const int oct = ((int)blockIdx.x - b * blocks_per_b) * TQ + t;
  const int h = oct / (R / 8), c0 = 8 * (oct - h * (R / 8));
  const float* lp = lse_part + (int64_t)b * num_splits * H + h;
  const int64_t sstride = (int64_t)H * R;
  const PT* op = o_part + (int64_t)b * num_splits * sstride + (int64_t)oct * 8;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  float w = 0.f, m = -INFINITY;
  for (int s0 = sg; s0 < num_splits; s0 += U * SG) {
    float l[U];
    f32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SG;
      l[u] = s < num_splits ? lp[(int64_t)s * H] : -INFINITY;
    }
    typename Oct<PT>::Raw raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SG;
      // an empty split (lse -inf) never wrote its partial
      Oct<PT>::zero(raw[u]);
      if (s < num_splits && l[u] != -INFINITY) Oct<PT>::load(op + s * sstride, raw[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) Oct<PT>::unpack(raw[u], va[u], vb[u]);
    float n = m;
#pragma unroll
    for (int u = 0; u < U; ++u) n = fmaxf(n, l[u]);
    if (n == -INFINITY) continue;  // only empty splits so far
    const float c = __expf(m - n);  // 0 while m = -inf
    acc0 *= c;
    acc1 *= c;
    w *= c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = __expf(l[u] - n);
      w += e;
      acc0 += e * va[u];
      acc1 += e * vb[u];
    }
    m = n;
  }
  part[threadIdx.x][0] = acc0;
  part[threadIdx.x][1] = acc1;
  wpart[threadIdx.x] = w;
  mpart[threadIdx.x] = m;
  __syncthreads();
  if (sg == 0) {
    float mt = -INFINITY;
    for (int g = 0; g < SG; ++g) mt = fmaxf(mt, mpart[g * TQ + t]);
    f32x4 tot0 = {0.f, 0.f, 0.f, 0.f}, tot1 = tot0;
    float wt = 0.f;
    for (int g = 0; g < SG; ++g) {
      const float mg = mpart[g * TQ + t];
      if (mg == -INFINITY) continue;  // a group that saw only empty splits
      const float c = __expf(mg - mt);
      tot0 += c * part[g * TQ + t][0];
      tot1 += c * part[g * TQ + t][1];
      wt += c * wpart[g * TQ + t];
    }
    const int64_t row = (int64_t)b * H + h;
    float* dst = o_lat + row * R + c0;
    *(f32x4*)dst = tot0 * (1.f / wt);
    *(f32x4*)(dst + 4) = tot1 * (1.f / wt);
    if (lse_out != nullptr && c0 == 0) lse_out[row] = mt + __logf(wt);
  }
}

// ---------------------------------------------------------------------------
// K1: q~^T[j][b] = sum_d W_UK[h][d][j] q_nope[b][h][d].  One work-group per
// (head, block of 32*NW latent columns); W_UK[h][:, block] is staged in LDS
// (row-major, swizzled) and read as columns with transpose reads.
// ---------------------------------------------------------------------------

template <typename T, int NW, int DH>
__global__ __launch_bounds__(NW * 64) void absorb_q_kernel(const T* __restrict__ q_nope,
                                                           const T* __restrict__ w_uk, int B, int H, int R,
                                                           T* __restrict__ q_lat, int W) {
  using M = Mma<T>;
  constexpr int ES = (int)sizeof(T);
  constexpr int COLS = 32 * NW;
  constexpr int ROWB = COLS * ES;
  constexpr int NCH = ROWB / 16;
  constexpr int KS = DH / M::KSTEP;
  static_assert(ROWB % 16 == 0 && DH % M::KSTEP == 0, "shape");
  __shared__ __attribute__((aligned(16))) char smem[DH * ROWB];

  const int nblk = R / COLS;
  // The nblk column blocks of a head run on one XCD (work-groups are dealt to
  // the 8 XCDs round-robin), so that the head's q_nope rows come from HBM into
  // one L2 once.  The grid covers whole groups of 8 heads.
  int h, blk;
  {
    const int bid = (int)blockIdx.x;
    const int grp = bid / (kXcds * nblk);
    const int rem = bid - grp * (kXcds * nblk);
    h = grp * kXcds + rem % kXcds;
    blk = rem / kXcds;
  }
  if (h >= H) return;
  const int j0 = blk * COLS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  // query fragments of 32 sequences (rows past B read sequence 0 and are
  // zeroed before use)
  typedef typename M::Frag QF[KS];
  auto load_q = [&](QF& f, int b0) {
    const int bb = b0 + l32;
    const T* qrow = q_nope + ((int64_t)(bb < B ? bb : 0) * H + h) * DH;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (ES == 2) {
        f[kk] = *(const i16x8*)(qrow + 16 * kk + 8 * hf);
      } else {
        f[kk] = qrow[2 * kk + hf];
      }
    }
  };
  // The first 32 queries and the whole weight tile (W_UK[h][:, j0:j0+COLS],
  // PER 16-byte chunks per thread) are all requested before the first wait.
  QF bq;
  load_q(bq, 0);
  constexpr int PER = DH * NCH / (NW * 64);
  static_assert(PER * NW * 64 == DH * NCH, "tile chunks split evenly over the threads");
  int4 wv[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int idx = (int)threadIdx.x + it * NW * 64;
    const int d = idx / NCH, c = idx - (idx / NCH) * NCH;
    wv[it] = *(const int4*)((const char*)(w_uk + ((int64_t)h * DH + d) * R + j0) + 16 * c);
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int idx = (int)threadIdx.x + it * NW * 64;
    const int d = idx / NCH, c = idx - (idx / NCH) * NCH;
    *(int4*)(smem + d * ROWB + 16 * swz_chunk<NCH>(d, c)) = wv[it];
  }
  __syncthreads();

  typename M::Frag af[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if constexpr (ES == 2) {
      af[kk] = load_col8_tr<ROWB, NCH>(smem, 32 * wave, 16 * kk + 8 * hf, 16 * kk + 8 * hf + 4, lane);
    } else {
      af[kk] = *(const float*)(smem + tile_off<ROWB, NCH>(2 * kk + hf, (32 * wave + l32) * 4));
    }
  }
  const int jw = j0 + 32 * wave;
  for (int b0 = 0; b0 < B; b0 += 32) {
    const int bb = b0 + l32;
    const bool bok = bb < B;
    if (b0 > 0) {
      load_q(bq, b0);
      __builtin_amdgcn_sched_barrier(0);  // all KS loads in flight before the first MFMA waits
    }
    f32x16 acc = zero16();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      typename M::Frag b = bq[kk];
      if constexpr (ES == 2) {
        if (!bok) b = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      } else {
        if (!bok) b = 0.f;
      }
      acc = M::mma(af[kk], b, acc);
    }
    if (bok) {
      T* dst = q_lat + ((int64_t)bb * H + h) * W + jw;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 8 * q + 4 * hf;
        if constexpr (ES == 2) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          *(u32x2*)(dst + j) = u32x2{pack2bf(acc[4 * q], acc[4 * q + 1]), pack2bf(acc[4 * q + 2], acc[4 * q + 3])};
        } else {
          *(f32x4*)(dst + j) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
      }
    }
  }
}

constexpr int kMaxRopePairs = 32;  // d_rope <= 64
struct RopeFreqs {
  double theta[kMaxRopePairs];  // theta_i = base^(-2i/d_rope), i < d_rope/2
};

__device__ __forceinline__ void sincos_reduced(double ang, double* s, double* c) {
  // 2*pi = P1 + P2 (P1 the double nearest 2*pi); fma keeps each k*Pn exact
  // inside its subtraction, so |r| <= pi with an error of a few 1e-16
  constexpr double kInv2Pi = 0.15915494309189533577;
  constexpr double P1 = 6.28318530717958623200e+00;
  constexpr double P2 = 2.44929359829470635445e-16;
  const double k = rint(ang * kInv2Pi);
  double r = fma(-k, P1, ang);
  r = fma(-k, P2, r);
  sincos(r, s, c);
}

// RoPE work that the fused bf16 launch hands to the absorption blocks
struct RopeArgs {
  const u16* q_rope;
  const u16* c_kv_new;
  const u16* k_rope_new;
  const int32_t* positions;
  CacheMap cm;  // where the appended rows go
  int DR;
  u16* cache;      // bf16 cache rows [c_kv | k_rope] (nullptr with an fp8 cache)
  uint8_t* cache8;  // fp8 cache rows [codes of c_kv | bf16 k_rope], or nullptr
  float* scale8;    // their power-of-two row scales
};

// fp8 latent cache rows.  The pages name FP8 storage for the latent cache
// ("MLA from scratch", what a production implementation adds) and fix nothing
// else; this library stores c_kv as OCP E4M3FN codes of c_kv / 2^e with one
// exponent per row, e the smallest integer with max|c_kv| <= 448 * 2^e,
// clamped to [kFp8MinExp, kFp8MaxExp] (dequantised values are then exact in
// bf16, and a weight of at most 2^64 times a scale stays finite).
constexpr int kFp8MinExp = -116, kFp8MaxExp = 63;

__device__ __forceinline__ int fp8_row_exponent(float amax) {
  if (!(amax > 0.f)) return kFp8MinExp;
  int x;
  const float m = frexpf(amax, &x);  // amax = m 2^x, m in [0.5, 1); 448 = 0.875 * 2^9
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < kFp8MinExp ? kFp8MinExp : (e > kFp8MaxExp ? kFp8MaxExp : e);
}

// E4M3FN code of y (finite): nearest value, ties to even, magnitudes above
// 448 saturate to 448; the sign bit is kept (also for a zero result).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7eu;
  } else if (a < 0x1p-6f) {  // subnormal range: multiples of 2^-9 (8 * 2^-9 is the first normal)
    code = (uint32_t)rintf(a * 512.f);
  } else {
    int x;
    frexpf(a, &x);  // a = 1.f * 2^(x - 1)
    const int E = x - 1;
    const uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - E));  // 8 .. 16 (16 carries into the exponent)
    code = ((uint32_t)(E + 7) << 3) + (m - 8u);
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

// A bf16 pair (x0, x1) turned by the angle whose sine and cosine are (sn, cn),
// rounded once
__device__ __forceinline__ uint32_t rope_rotate_bf16(uint32_t x, double sn, double cn) {
  const double x0 = (double)bf2f((u16)(x & 0xffffu)), x1 = (double)bf2f((u16)(x >> 16));
  return (uint32_t)d2bf(x0 * cn - x1 * sn) | ((uint32_t)d2bf(x0 * sn + x1 * cn) << 16);
}

// RoPE of pair i of a bf16 pair (x0, x1) at position pos, rounded once
__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t x, int pos, double theta) {
  double sn, cn;
  sincos_reduced((double)pos * theta, &sn, &cn);
  return rope_rotate_bf16(x, sn, cn);
}

// bf16: the weight tile and the queries of 64 sequences at a time are copied
// into LDS by DMA (1 KB per wave instruction, no register staging), all issued
// before the one wait, so a work-group pays a single HBM round trip up front.
// Query rows are stored with their 16-byte chunks XOR-swizzled by row, which
// makes the fragment reads (lane = sequence) conflict-free.
// The bf16 instance's latent and RoPE widths are compile-time constants here
// (the block index split and the RoPE pair indexing are then shifts, not
// divisions); the launchers check them.
constexpr int kAbsorbR = 512, kAbsorbDR = 64;

template <int DH, bool ROPE, bool PAGED>
__device__ __forceinline__ void absorb_bf16_block(int bid, const u16* __restrict__ q_nope,
                                                  const u16* __restrict__ w_uk, int B, int H,
                                                  u16* __restrict__ q_lat, int W, char* wt, char* qs,
                                                  const RopeArgs& ra, const RopeFreqs& freqs) {
  constexpr int R = kAbsorbR, DR = kAbsorbDR;
  using M = Mma<u16>;
  constexpr int COLS = 64, ROWB = 2 * COLS, NCH = ROWB / 16, KS = DH / M::KSTEP;
  constexpr int QROWS = 64, QROWB = 2 * DH, QCH = QROWB / 16;
  constexpr int WCOP = DH * ROWB / 1024 / 2;      // weight DMA copies per wave
  constexpr int QCOP = QROWS * QROWB / 1024 / 2;  // query DMA copies per wave
  static_assert(WCOP >= 1 && QCOP >= 1 && (QCH & (QCH - 1)) == 0, "shape");

  constexpr int nblk = R / COLS;
  // the nblk column blocks of a head run on one XCD (its L2 then serves the
  // head's queries to all of them); the grid covers whole groups of 8 heads
  int h, blk;
  {
    const int grp = bid / (kXcds * nblk);
    const int rem = bid - grp * (kXcds * nblk);
    h = grp * kXcds + rem % kXcds;
    blk = rem / kXcds;
  }
  if (h >= H) return;
  const int j0 = blk * COLS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  // RoPE (fused launch, waves 2 and 3 of the work-group).  The query
  // rotations come in units of (sequence, 8 heads): work-group g = h*nblk +
  // blk takes units g, g + H*nblk, ...; in wave 2, lane l turns pair l % 32
  // of heads 8*group + l/32 + 2k (k = 0..3), so that the angle's sine and
  // cosine (fp64, the costly part) are formed once per four rotations.
  // Wave 3 appends the cache row of sequence h*nblk + blk (mod H*nblk).
  // These waves touch no LDS and wait only for their own loads, so their work
  // runs while waves 0 and 1 wait for their copies; they then join the
  // absorption waves' barriers (one, plus two per further block of 64
  // sequences) and leave.
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (ROPE) {
    if (threadIdx.x >= 128) {
      constexpr int half = DR / 2;
      static_assert(half == 32, "a lane's pair is its lane index mod 32");
      const int tid = (int)threadIdx.x - 128;
      const int W2 = R + DR;
      if (tid < 64) {
        const int hgs = (H + 7) / 8;  // head groups of 8
        const int units = B * hgs;
        const int i = tid & 31;
        for (int u = h * nblk + blk; u < units; u += H * nblk) {
          const int bb = u / hgs, h0 = 8 * (u - bb * hgs) + (tid >> 5);
          // the four pairs' loads, then the angle, then the rotations
          uint32_t x[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            x[k] = *(const uint32_t*)(ra.q_rope + ((int64_t)bb * H + min(h0 + 2 * k, H - 1)) * DR + 2 * i);
          double sn, cn;
          sincos_reduced((double)ra.positions[bb] * freqs.theta[i], &sn, &cn);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (h0 + 2 * k < H)
              *(uint32_t*)(q_lat + ((int64_t)bb * H + h0 + 2 * k) * W2 + R + 2 * i) = rope_rotate_bf16(x[k], sn, cn);
        }
      }
      // the appended rows, by wave 3 (eight latent values per lane): [c_kv_new |
      // RoPE(k_rope_new)] with c_kv_new bit for bit, or the fp8 row: codes of
      // c_kv_new / 2^e with e from the row's max |c_kv_new| (a wave-wide
      // maximum), then the rotated key and the scale
      static_assert(R == 8 * 64, "one wave holds the appended latent, eight values per lane");
      if (tid >= 64) {
        const int al = tid - 64;  // lane of wave 3
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const bool fp8 = ra.cache8 != nullptr;
        for (int bb = h * nblk + blk; bb < B; bb += H * nblk) {
          const int ti = min(al, half - 1);
          const u32x4 cv = *(const u32x4*)(ra.c_kv_new + (int64_t)bb * R + 8 * al);
          const uint32_t k = *(const uint32_t*)(ra.k_rope_new + (int64_t)bb * DR + 2 * ti);
          const int pos = ra.positions[bb];
          const int64_t off = PAGED ? 0 : ra.cm.row_offsets[bb];
          const int64_t row = ra.cm.row(bb, pos, off);
          const uint32_t kr = rope_pair_bf16(k, pos, freqs.theta[ti]);
          if (!fp8) {
            u16* crow = ra.cache + row * W2;
            *(u32x4*)(crow + 8 * al) = cv;
            if (al < half) *(uint32_t*)(crow + R + 2 * al) = kr;
          } else {
            uint8_t* crow = ra.cache8 + row * (R + 2 * DR);
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[2 * e] = bf2f((u16)(cv[e] & 0xffffu));
              v[2 * e + 1] = bf2f((u16)(cv[e] >> 16));
            }
            float mx = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
            const int ex = fp8_row_exponent(wave_reduce_f(mx, [](float a, float b) { return fmaxf(a, b); }));
            const float inv = ldexpf(1.f, -ex);
            uint32_t c[2];
#pragma unroll
            for (int w = 0; w < 2; ++w)
              c[w] = e4m3_code(v[4 * w] * inv) | (e4m3_code(v[4 * w + 1] * inv) << 8) |
                     (e4m3_code(v[4 * w + 2] * inv) << 16) | (e4m3_code(v[4 * w + 3] * inv) << 24);
            *(u32x2*)(crow + 8 * al) = u32x2{c[0], c[1]};
            if (al < half) *(uint32_t*)(crow + R + 4 * al) = kr;
            if (al == 0) ra.scale8[row] = ldexpf(1.f, ex);
          }
        }
      }
      const int nbar = 1 + 2 * ((B + QROWS - 1) / QROWS - 1);
      for (int n = 0; n < nbar; ++n) __syncthreads();
      return;
    }
  }
  // LDS chunk p of the query block holds row p / QCH, chunk (p % QCH) ^ (row % QCH)
  auto issue_q = [&](int b0) {
#pragma unroll
    for (int n = 0; n < QCOP; ++n) {
      if ((wave * QCOP + n) * 64 / QCH >= B - b0) break;  // the copy's rows are all past B
      const int p = (wave * QCOP + n) * 64 + lane;
      const int row = p / QCH, c = (p % QCH) ^ (row & (QCH - 1));
      const int bb = b0 + row;
      const char* src = (const char*)(q_nope + ((int64_t)(bb < B ? bb : 0) * H + h) * DH) + 16 * c;
      __builtin_amdgcn_global_load_lds(src, (LDS_AS char*)qs + (wave * QCOP + n) * 1024, 16, 0, 0);
    }
  };
  issue_q(0);
  // weight tile W_UK[h][:, j0:j0+64]: LDS chunk p holds row d = p / NCH, chunk
  // swz(d, p % NCH) (the swizzle is an XOR, its own inverse)
#pragma unroll
  for (int n = 0; n < WCOP; ++n) {
    const int p = (wave * WCOP + n) * 64 + lane;
    const int d = p / NCH, c = swz_chunk<NCH>(d, p % NCH);
    const char* src = (const char*)(w_uk + ((int64_t)h * DH + d) * R + j0) + 16 * c;
    __builtin_amdgcn_global_load_lds(src, (LDS_AS char*)wt + (wave * WCOP + n) * 1024, 16, 0, 0);
  }
  __syncthreads();  // (waits for this work-group's DMA)
  typename M::Frag af[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    af[kk] = load_col8_tr<ROWB, NCH>(wt, 32 * wave, 16 * kk + 8 * hf, 16 * kk + 8 * hf + 4, lane);
  const int jw = j0 + 32 * wave;
  for (int b0 = 0; b0 < B; b0 += QROWS) {
    if (b0 > 0) {
      __syncthreads();  // every wave is done with the previous block
      issue_q(b0);
      __syncthreads();
    }
#pragma unroll
    for (int sub = 0; sub < QROWS / 32; ++sub) {
      const int row = 32 * sub + l32, bb = b0 + row;
      if (b0 + 32 * sub >= B) break;
      const bool bok = bb < B;
      f32x16 acc = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        i16x8 b = *(const i16x8*)(qs + row * QROWB + 16 * ((2 * kk + hf) ^ (row & (QCH - 1))));
        if (!bok) b = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
        acc = M::mma(af[kk], b, acc);
      }
      if (bok) {
        u16* dst = q_lat + ((int64_t)bb * H + h) * W + jw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          *(u32x2*)(dst + 8 * q + 4 * hf) =
              u32x2{pack2bf(acc[4 * q], acc[4 * q + 1]), pack2bf(acc[4 * q + 2], acc[4 * q + 3])};
        }
      }
    }
  }
}

// LDS of one absorption block: the weight tile and 64 query rows
template <int DH> struct AbsorbLds {
  static constexpr int WT = DH * 128, QS = 64 * 2 * DH;
};

template <int DH>
__global__ __launch_bounds__(128) void absorb_q_bf16_kernel(const u16* __restrict__ q_nope,
                                                            const u16* __restrict__ w_uk, int B, int H, int R,
                                                            u16* __restrict__ q_lat, int W) {
  __shared__ __attribute__((aligned(1024))) char wt[AbsorbLds<DH>::WT];
  __shared__ __attribute__((aligned(1024))) char qs[AbsorbLds<DH>::QS];
  (void)R;  // kAbsorbR (checked by the launcher)
  absorb_bf16_block<DH, false, false>((int)blockIdx.x, q_nope, w_uk, B, H, q_lat, W, wt, qs, RopeArgs{}, RopeFreqs{});
}

// ---------------------------------------------------------------------------
// K5: out^T[d][b] = sum_j W_UV[h][d][j] o_lat[b][h][j].
// bf16: one work-group per (head, 32 output rows).  The weight tile (32 rows of
// R bf16) and the o_lat rows of 16 sequences at a time are copied into LDS by
// coalesced DMA (one 1 KB row slice per instruction), their 16-byte chunks
// XOR-swizzled by row so that fragment reads are conflict-free.  The 4 waves
// split the j range and sum their 32x32 partial tiles through LDS, each wave
// finishing one quarter of the rows.  The fp32 o_lat enters as hi + lo bf16
// parts (two MFMAs per step), keeping it exact to about 2^-16.  The row blocks
// of one head run on one XCD.
// fp32: one wave per (head, 32 rows), fp32 MFMA over the whole j range.
// ---------------------------------------------------------------------------

template <int R>
__global__ __launch_bounds__(256) void up_v_bf16_kernel(const float* __restrict__ o_lat, const u16* __restrict__ w_uv,
                                                        int B, int H, int DV, float* __restrict__ out) {
  using M = Mma<u16>;
  constexpr int JW = R / 4;          // j range of one wave
  constexpr int G4 = JW / 64;        // groups of 4 MFMA steps
  constexpr int WROW = R * 2;        // bytes of a weight row
  constexpr int OROW = R * 4;        // bytes of an o_lat row
  constexpr int BCH = 16;            // sequences per o_lat chunk
  static_assert(R == 512, "one 1 KB DMA per weight row and two per o_lat row");
  __shared__ __attribute__((aligned(16))) char wt[32 * WROW];
  __shared__ __attribute__((aligned(16))) char ot[BCH * OROW];
  __shared__ f32x4 red[4][4][64];    // [wave][row quarter][lane]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int nblk = DV / 32;
  // the nblk row blocks of a head run on one XCD, whose L2 then serves them
  // the head's o_lat rows; the grid covers whole groups of 8 heads
  int h, d0;
  {
    const int bid = (int)blockIdx.x;
    const int grp = bid / (kXcds * nblk);
    const int rem = bid - grp * (kXcds * nblk);
    h = grp * kXcds + rem % kXcds;
    d0 = (rem / kXcds) * 32;
  }
  if (h >= H) return;

  // weight rows 8*wave .. 8*wave+7: LDS chunk l of row n holds source chunk l ^ (n & 15)
  {
    const char* wbase = (const char*)(w_uv + ((int64_t)h * DV + d0) * R);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = 8 * wave + i;
      const char* src = wbase + (int64_t)n * WROW + 16 * (lane ^ (n & 15));
      __builtin_amdgcn_global_load_lds(src, (LDS_AS char*)wt + n * WROW, 16, 0, 0);
    }
  }
  const int jw = wave * JW;
  for (int b0 = 0; b0 < B; b0 += BCH) {
    // o_lat rows b0 .. b0+15 (two 1 KB halves each, chunk c at c ^ (row & 15))
#pragma unroll
    for (int i = 0; i < 2 * BCH / 4; ++i) {
      const int k = wave * (2 * BCH / 4) + i;  // copy k: row k/2, half k%2
      const int r = k >> 1, half = k & 1;
      if (b0 + r < B) {
        const char* src = (const char*)(o_lat + ((int64_t)(b0 + r) * H + h) * R) + 16 * ((64 * half + lane) ^ (r & 15));
        __builtin_amdgcn_global_load_lds(src, (LDS_AS char*)ot + r * OROW + half * 1024, 16, 0, 0);
      }
    }
    __syncthreads();  // (waits for the DMA of this work-group)
    const int bb = b0 + l32;
    const bool bok = l32 < BCH && bb < B;
    f32x16 acc = zero16();
#pragma unroll
    for (int g = 0; g < G4; ++g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kw = jw + 64 * g + 16 * u + 8 * hf;  // this lane's 8 k slots: kw .. kw+7
        const i16x8 a = *(const i16x8*)(wt + l32 * WROW + 16 * ((kw >> 3) ^ (l32 & 15)));
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
        if (bok) {
          const int c = kw >> 2;  // fp32 chunks c, c+1
          x0 = *(const f32x4*)(ot + l32 * OROW + 16 * (c ^ (l32 & 15)));
          x1 = *(const f32x4*)(ot + l32 * OROW + 16 * ((c + 1) ^ (l32 & 15)));
        }
        const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = cvt_pk_bf16(xv[2 * e], xv[2 * e + 1]);
          lo[e] = cvt_pk_bf16(xv[2 * e] - __uint_as_float(hi[e] << 16),
                              xv[2 * e + 1] - __uint_as_float(hi[e] & 0xffff0000u));
        }
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        acc = M::mma(a, __builtin_bit_cast(i16x8, u32x4{hi[0], hi[1], hi[2], hi[3]}), acc);
        acc = M::mma(a, __builtin_bit_cast(i16x8, u32x4{lo[0], lo[1], lo[2], lo[3]}), acc);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    __syncthreads();
    // wave w sums row quarter q = w (rows 8w + 4hf + 0..3 of the 32-row block)
    f32x4 sum = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
    if (bok) *(f32x4*)(out + ((int64_t)bb * H + h) * DV + d0 + 8 * wave + 4 * hf) = sum;
    __syncthreads();  // red and ot are reused by the next chunk
  }
}

__global__ __launch_bounds__(64) void up_v_f32_kernel(const float* __restrict__ o_lat, const float* __restrict__ w_uv,
                                                      int B, int H, int DV, int R, float* __restrict__ out) {
  using M = Mma<float>;
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  const int nblk = DV / 32;
  const int h = blockIdx.x / nblk;
  const int d0 = (blockIdx.x - h * nblk) * 32;
  const float* wrow = w_uv + ((int64_t)h * DV + d0 + l32) * R;
  for (int b0 = 0; b0 < B; b0 += 32) {
    const int bb = b0 + l32;
    const bool bok = bb < B;
    const float* orow = o_lat + ((int64_t)(bok ? bb : 0) * H + h) * R;
    f32x16 acc = zero16();
    for (int kk = 0; kk < R / 2; ++kk) {
      const float x = bok ? orow[2 * kk + hf] : 0.f;
      acc = M::mma(wrow[2 * kk + hf], x, acc);
    }
    if (bok) {
      float* dst = out + ((int64_t)bb * H + h) * DV + d0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(dst + 8 * q + 4 * hf) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  }
}

// ---------------------------------------------------------------------------
// K4 + K5 in one kernel: out[b][h][d] = sum_j W_UV[h][d][j] o[b][h][j], where
// o is the merge of the splits (as K4), formed where it is consumed instead of
// going through memory.
// bf16: one work-group (8 waves) per (head, block of DB = 32*NH output rows);
// the blocks of a head run on one XCD, whose L2 then serves them the head's
// partials.  The DB weight rows are copied into LDS by DMA at the start.  Per
// chunk of up to 32 sequences:
//   merge: a unit is a (sequence, part) pair covering the splits s = part
//     (mod WPR) of that sequence; WPR is the largest power of two with
//     rows * WPR <= 8 (1 from 5 rows up), so that short chunks still use
//     every wave, and then each wave holds at most one unit.  A wave takes
//     up to UPW units: it reads their log-sum-exps, then issues the loads of
//     all their splits that hold data (one contiguous 1 KB partial row each,
//     16 bytes per lane) together, so a second round trip serves them.
//     Units of one sequence add their sums through LDS.  The merged fp32 row
//     enters LDS as a hi and a lo bf16 row (16-byte chunk k of row t at slot
//     k ^ (t & 15)).
//   product: wave w takes output rows 32*(w/4) .. +31 of the block and the j
//     quarter w % 4 (two MFMAs per k step, hi and lo); the four quarters are
//     summed through LDS (which then reuses the merged rows' bytes).
// fp32: one wave per (sequence, head): lane c merges column c, then lane d
// forms out[d] with fp32 FMAs over j from the merged row in LDS.
// ---------------------------------------------------------------------------

constexpr int kCuvWaves = 8;
constexpr int kCuvRows = 32;      // sequences per chunk (the MFMA's N)
constexpr int kCuvMaxRankF32 = 256;

__device__ __forceinline__ float wave_max_f(float v) {
  return wave_reduce_f(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum_f(float v) {
  return wave_reduce_f(v, [](float a, float b) { return a + b; });
}

// Log-sum-exp statistics of one (sequence, head) over its S splits (lse at
// lp[s * H]): mx = max_s lse, wsum = sum_s exp(lse - mx); -inf and 0 when
// every split is empty.  Every lane returns the same values.
__device__ __forceinline__ void lse_stats(const float* __restrict__ lp, int S, int H, int lane, float& mx,
                                          float& wsum) {
  float ml = -INFINITY, wl = 0.f;
  for (int s = lane; s < S; s += 64) {
    const float l = lp[(int64_t)s * H];
    if (l > ml) {
      wl = wl * __expf(ml - l) + 1.f;  // (0 while ml = -inf)
      ml = l;
    } else if (l != -INFINITY) {
      wl += __expf(l - ml);
    }
  }
  mx = wave_max_f(ml);
  wsum = wave_sum_f(ml == -INFINITY ? 0.f : wl * __expf(ml - mx));
}

// hi + lo bf16 parts of a merged row's 8 columns of this lane into LDS row t
__device__ __forceinline__ void cuv_put_row(char* ot, int t, int lane, const float (&o)[8]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = cvt_pk_bf16(o[2 * e], o[2 * e + 1]);
    lo[e] = cvt_pk_bf16(o[2 * e] - __uint_as_float(hi[e] << 16), o[2 * e + 1] - __uint_as_float(hi[e] & 0xffff0000u));
  }
  LDS_AS char* row = (LDS_AS char*)ot + t * 2048 + 16 * (lane ^ (t & 15));
  *(LDS_AS u32x4*)row = hi;
  *(LDS_AS u32x4*)(row + 1024) = lo;
}

// The merge of one chunk (see above), UPW units per wave with NB splits of
// each in flight.  The splits of a unit are taken 64 at a time: lane i holds
// the log-sum-exp of the group's split i (one load), the group raises the
// unit's running maximum (the sums so far rescaled), and split i's weight is
// read from lane i.  A split past its sequence's last (fewer rows than
// num_splits chunks) has log-sum-exp -inf and was never written: its row is
// not loaded, so a ragged batch reads only the rows that hold data.  Leaves
// the merged rows in ot and, if lse_out is not null, the merged
// log-sum-exps there.  NWAVES: the work-group's waves.
template <int UPW, int NB, int NWAVES = kCuvWaves>
__device__ __forceinline__ void cuv_merge(const u16* __restrict__ o_part, const float* __restrict__ lse_part,
                                          int S, int H, int h, int b0, int nb, int WPR, int wave, int lane,
                                          char* ot, float (*xs)[64][8], float* xm, float* xw,
                                          float* __restrict__ lse_out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  static_assert(64 % NB == 0, "a batch of splits lies in one group of 64");
  constexpr int R = 512;
  const int units = nb * WPR;
  const int part = wave % WPR;                                // the same for all units of a wave
  const int spu = part < S ? (S - part + WPR - 1) / WPR : 0;  // splits of this part: s = part + WPR*i
  bool uok[UPW];
  int trow[UPW];
  int64_t base[UPW];  // (b*S + part)*H + h: split i of the unit is row base + i*WPR*H of o_part / lse_part
  // The partial rows are read through a buffer resource over the sequence's
  // S*H*R values (at most 512 MB): every lane's offset is 16*lane and each
  // row's (uniform) byte offset goes in the scalar offset, so a batch of loads
  // needs no offset registers.
  __amdgpu_buffer_rsrc_t rsrc[UPW];
  const uint32_t nrec = (uint32_t)S * (uint32_t)H * (R * 2);
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    const int u = wave + NWAVES * k;
    uok[k] = u < units;
    trow[k] = uok[k] ? u / WPR : 0;
    base[k] = ((int64_t)(b0 + trow[k]) * S + part) * H + h;
    rsrc[k] = __builtin_amdgcn_make_buffer_rsrc((void*)(o_part + (int64_t)(b0 + trow[k]) * S * H * R), (short)0,
                                                (int)nrec, 0x00020000);
  }
  const int64_t istride = (int64_t)WPR * H;
  float acc[UPW][8], mx[UPW], wsum[UPW];
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    mx[k] = -INFINITY;
    wsum[k] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  }
  for (int g0 = 0; g0 < spu; g0 += 64) {
    const int gn = min(64, spu - g0);  // splits of this group (per unit)
    float ev[UPW];
    uint64_t live[UPW];  // bit i: split g0 + i holds data (finite log-sum-exp)
    int nlive = 0;       // one past the last such split over the wave's units
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      float lv = -INFINITY;
      if (uok[k] && lane < gn) lv = lse_part[base[k] + (int64_t)(g0 + lane) * istride];
      live[k] = __ballot(lv != -INFINITY);
      nlive = max(nlive, live[k] == 0 ? 0 : 64 - __builtin_clzll(live[k]));
      // the group raises the unit's running maximum
      const float mn = fmaxf(mx[k], wave_max_f(lv));
      ev[k] = 0.f;
      if (mn != -INFINITY) {
        const float c = __expf(mx[k] - mn);  // 0 while mx = -inf
        wsum[k] *= c;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] *= c;
        mx[k] = mn;
        ev[k] = lv == -INFINITY ? 0.f : __expf(lv - mn);
        wsum[k] += wave_sum_f(ev[k]);
      }
    }
    for (int u0 = 0; u0 < nlive; u0 += NB) {
      u32x4 raw[UPW][NB];
#pragma unroll
      for (int k = 0; k < UPW; ++k)
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          raw[k][u] = u32x4{0u, 0u, 0u, 0u};
          if (((live[k] >> (u0 + u)) & 1) == 0) continue;  // (u0 + u < 64: NB divides 64)
          const uint32_t soff = (uint32_t)((part + WPR * (g0 + u0 + u)) * H + h) * (R * 2);
          raw[k][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc[k], 16 * lane, soff, 0));
        }
#pragma unroll
      for (int k = 0; k < UPW; ++k)
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          // the split's weight (0 for a split without data, which was not loaded)
          const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ev[k]), u0 + u));
          if (c == 0.f) continue;
          const u32x4 v = raw[k][u];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[k][2 * e] = fmaf(c, __uint_as_float(v[e] << 16), acc[k][2 * e]);
            acc[k][2 * e + 1] = fmaf(c, __uint_as_float(v[e] & 0xffff0000u), acc[k][2 * e + 1]);
          }
        }
    }
  }
  if (WPR == 1) {
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      if (!uok[k]) continue;
      const float inv = wsum[k] > 0.f ? 1.f / wsum[k] : 0.f;  // 0: every split empty
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = acc[k][e] * inv;
      cuv_put_row(ot, trow[k], lane, o);
      if (lse_out != nullptr && lane == 0) lse_out[(int64_t)(b0 + trow[k]) * H + h] = mx[k] + __logf(wsum[k]);
    }
  } else {  // one unit per wave (units <= NWAVES): the parts of a sequence are waves t*WPR .. t*WPR + WPR-1
    if (uok[0]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[wave][lane][e] = acc[0][e];
      if (lane == 0) {
        xm[wave] = mx[0];
        xw[wave] = wsum[0];
      }
    }
    __syncthreads();
    if (uok[0] && part == 0) {
      float mt = -INFINITY;
      for (int p = 0; p < WPR; ++p) mt = fmaxf(mt, xm[wave + p]);
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float wt = 0.f;
      if (mt != -INFINITY) {
        for (int p = 0; p < WPR; ++p) {
          if (xm[wave + p] == -INFINITY) continue;  // a part with only empty splits
          const float c = __expf(xm[wave + p] - mt);
          wt += c * xw[wave + p];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = fmaf(c, xs[wave + p][lane][e], o[e]);
        }
        const float inv = 1.f / wt;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= inv;
      }
      cuv_put_row(ot, trow[0], lane, o);
      if (lse_out != nullptr && lane == 0) lse_out[(int64_t)(b0 + trow[0]) * H + h] = mt + __logf(wt);
    }
  }
}

template <int NH>
__global__ __launch_bounds__(kCuvWaves * 64) void combine_up_v_bf16_kernel(
    const u16* __restrict__ o_part, const float* __restrict__ lse_part, int num_splits,
    const u16* __restrict__ w_uv, int B, int H, int DV, float* __restrict__ out, float* __restrict__ lse_out) {
  using M = Mma<u16>;
  constexpr int R = 512, WROW = R * 2, DB = 32 * NH;
  __shared__ __attribute__((aligned(16))) char wt[DB * WROW];             // weight rows d0 .. d0+DB-1
  __shared__ __attribute__((aligned(16))) char ot[kCuvRows * 2 * WROW];   // merged rows (hi | lo)
  __shared__ float xs[kCuvWaves][64][8];                                   // unit sums of shared sequences
  __shared__ float xm[kCuvWaves], xw[kCuvWaves];                           // their maxima and weight sums
  static_assert(kCuvWaves * 4 * 64 * 16 <= kCuvRows * 2 * WROW, "the reduction fits in the merged rows' bytes");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int nblk = DV / DB;
  int h, d0;
  {
    const int bid = (int)blockIdx.x;
    const int grp = bid / (kXcds * nblk);
    const int rem = bid - grp * (kXcds * nblk);
    h = grp * kXcds + rem % kXcds;
    d0 = (rem / kXcds) * DB;
  }
  if (h >= H) return;
  // weight row n (1 KB) into LDS: chunk l of the row at slot l ^ (n & 15)
  {
    const char* wbase = (const char*)(w_uv + ((int64_t)h * DV + d0) * R);
#pragma unroll
    for (int i = 0; i < DB / kCuvWaves; ++i) {
      const int n = wave + kCuvWaves * i;
      __builtin_amdgcn_global_load_lds(wbase + (int64_t)n * WROW + 16 * (lane ^ (n & 15)),
                                       (LDS_AS char*)wt + n * WROW, 16, 0, 0);
    }
  }
  float* lse_w = d0 == 0 ? lse_out : nullptr;
  const int dh = wave >> 2, jq = wave & 3;
  for (int b0 = 0; b0 < B; b0 += kCuvRows) {
    const int nb = min(kCuvRows, B - b0);
    // waves per sequence: the largest power of two with nb * WPR <= 8 (1 from 5 rows up)
    const int WPR = nb >= 5 ? 1 : (nb >= 3 ? 2 : (nb == 2 ? 4 : 8));
    const int upw = (nb * WPR + kCuvWaves - 1) / kCuvWaves;
    if (upw == 1) {
      cuv_merge<1, 32>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_w);
    } else if (upw == 2) {
      cuv_merge<2, 16>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_w);
    } else {
      cuv_merge<4, 8>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_w);
    }
    __syncthreads();  // merged rows written (and, the first time, the weight DMA landed)
    f32x16 acc = zero16();
    if (dh < NH) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ch = 16 * jq + 2 * u + hf;  // 16-byte chunk: k = 128*jq + 16*u + 8*hf .. +7
        const int sl = 16 * (ch ^ (l32 & 15));
        const i16x8 a = *(const LDS_AS i16x8*)((LDS_AS char*)wt + (32 * dh + l32) * WROW + sl);
        const i16x8 bh = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + sl);
        const i16x8 bl = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + WROW + sl);
        acc = M::mma(a, bh, acc);
        acc = M::mma(a, bl, acc);
      }
    }
    __syncthreads();  // every wave has read the merged rows: their bytes take the partial tiles
    LDS_AS f32x4* red = (LDS_AS f32x4*)(LDS_AS char*)ot;  // [wave][row quarter][lane]
    if (dh < NH) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        red[(wave * 4 + q) * 64 + lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
    __syncthreads();
    if (dh < NH && l32 < nb) {
      const int q = wave & 3;  // rows 8q + 4hf .. +3 of the 32-row half dh
      const f32x4 sum = red[((4 * dh + 0) * 4 + q) * 64 + lane] + red[((4 * dh + 1) * 4 + q) * 64 + lane] +
                        red[((4 * dh + 2) * 4 + q) * 64 + lane] + red[((4 * dh + 3) * 4 + q) * 64 + lane];
      *(f32x4*)(out + ((int64_t)(b0 + l32) * H + h) * DV + d0 + 32 * dh + 8 * q + 4 * hf) = sum;
    }
    __syncthreads();  // the next chunk rewrites these bytes
  }
}

// d_v = 128 (the DeepSeek-V2 shape): one work-group per (head, half of the
// sequences), so that each partial row is merged once; the head's W_UV (128
// rows x 512, 128 KB) is held in registers over the 8 waves (wave w: rows
// 32*(w%4) .. +31, latent half w/4: 16 k-steps, 64 VGPRs), read straight from
// global memory (the two work-groups of a head run on one XCD, whose L2
// serves the second).  The two latent halves are added through LDS.  The
// merge keeps 16 partial rows in flight per lane here (the weights take the
// registers of the other 16).
__global__ __launch_bounds__(kCuvWaves * 64) void combine_up_v_bf16_d128_kernel(
    const u16* __restrict__ o_part, const float* __restrict__ lse_part, int num_splits,
    const u16* __restrict__ w_uv, int B, int H, float* __restrict__ out, float* __restrict__ lse_out) {
  using M = Mma<u16>;
  constexpr int R = 512, DV = 128, WROW = R * 2;
  __shared__ __attribute__((aligned(16))) char ot[kCuvRows * 2 * WROW];  // merged rows (hi | lo)
  __shared__ float xs[kCuvWaves][64][8];
  __shared__ float xm[kCuvWaves], xw[kCuvWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  int h, part;
  {
    const int bid = (int)blockIdx.x;
    const int grp = bid / (kXcds * 2);
    const int rem = bid - grp * (kXcds * 2);
    h = grp * kXcds + rem % kXcds;
    part = rem / kXcds;
  }
  if (h >= H) return;
  const int half = (B + 1) / 2;
  const int b_lo = part * half, b_hi = min(B, b_lo + half);
  const int db = wave & 3, jh = wave >> 2;
  i16x8 a[16];
  {
    const u16* wrow = w_uv + ((int64_t)h * DV + 32 * db + l32) * R + 256 * jh + 8 * hf;
#pragma unroll
    for (int u = 0; u < 16; ++u) a[u] = *(const i16x8*)(wrow + 16 * u);
  }
  for (int b0 = b_lo; b0 < b_hi; b0 += kCuvRows) {
    const int nb = min(kCuvRows, b_hi - b0);
    // waves per sequence: the largest power of two with nb * WPR <= 8 (1 from 5 rows up)
    const int WPR = nb >= 5 ? 1 : (nb >= 3 ? 2 : (nb == 2 ? 4 : 8));
    const int upw = (nb * WPR + kCuvWaves - 1) / kCuvWaves;
    if (upw == 1) {
      cuv_merge<1, 16>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_out);
    } else if (upw == 2) {
      cuv_merge<2, 8>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_out);
    } else {
      cuv_merge<4, 4>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_out);
    }
    __syncthreads();  // merged rows written
    f32x16 acc = zero16();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int ch = 32 * jh + 2 * u + hf;  // 16-byte chunk: k = 256*jh + 16*u + 8*hf .. +7
      const int sl = 16 * (ch ^ (l32 & 15));
      const i16x8 bh = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + sl);
      const i16x8 bl = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + WROW + sl);
      acc = M::mma(a[u], bh, acc);
      acc = M::mma(a[u], bl, acc);
    }
    __syncthreads();  // every wave has read the merged rows: their bytes take the partial tiles
    LDS_AS f32x4* red = (LDS_AS f32x4*)(LDS_AS char*)ot;  // [wave][row quarter][lane]
#pragma unroll
    for (int q = 0; q < 4; ++q)
      red[(wave * 4 + q) * 64 + lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    __syncthreads();
    if (l32 < nb) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = 2 * jh + qq;  // wave w adds rows 8q + 4hf .. +3 of block db over the two latent halves
        const f32x4 sum = red[(db * 4 + q) * 64 + lane] + red[((db + 4) * 4 + q) * 64 + lane];
        *(f32x4*)(out + ((int64_t)(b0 + l32) * H + h) * DV + 32 * db + 8 * q + 4 * hf) = sum;
      }
    }
    __syncthreads();  // the next chunk rewrites these bytes
  }
}

// The d_v = 128 merge with 16 waves (more than 16 sequences per work-group):
// two sequences per wave and chunk with 4 split rows each in flight (with 16
// waves that is 128 KB per work-group, more than the latency needs).  The
// head's W_UV is read into registers at the start, so that its 128 KB stream
// in with the partial rows: wave w holds rows 32*(w % 4) .. +31 over latent
// quarter w / 4 (8 fragments, the registers that the halved batch of rows
// leaves free), and the four quarters are added through LDS.
constexpr int kCuvWaves16 = 16;

__global__ __launch_bounds__(kCuvWaves16 * 64) void combine_up_v_bf16_d128_w16_kernel(
    const u16* __restrict__ o_part, const float* __restrict__ lse_part, int num_splits,
    const u16* __restrict__ w_uv, int B, int H, float* __restrict__ out, float* __restrict__ lse_out) {
  using M = Mma<u16>;
  constexpr int R = 512, DV = 128, WROW = R * 2, NWV = kCuvWaves16;
  __shared__ __attribute__((aligned(16))) char ot[kCuvRows * 2 * WROW];  // merged rows (hi | lo)
  __shared__ float xs[NWV][64][8];
  __shared__ float xm[NWV], xw[NWV];
  static_assert(NWV * 4 * 64 * 16 <= kCuvRows * 2 * WROW, "the quarter sums fit the merged rows' bytes");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  int h, part;
  {
    const int bid = (int)blockIdx.x;
    const int grp = bid / (kXcds * 2);
    const int rem = bid - grp * (kXcds * 2);
    h = grp * kXcds + rem % kXcds;
    part = rem / kXcds;
  }
  if (h >= H) return;
  const int half = (B + 1) / 2;
  const int b_lo = part * half, b_hi = min(B, b_lo + half);
  const int db = wave & 3, jq = wave >> 2;
  // this wave's quarter of the head's W_UV (8 fragments), loaded once, first
  const u16* wrow = w_uv + ((int64_t)h * DV + 32 * db + l32) * R + 128 * jq + 8 * hf;
  i16x8 a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = *(const i16x8*)(wrow + 16 * u);
  for (int b0 = b_lo; b0 < b_hi; b0 += kCuvRows) {
    const int nb = min(kCuvRows, b_hi - b0);
    // waves per sequence: the largest power of two with nb * WPR <= 16 (1 from 9 rows up)
    const int WPR = nb >= 9 ? 1 : (nb >= 5 ? 2 : (nb >= 3 ? 4 : (nb == 2 ? 8 : 16)));
    if (nb * WPR > NWV) {
      cuv_merge<2, 4, NWV>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_out);
    } else {
      cuv_merge<1, 8, NWV>(o_part, lse_part, num_splits, H, h, b0, nb, WPR, wave, lane, ot, xs, xm, xw, lse_out);
    }
    __syncthreads();  // merged rows written
    f32x16 acc = zero16();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ch = 16 * jq + 2 * u + hf;  // 16-byte chunk: k = 128*jq + 16*u + 8*hf .. +7
      const int sl = 16 * (ch ^ (l32 & 15));
      const i16x8 bh = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + sl);
      const i16x8 bl = *(const LDS_AS i16x8*)((LDS_AS char*)ot + l32 * 2 * WROW + WROW + sl);
      acc = M::mma(a[u], bh, acc);
      acc = M::mma(a[u], bl, acc);
    }
    __syncthreads();  // every wave has read the merged rows: their bytes take the quarter sums
    LDS_AS f32x4* red = (LDS_AS f32x4*)(LDS_AS char*)ot;  // [wave][row quarter][lane]
#pragma unroll
    for (int q = 0; q < 4; ++q)
      red[(wave * 4 + q) * 64 + lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    __syncthreads();
    if (l32 < nb) {
      // wave w adds rows 8q + 4hf .. +3 of block db (q = w / 4) over the four latent quarters
      const int q = jq;
      const f32x4 sum = ((red[(db * 4 + q) * 64 + lane] + red[((db + 4) * 4 + q) * 64 + lane]) +
                         red[((db + 8) * 4 + q) * 64 + lane]) + red[((db + 12) * 4 + q) * 64 + lane];
      *(f32x4*)(out + ((int64_t)(b0 + l32) * H + h) * DV + 32 * db + 8 * q + 4 * hf) = sum;
    }
    __syncthreads();  // the next chunk rewrites these bytes
  }
}

__global__ __launch_bounds__(64) void combine_up_v_f32_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ lse_part, int S,
                                                              const float* __restrict__ w_uv, int H, int DV, int R,
                                                              float* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float orow[kCuvMaxRankF32];
  const int lane = threadIdx.x & 63;
  const int b = (int)blockIdx.x / H, h = (int)blockIdx.x - b * H;
  const int64_t base = (int64_t)b * S * H + h;
  float mx, wsum;
  lse_stats(lse_part + base, S, H, lane, mx, wsum);
  const float sc = 1.f / wsum;
  for (int c = lane; c < R; c += 64) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float l = lse_part[base + (int64_t)s * H];
      if (l == -INFINITY) continue;  // an empty split never wrote its partial
      acc = fmaf(__expf(l - mx) * sc, o_part[(base + (int64_t)s * H) * R + c], acc);
    }
    orow[c] = acc;
  }
  __syncthreads();
  for (int d = lane; d < DV; d += 64) {
    const float* wr = w_uv + ((int64_t)h * DV + d) * R;
    float acc = 0.f;
    for (int j = 0; j < R; ++j) acc = fmaf(wr[j], orow[j], acc);
    out[((int64_t)b * H + h) * DV + d] = acc;
  }
  if (lse_out != nullptr && lane == 0) lse_out[(int64_t)b * H + h] = mx + __logf(wsum);
}

// ---------------------------------------------------------------------------
// Latent KV production from the hidden state (the step before the path):
// x = W_DKV h, c_kv_new = norm_w * x / sqrt(mean(x^2) + eps), k_rope_new =
// W_KR h, for the R + DR = 576 output features of each sequence.  bf16.
// Pass 1: one work-group per (32 features, 512 of the d_model inputs); wave
// w takes 128 of the inputs (8 k-steps of the 32x32x16 MFMA, A = weight rows,
// B = hidden-state rows, both straight from global memory, all loads issued
// before the first MFMA), the four waves are summed through LDS, and the fp32
// partial goes to the workspace [chunk][B][576].  Pass 2: one work-group per
// sequence; a thread sums its features' chunks in order (deterministic, eight
// loads in flight per feature), the sum of squares of the first R features
// goes through LDS, and each output is rounded once after the RMSNorm.
// ---------------------------------------------------------------------------

constexpr int kKvChunk = 512;  // d_model inputs per pass-1 work-group

__global__ __launch_bounds__(256) void kv_down_partial_kernel(const u16* __restrict__ h, const u16* __restrict__ w_dkv,
                                                              const u16* __restrict__ w_kr, int B, int DM, int R,
                                                              int DR, float* __restrict__ part) {
  using M = Mma<u16>;
  const int NF = R + DR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int nfb = (NF + 31) / 32;
  const int fb = (int)blockIdx.x % nfb, kc = (int)blockIdx.x / nfb;
  const int f = fb * 32 + l32;  // this lane's A row (output feature)
  const u16* wrow = f < R ? w_dkv + (int64_t)f * DM : w_kr + (int64_t)(min(f, NF - 1) - R) * DM;
  const int kbase = kc * kKvChunk + wave * (kKvChunk / 4) + 8 * hf;
  __shared__ f32x4 red[4][4][64];
  i16x8 a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = *(const i16x8*)(wrow + kbase + 16 * u);
  for (int b0 = 0; b0 < B; b0 += 32) {
    const int bb = min(b0 + l32, B - 1);  // rows past B compute garbage columns that are not stored
    i16x8 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *(const i16x8*)(h + (int64_t)bb * DM + kbase + 16 * u);
    f32x16 acc = zero16();
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = M::mma(a[u], x[u], acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    __syncthreads();
    // wave w sums the four k-quarters of feature rows 8w + 4hf .. +3
    const f32x4 sum = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
    const int ff = fb * 32 + 8 * wave + 4 * hf;
    if (b0 + l32 < B && ff < NF) *(f32x4*)(part + ((int64_t)kc * B + b0 + l32) * NF + ff) = sum;
    __syncthreads();  // red is rewritten for the next batch block
  }
}

__global__ __launch_bounds__(256) void kv_down_final_kernel(const float* __restrict__ part, int nchunks, int B, int R,
                                                            int DR, const u16* __restrict__ norm_w, float eps,
                                                            u16* __restrict__ c_kv_new, u16* __restrict__ k_rope_new) {
  constexpr int FPT = 4, CG = 8;  // features per thread (R + DR <= 1024), chunk loads in flight per feature
  const int NF = R + DR;
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = (int)blockIdx.x;
  __shared__ float wss[4];
  float v[FPT] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nchunks; c0 += CG) {
    float x[FPT][CG];
#pragma unroll
    for (int j = 0; j < FPT; ++j)
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const int f = min(tid + 256 * j, NF - 1), c = min(c0 + u, nchunks - 1);
        x[j][u] = part[((int64_t)c * B + b) * NF + f];
      }
#pragma unroll
    for (int j = 0; j < FPT; ++j)
#pragma unroll
      for (int u = 0; u < CG; ++u)
        if (c0 + u < nchunks) v[j] += x[j][u];  // chunks in order
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < FPT; ++j)
    if (tid + 256 * j < R) ss = fmaf(v[j], v[j], ss);
  ss = wave_sum_f(ss);
  if (lane == 0) wss[wave] = ss;
  __syncthreads();
  const float inv = 1.f / sqrtf((wss[0] + wss[1] + wss[2] + wss[3]) / (float)R + eps);
#pragma unroll
  for (int j = 0; j < FPT; ++j) {
    const int f = tid + 256 * j;
    if (f < R) c_kv_new[(int64_t)b * R + f] = f2bf(v[j] * inv * bf2f(norm_w[f]));
    else if (f < NF) k_rope_new[(int64_t)b * DR + (f - R)] = f2bf(v[j]);
  }
}

// ---------------------------------------------------------------------------
// K2: RoPE on q_rope and on the new token's shared key; append the new row.
// One work-group per (sequence, block of HB heads: 16 in this kernel); the
// work-group of head block 0 also writes the cache row.  Pair frequencies come from the host (in
// double); each angle pos * theta_i is reduced modulo 2*pi in double (two-
// part constant) before sincos, and rotations and the final rounding are done
// in double precision.
// ---------------------------------------------------------------------------

template <typename T, int NT, int HB>
__device__ __forceinline__ void rope_block(int blk, const T* __restrict__ q_rope, const T* __restrict__ c_kv_new,
                                           const T* __restrict__ k_rope_new, const int32_t* __restrict__ positions,
                                           const CacheMap& cm, int H, int R,
                                           int DR, const RopeFreqs& freqs, T* __restrict__ q_lat,
                                           T* __restrict__ cache, double* cs /* LDS, 2 * kMaxRopePairs */) {
  constexpr int QP = HB * kMaxRopePairs / NT;  // q_rope pairs per thread (HB heads x d_rope/2)
  constexpr int CV = 1024 / NT;                // c_kv_new values per thread (R <= 1024)
  typedef T T2 __attribute__((ext_vector_type(2)));
  const int hblocks = (H + HB - 1) / HB;
  const int b = blk / hblocks;
  const int hb = blk - b * hblocks;
  const int half = DR / 2;
  const int W = R + DR;
  const int h0 = hb * HB, h1 = min(H, h0 + HB);
  const int npairs = (h1 - h0) * half;
  const int tid = (int)threadIdx.x;
  const bool row_block = hb == 0;
  // Every global load is issued up front, unconditionally (indices clamped
  // into range), so that they all share one round trip: the position, this
  // thread's angle frequency, q_rope pairs, and (used by the work-group of
  // head block 0 only) the new key pair, c_kv_new values and the row offset.
  const int pos = positions[b];
  const int ti = min(tid, half - 1);
  const double theta = freqs.theta[ti];
  T2 qx[QP];
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int idx = tid + u * NT;
    const int hh = h0 + idx / half, i = idx % half;
    qx[u] = *(const T2*)(q_rope + ((int64_t)b * H + (idx < npairs ? hh : h0)) * DR + 2 * i);
  }
  const T2 kx = *(const T2*)(k_rope_new + (int64_t)b * DR + 2 * ti);
  T cv[CV];
#pragma unroll
  for (int u = 0; u < CV; ++u) cv[u] = c_kv_new[(int64_t)b * R + min(tid + u * NT, R - 1)];
  const int64_t row_off = cm.block_table == nullptr ? cm.row_offsets[b] : 0;  // (paged: looked up below)

  if (tid < half) sincos_reduced((double)pos * theta, &cs[kMaxRopePairs + tid], &cs[tid]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int idx = tid + u * NT;
    if (idx >= npairs) break;
    const int hh = h0 + idx / half, i = idx % half;
    const double x0 = load_d<T>(qx[u][0]), x1 = load_d<T>(qx[u][1]);
    const double c = cs[i], s = cs[kMaxRopePairs + i];
    *(T2*)(q_lat + ((int64_t)b * H + hh) * W + R + 2 * i) = T2{store_d<T>(x0 * c - x1 * s), store_d<T>(x0 * s + x1 * c)};
  }
  if (!row_block) return;
  T* crow = cache + cm.row(b, pos, row_off) * W;
#pragma unroll
  for (int u = 0; u < CV; ++u) {
    const int k = tid + u * NT;
    if (k < R) crow[k] = cv[u];
  }
  if (tid < half) {
    const double x0 = load_d<T>(kx[0]), x1 = load_d<T>(kx[1]);
    const double c = cs[tid], s = cs[kMaxRopePairs + tid];
    *(T2*)(crow + R + 2 * tid) = T2{store_d<T>(x0 * c - x1 * s), store_d<T>(x0 * s + x1 * c)};
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(const T* __restrict__ q_rope, const T* __restrict__ c_kv_new,
                                                          const T* __restrict__ k_rope_new,
                                                          const int32_t* __restrict__ positions, CacheMap cm,
                                                          int H, int R, int DR, RopeFreqs freqs,
                                                          T* __restrict__ q_lat, T* __restrict__ cache) {
  __shared__ double cs[2 * kMaxRopePairs];
  rope_block<T, 256, 16>((int)blockIdx.x, q_rope, c_kv_new, k_rope_new, positions, cm, H, R, DR, freqs, q_lat,
                         cache, cs);
}

// K1 + K2 in one bf16 launch: the absorption blocks also do the RoPE work
// (see absorb_bf16_block); q~ and the rotated RoPE part are disjoint columns
// of q_lat.
template <int DH, bool PAGED>
__global__ __launch_bounds__(256) void absorb_rope_bf16_kernel(const u16* __restrict__ q_nope,
                                                               const u16* __restrict__ w_uk, int B, int H, int R,
                                                               RopeArgs ra, RopeFreqs freqs, u16* __restrict__ q_lat) {
  __shared__ __attribute__((aligned(1024))) char wt[AbsorbLds<DH>::WT];
  __shared__ __attribute__((aligned(1024))) char qs[AbsorbLds<DH>::QS];
  // Every kernel argument the block uses, fetched in one batch at entry: left
  // to itself the compiler loads them in dependent rounds, one between each
  // of the branches below, before the first copy is issued.
  asm volatile("" ::"s"(q_nope), "s"(w_uk), "s"(B), "s"(H), "s"(q_lat), "s"(ra.q_rope), "s"(ra.c_kv_new),
               "s"(ra.k_rope_new), "s"(ra.positions), "s"(ra.cm.row_offsets), "s"(ra.cm.block_table),
               "s"(ra.cm.total_rows), "s"(ra.cm.total_pages), "s"(ra.cm.bt_stride), "s"(ra.cm.page_shift),
               "s"(ra.cache), "s"(ra.cache8), "s"(ra.scale8));
  (void)R;  // kAbsorbR (checked by the launcher)
  absorb_bf16_block<DH, true, PAGED>((int)blockIdx.x, q_nope, w_uk, B, H, q_lat, kAbsorbR + kAbsorbDR, wt, qs, ra,
                                     freqs);
}

// ---------------------------------------------------------------------------
// Host side: validation, dispatch, launch
// ---------------------------------------------------------------------------

thread_local std::string g_last_error;

mla_status fail(mla_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

enum Inst { kInstNone = -1, kF32H8R64D16 = 0, kF32H16R64D32 = 1, kBf16H128R512D64 = 2 };

int find_inst(const mla_dims& d) {
  if (d.dtype == MLA_F32 && d.heads == 8 && d.rank == 64 && d.d_rope == 16) return kF32H8R64D16;
  if (d.dtype == MLA_F32 && d.heads == 16 && d.rank == 64 && d.d_rope == 32) return kF32H16R64D32;
  if (d.dtype == MLA_BF16 && d.heads == 128 && d.rank == 512 && d.d_rope == 64) return kBf16H128R512D64;
  return kInstNone;
}

mla_status check_dims_impl(const mla_dims* d) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->heads < 1 || d->d_head < 1 || d->d_v < 1 || d->rank < 1 || d->d_rope < 1)
    return fail(MLA_ERR_INVALID_ARG, "every dimension must be >= 1");
  if (d->d_rope % 2 != 0) return fail(MLA_ERR_INVALID_ARG, "d_rope must be even (RoPE rotates pairs)");
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return fail(MLA_ERR_INVALID_ARG, "dtype must be MLA_F32 or MLA_BF16");
  if (d->batch > (1 << 20)) return fail(MLA_ERR_UNSUPPORTED, "batch above 2^20");
  if (find_inst(*d) == kInstNone)
    return fail(MLA_ERR_UNSUPPORTED,
                "no kernel for (dtype, heads, rank, d_rope); supported: (F32,8,64,16) (F32,16,64,32) (BF16,128,512,64)");
  if (d->d_head != 32 && d->d_head != 64 && d->d_head != 128 && d->d_head != 256)
    return fail(MLA_ERR_UNSUPPORTED, "d_head must be 32, 64, 128 or 256");
  if (d->d_v % 32 != 0 || d->d_v > 1024) return fail(MLA_ERR_UNSUPPORTED, "d_v must be a multiple of 32, at most 1024");
  return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

mla_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (p == nullptr) return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (!aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  }
  return MLA_OK;
}

mla_status launch_result(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MLA_OK;
}

float scale_of(const mla_dims& d) {
  return d.softmax_scale > 0.f ? d.softmax_scale : (float)(1.0 / std::sqrt((double)(d.d_head + d.d_rope)));
}

int32_t chunk_rows(int32_t max_seq_len, int32_t num_splits) {
  const int64_t c = ((int64_t)max_seq_len + num_splits - 1) / num_splits;
  return (int32_t)(((c + 31) / 32) * 32);
}

constexpr int kMaxSplits = 4096;

template <typename T, int H, int R, int DR, int NW>
mla_status launch_decode(const mla_dims& d, const void* q_lat, const void* cache, const CacheMap& cm,
                         const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, void* o_part,
                         float* lse_part, hipStream_t stream) {
  using S = DecodeShape<T, H, R, DR, NW>;
  const int64_t items = (int64_t)d.batch * num_splits * S::GROUPS;
  const int64_t blocks = (items + kXcds - 1) / kXcds * kXcds;  // padded to whole rounds over the XCDs
  if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  const float scale_log2 = scale_of(d) * kLog2e;
  if (cm.block_table != nullptr) {
    hipLaunchKernelGGL((decode_latent_kernel<T, H, R, DR, NW, true>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       stream, (const T*)q_lat, (const T*)cache, cm, cm.block_table, seq_lens, d.batch, num_splits,
                       chunk_rows(max_seq_len, num_splits), (T*)o_part, lse_part, scale_log2);
    return launch_result("mla_decode_latent_paged");
  }
  hipLaunchKernelGGL((decode_latent_kernel<T, H, R, DR, NW, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                     (const T*)q_lat, (const T*)cache, cm, nullptr, seq_lens, d.batch, num_splits,
                     chunk_rows(max_seq_len, num_splits), (T*)o_part, lse_part, scale_log2);
  return launch_result("mla_decode_latent");
}

template <typename T, int NW, int DH>
mla_status launch_absorb(const mla_dims& d, const void* q_nope, const void* w_uk, void* q_lat, hipStream_t stream) {
  if (d.rank % (32 * NW) != 0) return fail(MLA_ERR_UNSUPPORTED, "rank must be a multiple of the column block");
  const int blocks = (d.heads + kXcds - 1) / kXcds * kXcds * (d.rank / (32 * NW));  // whole groups of 8 heads
  hipLaunchKernelGGL((absorb_q_kernel<T, NW, DH>), dim3(blocks), dim3(NW * 64), 0, stream, (const T*)q_nope,
                     (const T*)w_uk, d.batch, d.heads, d.rank, (T*)q_lat, d.rank + d.d_rope);
  return launch_result("mla_absorb_q");
}

template <int DH>
mla_status launch_absorb_bf16(const mla_dims& d, const void* q_nope, const void* w_uk, void* q_lat,
                              hipStream_t stream) {
  if (d.rank != kAbsorbR || d.d_rope != kAbsorbDR) return fail(MLA_ERR_UNSUPPORTED, "bf16 needs rank 512, d_rope 64");
  const int blocks = (d.heads + kXcds - 1) / kXcds * kXcds * (d.rank / 64);  // whole groups of 8 heads
  hipLaunchKernelGGL((absorb_q_bf16_kernel<DH>), dim3(blocks), dim3(128), 0, stream, (const u16*)q_nope,
                     (const u16*)w_uk, d.batch, d.heads, d.rank, (u16*)q_lat, d.rank + d.d_rope);
  return launch_result("mla_absorb_q");
}

template <int DH>
mla_status launch_absorb_rope_bf16(const mla_dims& d, const void* q_nope, const void* w_uk, const void* q_rope,
                                   const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                                   const CacheMap& cm, const RopeFreqs& freqs, void* q_lat, void* kv_cache,
                                   hipStream_t stream, uint8_t* cache8 = nullptr, float* scale8 = nullptr) {
  if (d.rank != kAbsorbR || d.d_rope != kAbsorbDR) return fail(MLA_ERR_UNSUPPORTED, "bf16 needs rank 512, d_rope 64");
  const int blocks = (d.heads + kXcds - 1) / kXcds * kXcds * (d.rank / 64);  // whole groups of 8 heads
  const RopeArgs ra{(const u16*)q_rope, (const u16*)c_kv_new, (const u16*)k_rope_new, positions, cm, d.d_rope,
                    (u16*)kv_cache, cache8, scale8};
  if (cm.block_table != nullptr) {
    hipLaunchKernelGGL((absorb_rope_bf16_kernel<DH, true>), dim3(blocks), dim3(256), 0, stream, (const u16*)q_nope,
                       (const u16*)w_uk, d.batch, d.heads, d.rank, ra, freqs, (u16*)q_lat);
    return launch_result("mla_absorb_rope_paged");
  }
  hipLaunchKernelGGL((absorb_rope_bf16_kernel<DH, false>), dim3(blocks), dim3(256), 0, stream, (const u16*)q_nope,
                     (const u16*)w_uk, d.batch, d.heads, d.rank, ra, freqs, (u16*)q_lat);
  return launch_result("mla_absorb_rope");
}

template <typename T, int NW>
mla_status launch_absorb_dh(const mla_dims& d, const void* q_nope, const void* w_uk, void* q_lat, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    switch (d.d_head) {
      case 32: return launch_absorb_bf16<32>(d, q_nope, w_uk, q_lat, stream);
      case 64: return launch_absorb_bf16<64>(d, q_nope, w_uk, q_lat, stream);
      case 128: return launch_absorb_bf16<128>(d, q_nope, w_uk, q_lat, stream);
      case 256: return launch_absorb_bf16<256>(d, q_nope, w_uk, q_lat, stream);
      default: return fail(MLA_ERR_UNSUPPORTED, "d_head");
    }
  } else {
    switch (d.d_head) {
      case 32: return launch_absorb<T, NW, 32>(d, q_nope, w_uk, q_lat, stream);
      case 64: return launch_absorb<T, NW, 64>(d, q_nope, w_uk, q_lat, stream);
      case 128: return launch_absorb<T, NW, 128>(d, q_nope, w_uk, q_lat, stream);
      case 256: return launch_absorb<T, NW, 256>(d, q_nope, w_uk, q_lat, stream);
      default: return fail(MLA_ERR_UNSUPPORTED, "d_head");
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

mla_status mla_check_dims(const mla_dims* dims) { return check_dims_impl(dims); }

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, void* q_lat, void* stream) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({q_nope, w_uk, q_lat})) != MLA_OK) return st;
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  switch (find_inst(*dims)) {
    case kF32H8R64D16:
    case kF32H16R64D32: return launch_absorb_dh<float, 1>(*dims, q_nope, w_uk, q_lat, s);
    case kBf16H128R512D64: return launch_absorb_dh<u16, 2>(*dims, q_nope, w_uk, q_lat, s);
  }
  return fail(MLA_ERR_UNSUPPORTED, "no instantiation");
}

}  // extern "C"

namespace {

// A paged cache description: block table, pages of page_rows (a power of two
// from 32 to 65536) rows, total_pages pages.
mla_status paged_map(const int32_t* block_table, int32_t bt_stride, int32_t page_rows, int64_t total_pages,
                     CacheMap* cm) {
  if (block_table == nullptr) return fail(MLA_ERR_INVALID_ARG, "block_table NULL");
  if (bt_stride < 1) return fail(MLA_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (page_rows < 32 || page_rows > 65536 || (page_rows & (page_rows - 1)) != 0)
    return fail(MLA_ERR_INVALID_ARG, "page_rows must be a power of two from 32 to 65536");
  if (total_pages < 1 || total_pages > ((int64_t)1 << 40)) return fail(MLA_ERR_INVALID_ARG, "total_pages out of range");
  int shift = 0;
  while ((1 << shift) < page_rows) ++shift;
  *cm = CacheMap{nullptr, block_table, total_pages * page_rows, total_pages, bt_stride, shift};
  return MLA_OK;
}

mla_status check_rope_args(const mla_dims* dims, const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                           const int32_t* positions, void* q_lat, void* kv_cache) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if (positions == nullptr) return fail(MLA_ERR_INVALID_ARG, "positions NULL");
  if ((st = check_ptrs({q_rope, c_kv_new, k_rope_new, q_lat, kv_cache})) != MLA_OK) return st;
  if (dims->d_rope > 2 * kMaxRopePairs) return fail(MLA_ERR_UNSUPPORTED, "d_rope above 64");  // 16 heads x d_rope/2 pairs per block
  if (dims->rank > 1024) return fail(MLA_ERR_UNSUPPORTED, "rank above 1024");  // c_kv_new values per thread
  return MLA_OK;
}

mla_status packed_map(const int64_t* row_offsets, int64_t total_rows, CacheMap* cm) {
  if (row_offsets == nullptr) return fail(MLA_ERR_INVALID_ARG, "row_offsets NULL");
  if (total_rows < 1) return fail(MLA_ERR_INVALID_ARG, "total_rows must be >= 1");
  *cm = CacheMap{row_offsets, nullptr, total_rows, 0, 0, 0};
  return MLA_OK;
}

RopeFreqs rope_freqs(const mla_dims* dims) {
  const double base = dims->rope_base > 0.f ? (double)dims->rope_base : 10000.0;
  RopeFreqs freqs;
  for (int i = 0; i < dims->d_rope / 2; ++i) freqs.theta[i] = std::pow(base, -2.0 * (double)i / (double)dims->d_rope);
  return freqs;
}

mla_status rope_append_impl(const mla_dims* dims, const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                            const int32_t* positions, const CacheMap& cm, void* q_lat, void* kv_cache,
                            void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const RopeFreqs freqs = rope_freqs(dims);
  const int blocks = dims->batch * ((dims->heads + 15) / 16);
  if (dims->dtype == MLA_BF16) {
    hipLaunchKernelGGL((rope_append_kernel<u16>), dim3(blocks), dim3(256), 0, s, (const u16*)q_rope,
                       (const u16*)c_kv_new, (const u16*)k_rope_new, positions, cm, dims->heads, dims->rank,
                       dims->d_rope, freqs, (u16*)q_lat, (u16*)kv_cache);
  } else {
    hipLaunchKernelGGL((rope_append_kernel<float>), dim3(blocks), dim3(256), 0, s, (const float*)q_rope,
                       (const float*)c_kv_new, (const float*)k_rope_new, positions, cm, dims->heads, dims->rank,
                       dims->d_rope, freqs, (float*)q_lat, (float*)kv_cache);
  }
  return launch_result(cm.block_table != nullptr ? "mla_rope_append_paged" : "mla_rope_append");
}

mla_status absorb_rope_impl(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                            const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                            const CacheMap& cm, void* q_lat, void* kv_cache, void* stream) {
  mla_status st;
  if ((st = check_ptrs({q_nope, w_uk})) != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (find_inst(*dims) != kBf16H128R512D64) {  // fp32: the two launches, in order
    if ((st = mla_absorb_q(dims, q_nope, w_uk, q_lat, stream)) != MLA_OK) return st;
    return rope_append_impl(dims, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache, stream);
  }
  const RopeFreqs freqs = rope_freqs(dims);
  switch (dims->d_head) {
    case 32: return launch_absorb_rope_bf16<32>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                freqs, q_lat, kv_cache, s);
    case 64: return launch_absorb_rope_bf16<64>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                freqs, q_lat, kv_cache, s);
    case 128: return launch_absorb_rope_bf16<128>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                  freqs, q_lat, kv_cache, s);
    case 256: return launch_absorb_rope_bf16<256>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                  freqs, q_lat, kv_cache, s);
  }
  return fail(MLA_ERR_UNSUPPORTED, "d_head");
}

}  // namespace

extern "C" {

mla_status mla_rope_append(const mla_dims* dims, const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                           const int32_t* positions, const int64_t* row_offsets, int64_t total_rows, void* q_lat,
                           void* kv_cache, void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  CacheMap cm;
  if ((st = packed_map(row_offsets, total_rows, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return rope_append_impl(dims, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache, stream);
}

mla_status mla_rope_append_paged(const mla_dims* dims, const void* q_rope, const void* c_kv_new,
                                 const void* k_rope_new, const int32_t* positions, const int32_t* block_table,
                                 int32_t bt_stride, int32_t page_rows, int64_t total_pages, void* q_lat,
                                 void* kv_cache, void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  CacheMap cm;
  if ((st = paged_map(block_table, bt_stride, page_rows, total_pages, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return rope_append_impl(dims, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache, stream);
}

mla_status mla_absorb_rope(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                           const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                           const int64_t* row_offsets, int64_t total_rows, void* q_lat, void* kv_cache,
                           void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  CacheMap cm;
  if ((st = packed_map(row_offsets, total_rows, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return absorb_rope_impl(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache, stream);
}

mla_status mla_absorb_rope_paged(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                                 const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                                 const int32_t* block_table, int32_t bt_stride, int32_t page_rows,
                                 int64_t total_pages, void* q_lat, void* kv_cache, void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  CacheMap cm;
  if ((st = paged_map(block_table, bt_stride, page_rows, total_pages, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return absorb_rope_impl(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache, stream);
}

}  // extern "C"

namespace {

mla_status decode_dispatch(const mla_dims* dims, const void* q_lat, const void* kv_cache, const CacheMap& cm,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, void* o_part,
                           float* lse_part, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (find_inst(*dims)) {
    case kF32H8R64D16:
      return launch_decode<float, 8, 64, 16, 1>(*dims, q_lat, kv_cache, cm, seq_lens, max_seq_len, num_splits,
                                                o_part, lse_part, s);
    case kF32H16R64D32:
      return launch_decode<float, 16, 64, 32, 1>(*dims, q_lat, kv_cache, cm, seq_lens, max_seq_len, num_splits,
                                                 o_part, lse_part, s);
    case kBf16H128R512D64:
      return launch_decode<u16, 128, 512, 64, 4>(*dims, q_lat, kv_cache, cm, seq_lens, max_seq_len, num_splits,
                                                 o_part, lse_part, s);
  }
  return fail(MLA_ERR_UNSUPPORTED, "no instantiation");
}

mla_status check_decode_args(const mla_dims* dims, const void* q_lat, const void* kv_cache, const int32_t* seq_lens,
                             int32_t max_seq_len, int32_t num_splits, void* o_part, float* lse_part) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if (seq_lens == nullptr) return fail(MLA_ERR_INVALID_ARG, "seq_lens NULL");
  if ((st = check_ptrs({q_lat, kv_cache, o_part, lse_part})) != MLA_OK) return st;
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (num_splits < 1) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (num_splits > kMaxSplits) return fail(MLA_ERR_WORKSPACE, "num_splits above 4096");
  return MLA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch memory of the no-allocation entry point: a fixed device array (each
// GPU the library runs on holds its own copy until the process ends).  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address is looked up once per device,
// with that device current, and kept.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

static std::mutex g_scratch_mutex;
static float* g_scratch_ptr[kScratchDevices] = {};

// The current device's copy of `scratch` (looked up on its first use there).
static mla_status scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices) return fail(MLA_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MLA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

extern "C" {

mla_status mla_decode_latent(const mla_dims* dims, const void* q_lat, const void* kv_cache, const int64_t* row_offsets,
                             const int32_t* seq_lens, int64_t total_rows, int32_t max_seq_len, int32_t num_splits,
                             void* o_part, float* lse_part, void* stream) {
  mla_status st = check_decode_args(dims, q_lat, kv_cache, seq_lens, max_seq_len, num_splits, o_part, lse_part);
  if (st != MLA_OK) return st;
  if (row_offsets == nullptr) return fail(MLA_ERR_INVALID_ARG, "row_offsets NULL");
  if (total_rows < 1) return fail(MLA_ERR_INVALID_ARG, "total_rows must be >= 1");
  g_last_error.clear();
  const CacheMap cm{row_offsets, nullptr, total_rows, 0, 0, 0};
  return decode_dispatch(dims, q_lat, kv_cache, cm, seq_lens, max_seq_len, num_splits, o_part, lse_part, stream);
}

mla_status mla_decode_latent_paged(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                   const int32_t* block_table, int32_t bt_stride, int32_t page_rows,
                                   int64_t total_pages, const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t num_splits, void* o_part, float* lse_part, void* stream) {
  mla_status st = check_decode_args(dims, q_lat, kv_cache, seq_lens, max_seq_len, num_splits, o_part, lse_part);
  if (st != MLA_OK) return st;
  CacheMap cm;
  if ((st = paged_map(block_table, bt_stride, page_rows, total_pages, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return decode_dispatch(dims, q_lat, kv_cache, cm, seq_lens, max_seq_len, num_splits, o_part, lse_part, stream);
}

// ---- fp8 latent cache (rows of 512 E4M3 codes + 64 bf16 RoPE values, one
// power-of-two scale per row; the bf16 instance H 128, r 512, d_rope 64)

static mla_status check_fp8_dims(const mla_dims* dims, const float* kv_scale) {
  if (find_inst(*dims) != kBf16H128R512D64)
    return fail(MLA_ERR_UNSUPPORTED, "the fp8 cache is supported for (BF16, heads 128, rank 512, d_rope 64)");
  if (kv_scale == nullptr) return fail(MLA_ERR_INVALID_ARG, "kv_scale NULL");
  if (((uintptr_t)kv_scale & 15u) != 0) return fail(MLA_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  return MLA_OK;
}

static mla_status decode_fp8_impl(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                  const float* kv_scale, const CacheMap& cm, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t num_splits, void* o_part, float* lse_part,
                                  void* stream) {
  const hipError_t e = mla_launch_decode_fp8(q_lat, kv_cache, kv_scale, cm, seq_lens, dims->batch, num_splits,
                                             chunk_rows(max_seq_len, num_splits), o_part, lse_part,
                                             scale_of(*dims) * kLog2e, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  if (e != hipSuccess) return fail(MLA_ERR_HIP, std::string("mla_decode_latent_fp8: ") + hipGetErrorString(e));
  return MLA_OK;
}

mla_status mla_decode_latent_fp8(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                 const float* kv_scale, const int64_t* row_offsets, const int32_t* seq_lens,
                                 int64_t total_rows, int32_t max_seq_len, int32_t num_splits, void* o_part,
                                 float* lse_part, void* stream) {
  mla_status st = check_decode_args(dims, q_lat, kv_cache, seq_lens, max_seq_len, num_splits, o_part, lse_part);
  if (st != MLA_OK) return st;
  if ((st = check_fp8_dims(dims, kv_scale)) != MLA_OK) return st;
  CacheMap cm;
  if ((st = packed_map(row_offsets, total_rows, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return decode_fp8_impl(dims, q_lat, kv_cache, kv_scale, cm, seq_lens, max_seq_len, num_splits, o_part, lse_part,
                         stream);
}

mla_status mla_decode_latent_fp8_paged(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                       const float* kv_scale, const int32_t* block_table, int32_t bt_stride,
                                       int32_t page_rows, int64_t total_pages, const int32_t* seq_lens,
                                       int32_t max_seq_len, int32_t num_splits, void* o_part, float* lse_part,
                                       void* stream) {
  mla_status st = check_decode_args(dims, q_lat, kv_cache, seq_lens, max_seq_len, num_splits, o_part, lse_part);
  if (st != MLA_OK) return st;
  if ((st = check_fp8_dims(dims, kv_scale)) != MLA_OK) return st;
  CacheMap cm;
  if ((st = paged_map(block_table, bt_stride, page_rows, total_pages, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return decode_fp8_impl(dims, q_lat, kv_cache, kv_scale, cm, seq_lens, max_seq_len, num_splits, o_part, lse_part,
                         stream);
}

static mla_status absorb_rope_fp8_impl(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                                       const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                                       const CacheMap& cm, void* q_lat, void* kv_cache, float* kv_scale,
                                       void* stream) {
  mla_status st;
  if ((st = check_ptrs({q_nope, w_uk})) != MLA_OK) return st;
  const RopeFreqs freqs = rope_freqs(dims);
  hipStream_t s = (hipStream_t)stream;
  switch (dims->d_head) {
    case 32: return launch_absorb_rope_bf16<32>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                freqs, q_lat, nullptr, s, (uint8_t*)kv_cache, kv_scale);
    case 64: return launch_absorb_rope_bf16<64>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                freqs, q_lat, nullptr, s, (uint8_t*)kv_cache, kv_scale);
    case 128: return launch_absorb_rope_bf16<128>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                  freqs, q_lat, nullptr, s, (uint8_t*)kv_cache, kv_scale);
    case 256: return launch_absorb_rope_bf16<256>(*dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm,
                                                  freqs, q_lat, nullptr, s, (uint8_t*)kv_cache, kv_scale);
  }
  return fail(MLA_ERR_UNSUPPORTED, "d_head");
}

mla_status mla_absorb_rope_fp8(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                               const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                               const int64_t* row_offsets, int64_t total_rows, void* q_lat, void* kv_cache,
                               float* kv_scale, void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  if ((st = check_fp8_dims(dims, kv_scale)) != MLA_OK) return st;
  CacheMap cm;
  if ((st = packed_map(row_offsets, total_rows, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return absorb_rope_fp8_impl(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache,
                              kv_scale, stream);
}

mla_status mla_absorb_rope_fp8_paged(const mla_dims* dims, const void* q_nope, const void* w_uk, const void* q_rope,
                                     const void* c_kv_new, const void* k_rope_new, const int32_t* positions,
                                     const int32_t* block_table, int32_t bt_stride, int32_t page_rows,
                                     int64_t total_pages, void* q_lat, void* kv_cache, float* kv_scale,
                                     void* stream) {
  mla_status st = check_rope_args(dims, q_rope, c_kv_new, k_rope_new, positions, q_lat, kv_cache);
  if (st != MLA_OK) return st;
  if ((st = check_fp8_dims(dims, kv_scale)) != MLA_OK) return st;
  CacheMap cm;
  if ((st = paged_map(block_table, bt_stride, page_rows, total_pages, &cm)) != MLA_OK) return st;
  g_last_error.clear();
  return absorb_rope_fp8_impl(dims, q_nope, w_uk, q_rope, c_kv_new, k_rope_new, positions, cm, q_lat, kv_cache,
                              kv_scale, stream);
}

mla_status mla_combine(const mla_dims* dims, const void* o_part, const float* lse_part, int32_t num_splits,
                       float* o_lat, float* lse, void* stream) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({o_part, lse_part, o_lat})) != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (num_splits > kMaxSplits) return fail(MLA_ERR_WORKSPACE, "num_splits above 4096");
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  // split groups: about eight splits per thread, 1 to 16 groups
  int groups = 1;
  while (groups < kCombineMaxGroups && groups * 8 < num_splits) groups *= 2;
  const int64_t octs = (int64_t)(dims->rank / 8) * dims->heads;  // octets per split
  const int tq = (int)std::min<int64_t>(kCombineThreads / groups, octs);
  if (octs % tq != 0) return fail(MLA_ERR_UNSUPPORTED, "rank/8 * heads must be a multiple of the thread count");
  const dim3 grid((unsigned)(dims->batch * (octs / tq)));
  const dim3 block((unsigned)(tq * groups));
  // partials are stored in the dtype of the cache (see the decode kernel)
  if (dims->dtype == MLA_BF16 && dims->rank == 512) {
    hipLaunchKernelGGL((combine_kernel<512, u16>), grid, block, 0, s, (const u16*)o_part, lse_part, num_splits,
                       dims->heads, groups, o_lat, lse);
  } else if (dims->dtype == MLA_F32 && dims->rank == 64) {
    hipLaunchKernelGGL((combine_kernel<64, float>), grid, block, 0, s, (const float*)o_part, lse_part, num_splits,
                       dims->heads, groups, o_lat, lse);
  } else {
    return fail(MLA_ERR_UNSUPPORTED, "rank");
  }
  return launch_result("mla_combine");
}

mla_status mla_up_v(const mla_dims* dims, const float* o_lat, const void* w_uv, float* out, void* stream) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({o_lat, w_uv, out})) != MLA_OK) return st;
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  if (dims->dtype == MLA_BF16) {
    if (dims->rank != 512) return fail(MLA_ERR_UNSUPPORTED, "bf16 up_v is built for rank 512");
    const int blocks = (dims->heads + kXcds - 1) / kXcds * kXcds * (dims->d_v / 32);  // whole groups of 8 heads
    hipLaunchKernelGGL((up_v_bf16_kernel<512>), dim3(blocks), dim3(256), 0, s, o_lat,
                       (const u16*)w_uv, dims->batch, dims->heads, dims->d_v, out);
  } else {
    hipLaunchKernelGGL(up_v_f32_kernel, dim3(dims->heads * (dims->d_v / 32)), dim3(64), 0, s, o_lat,
                       (const float*)w_uv, dims->batch, dims->heads, dims->d_v, dims->rank, out);
  }
  return launch_result("mla_up_v");
}

mla_status mla_combine_up_v(const mla_dims* dims, const void* o_part, const float* lse_part, int32_t num_splits,
                            const void* w_uv, float* out, float* lse, void* stream) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({o_part, lse_part, w_uv, out})) != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (num_splits > kMaxSplits) return fail(MLA_ERR_WORKSPACE, "num_splits above 4096");
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  if (dims->dtype == MLA_BF16) {
    if (dims->rank != 512) return fail(MLA_ERR_UNSUPPORTED, "bf16 combine_up_v is built for rank 512");
    if ((int64_t)num_splits * dims->heads * dims->rank * 2 >= ((int64_t)1 << 31))
      return fail(MLA_ERR_UNSUPPORTED, "one sequence's partials must stay under 2 GB");
    // d_v 128 from three sequences up: split by sequences (each partial merged
    // once).  With one or two sequences there is no repeated merge to save, and
    // the per-block kernel measured faster (B 2: 15.1 against 16.0 us).
    if (dims->d_v == 128 && dims->batch > 2) {
      const int blocks = (dims->heads + kXcds - 1) / kXcds * kXcds * 2;  // whole groups of 8 heads, two halves
      if ((dims->batch + 1) / 2 > 16) {  // more than 16 sequences per half: two per wave with 16 waves
        hipLaunchKernelGGL(combine_up_v_bf16_d128_w16_kernel, dim3(blocks), dim3(kCuvWaves16 * 64), 0, s,
                           (const u16*)o_part, lse_part, num_splits, (const u16*)w_uv, dims->batch, dims->heads,
                           out, lse);
      } else {
        hipLaunchKernelGGL(combine_up_v_bf16_d128_kernel, dim3(blocks), dim3(kCuvWaves * 64), 0, s,
                           (const u16*)o_part, lse_part, num_splits, (const u16*)w_uv, dims->batch, dims->heads,
                           out, lse);
      }
      return launch_result("mla_combine_up_v");
    }
    const int nh = dims->d_v % 64 == 0 ? 2 : 1;
    const int blocks = (dims->heads + kXcds - 1) / kXcds * kXcds * (dims->d_v / (32 * nh));  // whole groups of 8 heads
    if (nh == 2) {
      hipLaunchKernelGGL((combine_up_v_bf16_kernel<2>), dim3(blocks), dim3(kCuvWaves * 64), 0, s, (const u16*)o_part,
                         lse_part, num_splits, (const u16*)w_uv, dims->batch, dims->heads, dims->d_v, out, lse);
    } else {
      hipLaunchKernelGGL((combine_up_v_bf16_kernel<1>), dim3(blocks), dim3(kCuvWaves * 64), 0, s, (const u16*)o_part,
                         lse_part, num_splits, (const u16*)w_uv, dims->batch, dims->heads, dims->d_v, out, lse);
    }
  } else {
    if (dims->rank > kCuvMaxRankF32) return fail(MLA_ERR_UNSUPPORTED, "fp32 combine_up_v takes rank <= 256");
    hipLaunchKernelGGL(combine_up_v_f32_kernel, dim3(dims->batch * dims->heads), dim3(64), 0, s,
                       (const float*)o_part, lse_part, num_splits, (const float*)w_uv, dims->heads, dims->d_v,
                       dims->rank, out, lse);
  }
  return launch_result("mla_combine_up_v");
}

mla_status mla_kv_down_workspace_size(const mla_dims* dims, int32_t d_model, size_t* bytes) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if (bytes == nullptr) return fail(MLA_ERR_INVALID_ARG, "bytes NULL");
  if (d_model < kKvChunk || d_model % kKvChunk != 0) return fail(MLA_ERR_UNSUPPORTED, "d_model must be a multiple of 512");
  *bytes = (size_t)(d_model / kKvChunk) * dims->batch * (dims->rank + dims->d_rope) * sizeof(float);
  return MLA_OK;
}

mla_status mla_kv_down(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                       const void* norm_w, float eps, void* workspace, void* c_kv_new, void* k_rope_new,
                       void* stream) {
  size_t ws = 0;
  mla_status st = mla_kv_down_workspace_size(dims, d_model, &ws);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({h, w_dkv, w_kr, norm_w, workspace, c_kv_new, k_rope_new})) != MLA_OK) return st;
  if (dims->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "kv_down is built for bf16 storage");
  if (dims->rank + dims->d_rope > 1024) return fail(MLA_ERR_UNSUPPORTED, "rank + d_rope above 1024");
  if (!(eps >= 0.f)) return fail(MLA_ERR_INVALID_ARG, "eps must be >= 0");
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  const int nf = dims->rank + dims->d_rope, nchunks = d_model / kKvChunk;
  hipLaunchKernelGGL(kv_down_partial_kernel, dim3(((nf + 31) / 32) * nchunks), dim3(256), 0, s, (const u16*)h,
                     (const u16*)w_dkv, (const u16*)w_kr, dims->batch, d_model, dims->rank, dims->d_rope,
                     (float*)workspace);
  hipLaunchKernelGGL(kv_down_final_kernel, dim3(dims->batch), dim3(256), 0, s, (const float*)workspace, nchunks,
                     dims->batch, dims->rank, dims->d_rope, (const u16*)norm_w, eps, (u16*)c_kv_new,
                     (u16*)k_rope_new);
  return launch_result("mla_kv_down");
}

// ---------------------------------------------------------------------------
// Folded projections (kernels in fold.hip)
// ---------------------------------------------------------------------------

static mla_status check_fold_dims(const mla_dims* dims) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if (dims->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the folded projections are built for bf16 storage");
  if (dims->rank % 64 != 0) return fail(MLA_ERR_UNSUPPORTED, "rank must be a multiple of 64");
  if (((int64_t)dims->heads * dims->rank) % 256 != 0) return fail(MLA_ERR_UNSUPPORTED, "heads * rank must be a multiple of 256");
  return MLA_OK;
}

static mla_status check_d_c_q(int32_t d_c_q) {
  if (d_c_q < 1) return fail(MLA_ERR_INVALID_ARG, "d_c_q must be >= 1");
  if (d_c_q % 256 != 0 || d_c_q > 65536) return fail(MLA_ERR_UNSUPPORTED, "d_c_q must be a multiple of 256, at most 65536");
  return MLA_OK;
}

static mla_status check_d_model(int32_t d_model) {
  if (d_model < 1) return fail(MLA_ERR_INVALID_ARG, "d_model must be >= 1");
  if (d_model % 64 != 0 || d_model > 65536) return fail(MLA_ERR_UNSUPPORTED, "d_model must be a multiple of 64, at most 65536");
  return MLA_OK;
}

static mla_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MLA_OK;
}

mla_status mla_fold_query(const mla_dims* dims, int32_t d_c_q, const void* w_uq, const void* w_uk, void* w_qk,
                          void* stream) {
  mla_status st = check_fold_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_d_c_q(d_c_q)) != MLA_OK) return st;
  if ((st = check_ptrs({w_uq, w_uk, w_qk})) != MLA_OK) return st;
  g_last_error.clear();
  return hip_result(mla_detail::launch_fold_query(dims->heads, dims->d_head, dims->rank, d_c_q, w_uq, w_uk, w_qk,
                                                  (hipStream_t)stream),
                    "mla_fold_query");
}

mla_status mla_fold_output(const mla_dims* dims, int32_t d_model, const void* w_o, const void* w_uv, void* w_ov,
                           void* stream) {
  mla_status st = check_fold_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_d_model(d_model)) != MLA_OK) return st;
  if ((st = check_ptrs({w_o, w_uv, w_ov})) != MLA_OK) return st;
  g_last_error.clear();
  return hip_result(mla_detail::launch_fold_output(dims->heads, dims->d_v, dims->rank, d_model, w_o, w_uv, w_ov,
                                                   (hipStream_t)stream),
                    "mla_fold_output");
}

mla_status mla_absorb_q_folded(const mla_dims* dims, int32_t d_c_q, const void* c_q, const void* w_qk, void* q_lat,
                               void* stream) {
  mla_status st = check_fold_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_d_c_q(d_c_q)) != MLA_OK) return st;
  if ((st = check_ptrs({c_q, w_qk, q_lat})) != MLA_OK) return st;
  g_last_error.clear();
  return hip_result(mla_detail::launch_absorb_q_folded(dims->batch, dims->heads, dims->rank,
                                                       dims->rank + dims->d_rope, d_c_q, c_q, w_qk, q_lat,
                                                       (hipStream_t)stream),
                    "mla_absorb_q_folded");
}

mla_status mla_out_folded_workspace_size(const mla_dims* dims, int32_t d_model, size_t* bytes) {
  mla_status st = check_fold_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_d_model(d_model)) != MLA_OK) return st;
  if (bytes == nullptr) return fail(MLA_ERR_INVALID_ARG, "bytes NULL");
  *bytes = mla_detail::out_folded_workspace_bytes(dims->batch, d_model, (int64_t)dims->heads * dims->rank);
  return MLA_OK;
}

mla_status mla_out_folded(const mla_dims* dims, int32_t d_model, const float* o_lat, const void* w_ov,
                          void* workspace, float* y, void* stream) {
  size_t ws = 0;
  mla_status st = mla_out_folded_workspace_size(dims, d_model, &ws);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({o_lat, w_ov, workspace, y})) != MLA_OK) return st;
  g_last_error.clear();
  return hip_result(mla_detail::launch_out_folded(dims->batch, d_model, (int64_t)dims->heads * dims->rank, o_lat,
                                                  w_ov, y, (float*)workspace, (hipStream_t)stream),
                    "mla_out_folded");
}

mla_status mla_kv_down_noalloc(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv,
                               const void* w_kr, const void* norm_w, float eps, void* c_kv_new, void* k_rope_new,
                               void* stream) {
  size_t ws = 0;
  mla_status st = mla_kv_down_workspace_size(dims, d_model, &ws);
  if (st != MLA_OK) return st;
  if ((st = check_ptrs({h, w_dkv, w_kr, norm_w, c_kv_new, k_rope_new})) != MLA_OK) return st;
  if (dims->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "kv_down is built for bf16 storage");
  if (dims->rank + dims->d_rope > 1024) return fail(MLA_ERR_UNSUPPORTED, "rank + d_rope above 1024");
  if (!(eps >= 0.f)) return fail(MLA_ERR_INVALID_ARG, "eps must be >= 0");
  if (ws > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "mla_kv_down_noalloc: (d_model / 512) * batch * (rank + d_rope) * 4 bytes of "
                                   "partial sums exceed its 4 MiB scratch; use mla_kv_down with a workspace");
  float* part = nullptr;
  if ((st = scratch_on_current_device(&part)) != MLA_OK) return st;
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;
  const int nf = dims->rank + dims->d_rope, nchunks = d_model / kKvChunk;
  hipLaunchKernelGGL(kv_down_partial_kernel, dim3(((nf + 31) / 32) * nchunks), dim3(256), 0, s, (const u16*)h,
                     (const u16*)w_dkv, (const u16*)w_kr, dims->batch, d_model, dims->rank, dims->d_rope, part);
  hipLaunchKernelGGL(kv_down_final_kernel, dim3(dims->batch), dim3(256), 0, s, (const float*)part, nchunks,
                     dims->batch, dims->rank, dims->d_rope, (const u16*)norm_w, eps, (u16*)c_kv_new,
                     (u16*)k_rope_new);
  return launch_result("mla_kv_down_noalloc");
}

mla_status mla_partials_size(const mla_dims* dims, int32_t num_splits, size_t* o_part_bytes, size_t* lse_part_bytes) {
  mla_status st = check_dims_impl(dims);
  if (st != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (num_splits > kMaxSplits) return fail(MLA_ERR_WORKSPACE, "num_splits above 4096");
  if (o_part_bytes == nullptr || lse_part_bytes == nullptr) return fail(MLA_ERR_INVALID_ARG, "NULL output");
  const size_t bsh = (size_t)dims->batch * (size_t)num_splits * (size_t)dims->heads;
  *o_part_bytes = bsh * (size_t)dims->rank * (dims->dtype == MLA_BF16 ? sizeof(uint16_t) : sizeof(float));
  *lse_part_bytes = bsh * sizeof(float);
  return MLA_OK;
}

}  // extern "C"

namespace {

constexpr int64_t kSplitCost = 8, kItemCost = 12;

int32_t device_cus(int32_t num_cus) {
  if (num_cus > 0) return num_cus;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  return prop.multiProcessorCount;
}

// Estimated decode time of `items` work-groups of `chunk` rows, in units of
// tiles / num_cus.  A work-group runs on one compute unit at a time and the
// items are dealt evenly over the 8 XCDs, so the decode takes (rounds of
// work-groups per CU) x (tiles per split + a fixed per-split cost for the
// prologue and the partial's store, about kSplitCost tiles).  Every
// non-empty split also adds its partial to what all work-groups start by
// loading at once and to what the merge reads back: about kItemCost tiles per
// CU's worth of splits.
int64_t split_cost(int64_t items, int64_t chunk, int64_t num_cus) {
  const int64_t cus_per_xcd = std::max<int64_t>(1, num_cus / 8);
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t rounds = (per_xcd + cus_per_xcd - 1) / cus_per_xcd;
  return rounds * (chunk / 32 + kSplitCost) * num_cus + kItemCost * items;
}

}  // namespace

extern "C" {

int32_t mla_plan_splits(const mla_dims* dims, int32_t max_seq_len, int64_t total_rows, int32_t num_cus) {
  if (check_dims_impl(dims) != MLA_OK) return 0;
  if (max_seq_len < 1 || total_rows < 1) return 0;
  if ((num_cus = device_cus(num_cus)) <= 0) return 0;
  // The split count with the smallest estimated decode time (split_cost).
  // Only the total and the longest length are known here: the non-empty
  // splits are at most B * ceil(max / chunk), and for mixed lengths about
  // total / chunk plus the partial last split of every sequence (counted as
  // 0.6 of a split each, a little above the mean).  Ties go to fewer splits.
  const int64_t B = dims->batch;
  const int64_t s_max = std::min<int64_t>(kMaxSplits, ((int64_t)max_seq_len + 31) / 32);
  int64_t best = 1, best_cost = INT64_MAX;
  for (int64_t sp = 1; sp <= s_max; ++sp) {
    const int64_t chunk = chunk_rows(max_seq_len, (int32_t)sp);
    const int64_t full = B * (((int64_t)max_seq_len + chunk - 1) / chunk);
    const int64_t est = std::min(full, (total_rows + chunk - 1) / chunk + (6 * B + 9) / 10);
    const int64_t cost = split_cost(est, chunk, num_cus);
    if (cost < best_cost) best_cost = cost, best = sp;
  }
  return (int32_t)std::max<int64_t>(1, best);
}

int32_t mla_plan_splits_for_lengths(const mla_dims* dims, const int32_t* seq_lens, int32_t num_cus,
                                    int32_t* plan_max_seq_len) {
  if (check_dims_impl(dims) != MLA_OK || seq_lens == nullptr || plan_max_seq_len == nullptr) return 0;
  if ((num_cus = device_cus(num_cus)) <= 0) return 0;
  int64_t max_len = 0;
  for (int32_t b = 0; b < dims->batch; ++b) {
    if (seq_lens[b] < 1) return 0;
    max_len = std::max<int64_t>(max_len, seq_lens[b]);
  }
  // Every chunk of whole tiles is a candidate, with the split count it needs
  // (the largest per-sequence count) and the exact number of non-empty
  // splits, counted as the decode kernel counts its work items; the cost is
  // that of mla_plan_splits.  The chunk is then reached through
  // max_seq_len' = chunk * splits (>= every length), since the kernels take
  // ceil(max_seq_len' / splits) rounded up to whole tiles as the chunk.
  int64_t best_s = 1, best_chunk = ((max_len + 31) / 32) * 32, best_cost = INT64_MAX;
  for (int64_t tiles = (max_len + 31) / 32; tiles >= 1; --tiles) {
    const int64_t chunk = 32 * tiles;
    int64_t items = 0, splits = 0;
    for (int32_t b = 0; b < dims->batch; ++b) {
      const int64_t n = (seq_lens[b] + chunk - 1) / chunk;
      items += n;
      splits = std::max(splits, n);
    }
    if (splits > kMaxSplits || chunk * splits > INT32_MAX) break;  // (finer chunks only need more)
    const int64_t cost = split_cost(items, chunk, num_cus);
    if (cost < best_cost) best_cost = cost, best_s = splits, best_chunk = chunk;
  }
  *plan_max_seq_len = (int32_t)(best_chunk * best_s);
  return (int32_t)best_s;
}



}  // extern "C"
