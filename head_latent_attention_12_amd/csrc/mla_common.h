// Device helpers shared by the HIP sources of the MLA decode library
// (internal: not part of the C ABI).  Everything sits in an anonymous
// namespace, so each translation unit has its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace mla_detail {

// Where the rows of a sequence live in the cache.  Packed: in-sequence row t
// of sequence b is cache row row_offsets[b] + t.  Paged: the cache is pages
// of 2^page_shift rows (at least 32, so a 32-row tile never straddles two),
// and row t is row t & (page_rows - 1) of page block_table[b * bt_stride +
// (t >> page_shift)].  Rows are clamped into the cache either way, so that
// inconsistent metadata can only give wrong numbers, never a stray access.
struct CacheMap {
  const int64_t* row_offsets;  // packed (nullptr when paged)
  const int32_t* block_table;  // paged (nullptr when packed)
  int64_t total_rows;          // rows in the cache
  int64_t total_pages;         // paged: pages in the cache
  int32_t bt_stride;           // paged: entries per sequence in block_table
  int32_t page_shift;          // paged: log2(page_rows)
  // (bt: block_table, passed separately where a restrict-qualified pointer
  // lets the compiler read it with scalar loads)
  __device__ __forceinline__ int64_t paged_row(int b, int t, const int32_t* __restrict__ bt) const {
    int pi = t >> page_shift;
    pi = pi < 0 ? 0 : (pi >= bt_stride ? bt_stride - 1 : pi);
    int64_t pg = bt[(int64_t)b * bt_stride + pi];
    pg = pg < 0 ? 0 : (pg >= total_pages ? total_pages - 1 : pg);
    return (pg << page_shift) + (t & ((1 << page_shift) - 1));
  }
  // row t of sequence b; off = row_offsets[b] (packed, loaded by the caller)
  __device__ __forceinline__ int64_t row(int b, int t, int64_t off) const {
    if (block_table != nullptr) return paged_row(b, t, block_table);
    const int64_t r = off + t;
    return r < 0 ? 0 : (r >= total_rows ? total_rows - 1 : r);
  }
};

}  // namespace mla_detail

namespace {

using mla_detail::CacheMap;

using u16 = uint16_t;
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// Softmax reference: each head's exponent reference is fixed at the first tile
// of a split, and p = 2^(s - ref) is accepted up to 2^kRefSlack (finite in fp32
// and bf16, no overflow of the sums).  If a later score exceeds ref + kRefSlack,
// the work-group runs a scores-only pass over the split to find each head's
// exact maximum and then redoes the split with that reference (p <= 1), so the
// accumulators are never rescaled inside the loop and at most one redo happens.
// The bf16 pipelined loop checks this once per pass on the sum of the weights
// instead of per tile on the scores: every weight is non-negative, so a sum
// below 2^kRefSlack means every weight was, and a weight at or above it (or an
// infinite one) makes the sum fail the test (a few weights just under the bound
// may also trigger a redo, which is only slower).
constexpr float kRefSlack = 64.0f;
// MI355X: 8 accelerator complex dies (XCDs), each with its own L2
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// bf16 helpers (storage type u16 holds bf16 bits)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ u16 f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Round a finite fp32 value to the nearest bf16 (ties to even), kept as fp32.
__device__ __forceinline__ float round_bf16_finite(float a) {
  uint32_t u = __float_as_uint(a);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

// Two fp32 values rounded to bf16 (nearest even, v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Pack two fp32 values that are already bf16-representable into bf16x2.
__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// double -> bf16 with a single rounding: round to odd into fp32, then nearest
// even into bf16 (fp32 keeps more than two extra bits, so the result is the
// correctly rounded bf16).
__device__ __forceinline__ u16 d2bf(double x) {
  float f = (float)x;
  double fd = (double)f;
  uint32_t u = __float_as_uint(f);
  if (fd != x) {
    if (fabs(fd) > fabs(x)) u -= 1u;  // step toward zero (same sign)
    u |= 1u;
  }
  return f2bf(__uint_as_float(u));
}

template <typename T> __device__ __forceinline__ double load_d(T v);
template <> __device__ __forceinline__ double load_d<u16>(u16 v) { return (double)bf2f(v); }
template <> __device__ __forceinline__ double load_d<float>(float v) { return (double)v; }
template <typename T> __device__ __forceinline__ T store_d(double v);
template <> __device__ __forceinline__ u16 store_d<u16>(double v) { return d2bf(v); }
template <> __device__ __forceinline__ float store_d<float>(double v) { return (float)v; }

// ---------------------------------------------------------------------------
// MFMA traits
// ---------------------------------------------------------------------------

template <typename T> struct Mma;
template <> struct Mma<u16> {
  static constexpr int KSTEP = 16;  // k per instruction (8 per lane)
  using Frag = i16x8;
  __device__ static __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 2;  // k per instruction (1 per lane)
  using Frag = float;
  __device__ static __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Combine a value with the one held by lane ^ 32 (v_permlane32_swap: the two
// results together hold both halves' values in every lane).
template <typename F>
__device__ __forceinline__ float xor32(float v, F op) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A value combined over the 64 lanes of a wave, the result in every lane:
// DPP moves inside each row of 16 lanes (swap neighbours, swap pairs, mirror
// within 8, mirror within 16), then the rows exchanged with permlane16 and
// permlane32 swaps (no LDS round trips).  Every lane must be active.
template <typename F>
__device__ __forceinline__ float wave_reduce_f(float v, F op) {
  auto dpp = [](float x, int ctrl) -> float {
    switch (ctrl) {  // (the control is a constant of the instruction)
      case 0xb1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
      case 0x4e: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
      case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
    }
  };
  v = op(v, dpp(v, 0xb1));   // quad_perm [1,0,3,2]
  v = op(v, dpp(v, 0x4e));   // quad_perm [2,3,0,1]
  v = op(v, dpp(v, 0x141));  // row_half_mirror
  v = op(v, dpp(v, 0x140));  // row_mirror
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  return xor32(v, op);
}
// Sum and inclusive prefix sum of an int over the 64 lanes of a wave, with
// DPP lane moves (no LDS round trips): prefix sums within each row of 16
// lanes by shifts of 1, 2, 4 and 8 lanes (a lane shifted in from before its
// row start reads 0), then the last lane of row 0 is added to row 1 and that
// of row 2 to row 3 (row_bcast:15), then lane 31 to rows 2 and 3
// (row_bcast:31).  Every lane of the wave must be active.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_prefix_sum(v), 63); }

// A 64-bit value known to be uniform across the wave, in SGPRs
// (readfirstlane returns int: each half goes through uint32_t so that the low
// half is not sign-extended into the high one).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}



// Work items are the non-empty splits (b, s < n_b), n_b = ceil(seq_len_b /
// chunk) clamped to [1, num_splits], taken in sequence order (times GROUPS head
// groups).  Work-groups are dealt to the 8 XCDs round-robin (blockIdx % 8);
// item L goes to XCD L / per, so that the splits of one sequence share an
// XCD (its L2 serves their common q_lat) and each XCD gets the same number
// of items whatever the lengths.  The grid (host: 8 * ceil(B*num_splits*
// GROUPS / 8)) bounds the item count; work-groups without an item exit.
// The work-group of split 0 marks the sequence's empty splits (lse -inf).
// Each lane looks at one sequence per step of 64; the first 64 lengths and
// row offsets are loaded once and serve both passes, so that with B <= 64
// the item's metadata costs a single round of loads.
struct DecodeItem {
  int b, s, n_b, seq_len;
  int64_t row_off;  // packed cache: row_offsets[b]
};
template <bool PAGED, int GROUPS>
__device__ __forceinline__ bool decode_item(const int32_t* __restrict__ seq_lens, const CacheMap& cm, int batch,
                                            int num_splits, int chunk, DecodeItem& it) {
  auto splits_of = [&](int len) { return max(1, min(num_splits, (len + chunk - 1) / chunk)); };
  int b = 0, s = 0, n_b = 0, seq_len = 0;
  int64_t row_off = 0;
  const int lane = threadIdx.x & 63;
  {
    const int bid = (int)blockIdx.x;
    const bool in0 = lane < batch;
    const int len0 = in0 ? seq_lens[lane] : 0;
    const int64_t off0 = (!PAGED && in0) ? cm.row_offsets[lane] : 0;
    // pass 1: item count
    int items = wave_sum(in0 ? splits_of(len0) : 0);
    for (int c0 = 64; c0 < batch; c0 += 64) {
      const int bb = c0 + lane;
      items += wave_sum(bb < batch ? splits_of(seq_lens[bb]) : 0);
    }
    items *= GROUPS;
    const int per = (items + kXcds - 1) / kXcds;
    const int item = (bid % kXcds) * per + bid / kXcds;
    // an XCD's work-groups past its `per` items would repeat the next XCD's
    if (bid / kXcds >= per || item >= items) return false;
    // pass 2: the sequence holding the item (inclusive prefix sums per step)
    const int want = item / GROUPS;
    int base = 0;
    for (int c0 = 0; c0 < batch; c0 += 64) {
      const int bb = c0 + lane;
      int len = len0;
      int64_t off = off0;
      if (c0 > 0) {
        len = bb < batch ? seq_lens[bb] : 0;
        off = (!PAGED && bb < batch) ? cm.row_offsets[bb] : 0;
      }
      const int n = bb < batch ? splits_of(len) : 0;
      const int incl = wave_prefix_sum(n) + base;
      const uint64_t hit = __ballot(incl > want);
      if (hit != 0) {
        const int first = __builtin_ctzll(hit);
        b = c0 + first;
        n_b = __shfl(n, first);
        s = want - (__shfl(incl, first) - n_b);
        seq_len = __shfl(len, first);
        row_off = __shfl(off, first);
        break;
      }
      base = __builtin_amdgcn_readlane(incl, 63);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    s = __builtin_amdgcn_readfirstlane(s);
    n_b = __builtin_amdgcn_readfirstlane(n_b);
    seq_len = __builtin_amdgcn_readfirstlane(seq_len);
    row_off = (int64_t)uniform_u64((uint64_t)row_off);
  }
  it = DecodeItem{b, s, n_b, seq_len, row_off};
  return true;
}

}  // namespace

// fp8 latent cache decode (decode_fp8.hip), launched by the C-ABI entry points
// after their argument checks.
hipError_t mla_launch_decode_fp8(const void* q_lat, const void* cache, const float* scales,
                                 const mla_detail::CacheMap& cm,
                                 const int32_t* seq_lens, int32_t batch, int32_t num_splits, int32_t chunk,
                                 void* o_part, float* lse_part, float scale_log2, hipStream_t stream);

// Folded projections (fold.hip), launched by the C-ABI entry points after
// their argument checks.
namespace mla_detail {
hipError_t launch_fold_query(int H, int dh, int r, int dcq, const void* w_uq, const void* w_uk, void* w_qk,
                             hipStream_t stream);
hipError_t launch_fold_output(int H, int dv, int r, int d_model, const void* w_o, const void* w_uv, void* w_ov,
                              hipStream_t stream);
hipError_t launch_absorb_q_folded(int B, int H, int r, int W, int dcq, const void* c_q, const void* w_qk,
                                  void* q_lat, hipStream_t stream);
size_t out_folded_workspace_bytes(int B, int d_model, int64_t K);
hipError_t launch_out_folded(int B, int d_model, int64_t K, const float* o_lat, const void* w_ov, float* y,
                             float* workspace, hipStream_t stream);
}  // namespace mla_detail
