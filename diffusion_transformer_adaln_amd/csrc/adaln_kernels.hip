// Fused AdaLN (LayerNorm + per-sample modulation) kernels for gfx950 (CDNA4).
//
// The operator is the fused LayerNorm-modulate of the AdaptiveLoad technical
// summary (gist.science 2605.17923), section 2.B: one launch for the
// forward with row statistics kept on chip, and a backward whose per-sample
// modulation gradients are column sums over N taken with threads pinned to
// feature columns so every access is contiguous along D.
//
// The path is HBM-bound (about 2 flop per byte), so nothing here uses MFMA.
// What matters is bytes in flight, 16-byte vector accesses, and keeping the
// row in registers between the statistics and the output:
//
//   * A row of D elements is V = D/EPV vectors of 16 bytes (EPV = 8 for bf16,
//     4 for fp32).  LPR lanes (a multiple of 16) cooperate on one row, each
//     holding VPT vectors: lane l owns vectors l, l+LPR, ..., so each vector
//     load of a row is one contiguous 16*LPR-byte span.  A workgroup of NT
//     threads works on NT/LPR rows at a time ("slots"), and each slot keeps
//     RIF rows in flight per iteration.
//   * Rows of exactly 64 lanes x at most 10 vectors take a persistent forward
//     instead: one wave per row, a fixed grid of about four waves per CU
//     walking the rows grid-stride, each wave loading its next row into
//     registers while it reduces and writes the current one.
//   * Row reductions run in three fixed-order stages: a 16-lane butterfly
//     with DPP (quad_perm, row_half_mirror, row_mirror), cross-row lane
//     exchanges inside the wave, then LDS across the waves or 16-lane groups
//     that share the row, merged in ascending order by every thread.  Every
//     lane therefore ends with bitwise identical statistics, and the results
//     never depend on timing.
//   * Forward statistics are a parallel (Chan) Welford merge of per-lane
//     (mean, M2) pairs, so large row offsets and x20 outlier rows lose no
//     precision.
//   * The backward keeps each lane's column partial sums of dy and dy*xhat in
//     registers over a tile of rows inside one sample, combines the slots of a
//     workgroup through LDS in slot order, and writes them once per tile,
//     coalesced along D.  A finish kernel adds a sample's tiles in fp64, in
//     an order fixed by the shape and the CU count, and rounds each sum once
//     to the output type (the I/O type, or fp32 when the caller asks for
//     fp32 column sums).  No floating-point atomics anywhere: bitwise
//     repeatable.
//
// General kernels (any D, any alignment) cover the shapes the vector layout
// cannot; they compute the same quantities with scalar accesses.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_internal.hpp"

namespace adaln {

// ---------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int DT> struct Elem;
template <> struct Elem<F32> {
  static constexpr int EPV = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  // an fp64 sum stored with one rounding (to nearest, ties to even)
  __device__ static __forceinline__ void store_sum(void* p, int64_t i, double v) {
    static_cast<float*>(p)[i] = static_cast<float>(v);
  }
  // acc + the sum of the vector's elements
  __device__ static __forceinline__ float accumulate(const uint4& v, float acc) {
    return acc + __uint_as_float(v.x) + __uint_as_float(v.y) + __uint_as_float(v.z) +
           __uint_as_float(v.w);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);   // v_cvt_pk_bf16_f32: RNE
  return __builtin_bit_cast(uint32_t, b);
}

template <> struct Elem<BF16> {
  static constexpr int EPV = 8;
  __device__ static __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    unpack2(v.x, f[0], f[1]); unpack2(v.y, f[2], f[3]);
    unpack2(v.z, f[4], f[5]); unpack2(v.w, f[6], f[7]);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
  // An fp64 sum stored with one rounding to bf16 (to nearest, ties to even).
  // Rounding to fp32 first and then to bf16 could land a value just off a
  // bf16 midpoint exactly on it and break the tie the wrong way, so the
  // fp32 step rounds to odd instead: v itself if it is an fp32 value, else
  // whichever of the two fp32 values around v has an odd significand.  With
  // 24 >= 8 + 2 significand bits, round-to-odd followed by
  // round-to-nearest-even gives the correctly rounded result (Boldo and
  // Melquiond, "Emulation of FMA and correctly rounded sums: proved
  // algorithms using rounding to odd", IEEE TC 2008).  The nearest fp32
  // value t is one of the two; when it is even, its neighbour towards v (one
  // step in the bit pattern, whose parity alternates) is the odd one.
  __device__ static __forceinline__ void store_sum(void* p, int64_t i, double v) {
    const float t = static_cast<float>(v);
    const double back = static_cast<double>(t);
    uint32_t b = __float_as_uint(t);
    if (back != v && !(b & 1u)) b = fabs(v) > fabs(back) ? b + 1u : b - 1u;
    store1(p, i, __uint_as_float(b));
  }
  // acc + the sum of the vector's elements: one v_dot2_f32_bf16 against
  // (1, 1) per packed pair, straight from the stored bits (the products are
  // exact, so each step adds two elements to the fp32 accumulator).  Half the
  // instructions of unpack-and-add on the forward's critical path between a
  // row's arrival and its next row's request: persistent forward on the video
  // shape 66.9 -> 66.4 us; the slot kernel (DiT) showed no gain and keeps adds.
  __device__ static __forceinline__ float accumulate(const uint4& v, float acc) {
    const bf16x2_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.z), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w), one, acc, false);
    return acc;
  }
};

// x - c for every element of a 16-byte vector, as x + (-c): the same
// correctly rounded value as the subtraction.
template <int DT> struct Center {
  __device__ static __forceinline__ void apply(const uint4& v, float negc, float* d) {
    Elem<DT>::unpack(v, d);
#pragma unroll
    for (int k = 0; k < Elem<DT>::EPV; ++k) d[k] += negc;
  }
};

// Streaming (non-temporal) 16-byte accesses for the row tensors of the
// vectorised kernels: x, dy, y and dx are touched once per call and are far
// larger than L2 plus the MALL, so caching them buys nothing.  Measured on
// MI355X (video shape, fwd and bwd alternating on cold buffers): streaming
// loads take the backward row pass from 128 to 107 us, and streaming stores
// leave no dirty lines for the next kernel to write back (a following
// backward runs 117 instead of 128 us).  The general kernels re-read a row
// from cache and keep ordinary accesses.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// The backward's per-element arithmetic, shared by every backward kernel so
// that all of them produce the same bits for the same row:
//   g  = dy*(1 + scale) with one rounding, as fma(dy, scale, dy);
//   dx = rstd*((g - a) - xhat*c) with a = sum(g)/D, c = sum(g*xhat)/D.
// g - a comes first: it is exact when g is close to a, so dx is exactly 0
// where the formula gives 0 (D = 1, or a constant g on a constant row).
// Folding rstd in first (rstd*g - rstd*a, two fmas) saves one instruction
// but leaves the rounding error of rstd*a there instead.
__device__ __forceinline__ float grad_g(float dy, float scale) { return __builtin_fmaf(dy, scale, dy); }
struct RowGrad {
  float rs, a, c;
  __device__ __forceinline__ RowGrad(float sum_g, float sum_gx, float rstd, float inv_d)
      : rs(rstd), a(sum_g * inv_d), c(sum_gx * inv_d) {}
  __device__ __forceinline__ float dx(float g, float xh) const {
    return rs * __builtin_fmaf(-xh, c, g - a);
  }
};

// acc / n for a count n: the product with the rounded reciprocal, then one
// correction step (the residual acc - n*q is exact under an fma).  For a sum
// of n equal values c (acc = n*c exactly) the result is exactly c, so a row of
// equal values gets zero variance; a multiply by 1/n alone can miss c by an
// ulp when 1/n is not an fp32 value (n = 24, 80), and an IEEE division costs
// a longer dependent chain on the forward's critical path.
__device__ __forceinline__ float div_count(float acc, float n, float inv_n) {
  const float q = acc * inv_n;
  const float r = __builtin_fmaf(-q, n, acc);
  return __builtin_fmaf(r, inv_n, q);
}

// ---------------------------------------------------------------------------
// cross-lane exchange
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_1032 = 0xB1;       // quad_perm [1,0,3,2]: partner lane ^ 1
constexpr int DPP_QUAD_2301 = 0x4E;       // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <-> 7-i inside each 8-lane half row
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <-> 15-i inside each 16-lane row

// Partner value at level k (0..3) of the 16-lane butterfly.  After level k
// every lane of an aligned group of 2^(k+1) lanes holds that group's result,
// so any pairing across the two halves completes the next level.
template <int LEVEL>
__device__ __forceinline__ float partner16(float v) {
  if constexpr (LEVEL == 0) return dpp<DPP_QUAD_1032>(v);
  else if constexpr (LEVEL == 1) return dpp<DPP_QUAD_2301>(v);
  else if constexpr (LEVEL == 2) return dpp<DPP_ROW_HALF_MIRROR>(v);
  else return dpp<DPP_ROW_MIRROR>(v);
}

__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Chan, Golub and LeVeque's pairwise merge of two (mean, M2) summaries that
// cover the same count n each (half_n = n/2):
//   mean = (ma + mb)/2,  M2 = M2a + M2b + (mb - ma)^2 * n/2.
// Commutative in its two arguments bit for bit, so both partners agree.
__device__ __forceinline__ void chan_equal(float& m, float& s, float mo, float so, float half_n) {
  const float d = mo - m;
  m = 0.5f * (m + mo);
  s = (s + so) + (d * d) * half_n;
}

// Merge (mo, so) covering `no` elements into (m, s) covering `n` elements.
__device__ __forceinline__ void chan_merge(float& m, float& s, float& n, float mo, float so, float no) {
  const float nt = n + no;
  const float d = mo - m;
  const float w = no / nt;
  m = m + d * w;
  s = (s + so) + (d * d) * (n * w);
  n = nt;
}

// Reduce a (mean, M2) pair over an aligned group of `unit` lanes (16, 32 or
// 64); n_lane is each lane's element count.  All lanes of the group end with
// the same bits.
__device__ __forceinline__ void chan_reduce_unit(float& m, float& s, float n_lane, int unit) {
  float n = n_lane;
  float mo, so;
  mo = partner16<0>(m); so = partner16<0>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<1>(m); so = partner16<1>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<2>(m); so = partner16<2>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<3>(m); so = partner16<3>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  if (unit >= 32) { mo = xor_lane(m, 16); so = xor_lane(s, 16); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f; }
  if (unit >= 64) { mo = xor_lane(m, 32); so = xor_lane(s, 32); chan_equal(m, s, mo, so, 0.5f * n); }
}

// Sum over an aligned group of `unit` lanes; all lanes get the same bits.
__device__ __forceinline__ float sum_unit(float v, int unit) {
  v = v + partner16<0>(v);
  v = v + partner16<1>(v);
  v = v + partner16<2>(v);
  v = v + partner16<3>(v);
  if (unit >= 32) v = v + xor_lane(v, 16);
  if (unit >= 64) v = v + xor_lane(v, 32);
  return v;
}

// The two halves of a cross-row exchange: v_permlane16_swap exchanges the
// odd 16-lane rows of one register with the even rows of another, and
// v_permlane32_swap the upper 32 lanes with the lower 32.  Applied to two
// copies of v, both lanes of a partner pair receive the same ordered pair
// (value of the lower lane, value of the upper lane), so any function of the
// pair gives the same bits in both lanes, with no LDS and no lane-index
// arithmetic.
struct LanePair {
  float lower, upper;
};
__device__ __forceinline__ LanePair swap16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return LanePair{__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ LanePair swap32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return LanePair{__uint_as_float(p[0]), __uint_as_float(p[1])};
}

// Chan merge of the two halves of a lane pair covering n/2 elements each.
__device__ __forceinline__ void chan_pair(float& m, float& s, const LanePair& pm, const LanePair& ps,
                                          float half_n) {
  const float d = pm.upper - pm.lower;
  m = 0.5f * (pm.lower + pm.upper);
  s = (ps.lower + ps.upper) + (d * d) * half_n;
}

// (mean, M2) over the whole wave, n_lane elements per lane; every lane ends
// with the same bits.  Four DPP levels inside each 16-lane row, then the
// row pairs and the half-waves through the swap instructions.
__device__ __forceinline__ void chan_reduce_wave(float& m, float& s, float n_lane) {
  float n = n_lane;
  float mo, so;
  mo = partner16<0>(m); so = partner16<0>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<1>(m); so = partner16<1>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<2>(m); so = partner16<2>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  mo = partner16<3>(m); so = partner16<3>(s); chan_equal(m, s, mo, so, 0.5f * n); n *= 2.f;
  chan_pair(m, s, swap16(m), swap16(s), 0.5f * n); n *= 2.f;
  chan_pair(m, s, swap32(m), swap32(s), 0.5f * n);
}

// Sum over the whole wave; every lane ends with the same bits.
__device__ __forceinline__ float sum_wave(float v) {
  v = v + partner16<0>(v);
  v = v + partner16<1>(v);
  v = v + partner16<2>(v);
  v = v + partner16<3>(v);
  LanePair p = swap16(v);
  v = p.lower + p.upper;
  p = swap32(v);
  return p.lower + p.upper;
}

// Lanes that reduce together before LDS: a whole wave when a row covers whole
// waves, 32 lanes when two rows share a wave, else one 16-lane DPP row.
__device__ __forceinline__ int reduce_unit(int lpr) {
  return (lpr % 64 == 0) ? 64 : (lpr == 32 ? 32 : 16);
}

// ---------------------------------------------------------------------------
// row -> sample
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t sample_of_row(const RowMap& rm, int64_t row) {
  if (rm.offsets == nullptr) return row / rm.N;
  // largest b with offsets[b] <= row  (offsets non-decreasing; empty samples
  // skipped); always in [0, B) whatever the table holds
  int64_t lo = 0, hi = rm.B;   // invariant: offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (clamp_row(rm.offsets[mid], rm.R) <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// Packed batches of at most PACKED_FEW_SAMPLES (64) samples need no tile
// table in memory (and no prologue launch): any wave rebuilds it from the
// offsets.
// Lane i holds sample i's tile count (ceil of its clamped row count over
// tile_rows); an inclusive prefix sum over the wave gives every sample's tile
// range [excl, incl), both capped at tiles_alloc exactly as the prologue caps
// the table it writes, so both ways number the tiles identically.  Every lane
// of the wave must take part.
static_assert(PACKED_FEW_SAMPLES <= 64, "one sample per lane of a wave");

struct WaveTiles {
  int64_t excl, incl;   // this lane's sample: tiles [excl, incl)
};

// v from lane `lane` (wave-uniform) as a wave-uniform value, so that what is
// derived from it stays in scalar registers.
__device__ __forceinline__ int64_t lane_value(int64_t v, int lane) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
  const int32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane);
  return (static_cast<int64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ WaveTiles wave_tile_table(const RowMap& rm, const Tiling& tl) {
  const int lane = threadIdx.x & 63;
  int64_t cnt = 0;
  if (lane < rm.B) {
    const int64_t n = clamped_span(rm.offsets[lane], rm.offsets[lane + 1], rm.R).n;
    cnt = n > 0 ? (n + tl.tile_rows - 1) / tl.tile_rows : 0;
  }
  int64_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  return WaveTiles{min(incl - cnt, tl.tiles_alloc), min(incl, tl.tiles_alloc)};
}

// Sample b of packed tile t (the largest b whose first tile is <= t) and its
// tiles [t0, t1); false when t is at or past the last tile (a spare
// workgroup of the packed grid).  Table in memory, or rebuilt by the wave.
__device__ __forceinline__ bool varlen_tile_sample(const RowMap& rm, const Tiling& tl, int64_t t,
                                                   int64_t& b, int64_t& t0, int64_t& t1) {
  if (tl.tile_start == nullptr) {
    const WaveTiles w = wave_tile_table(rm, tl);
    const int lane = threadIdx.x & 63;
    if (t >= lane_value(w.incl, 63)) return false;   // lanes >= B add nothing: lane 63 has the total
    const unsigned long long below = __ballot(lane < rm.B && w.excl <= t);   // lane 0 always
    const int bl = 63 - __clzll(static_cast<long long>(below));
    b = bl;
    t0 = lane_value(w.excl, bl);
    t1 = lane_value(w.incl, bl);
    return true;
  }
  if (t >= tl.tile_start[rm.B]) return false;
  int64_t lo = 0, hi = rm.B;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (tl.tile_start[mid] <= t) lo = mid; else hi = mid;
  }
  b = lo;
  t0 = tl.tile_start[b];
  t1 = tl.tile_start[b + 1];
  return true;
}

// Rows of tile t: sample b, rows first + m*step for m in [0, count); false
// for a spare workgroup of the packed grid (past the last tile), which then
// has nothing to do.  Sample b's rows are split over its tiles either in
// contiguous runs of tile_rows rows (step 1) or, with tl.interleave,
// round-robin (tile k of the sample takes rows k, k + tiles, k + 2*tiles,
// ...), which keeps the rows in flight across the chip inside a narrow
// moving window.  Every thread of the workgroup calls this (the packed
// lookup may use wave-wide operations).  PACKED: the batch has an offsets
// table (a compile-time choice, so that the dense kernels carry none of the
// packed lookup's registers).
template <bool PACKED>
__device__ __forceinline__ bool tile_rows_of(const RowMap& rm, const Tiling& tl, int64_t t,
                                             int64_t& b, int64_t& first, int64_t& step,
                                             int64_t& count) {
  int64_t k, tiles, lo_row, n;
  if constexpr (!PACKED) {
    tiles = (rm.N + tl.tile_rows - 1) / tl.tile_rows;
    b = t / tiles;
    k = t - b * tiles;
    lo_row = b * rm.N;
    n = rm.N;
  } else {
    int64_t t0, t1;
    if (!varlen_tile_sample(rm, tl, t, b, t0, t1)) return false;
    k = t - t0;
    tiles = t1 - t0;
    const RowSpan sp = clamped_span(rm.offsets[b], rm.offsets[b + 1], rm.R);
    lo_row = sp.lo;
    n = sp.n;
  }
  if (tl.interleave) {
    first = lo_row + k;
    step = tiles;
    count = (n - k + tiles - 1) / tiles;
  } else {
    first = lo_row + k * tl.tile_rows;
    step = 1;
    count = min(tl.tile_rows, n - k * tl.tile_rows);
  }
  return true;
}

// Tile partials are chunk-major (PCOLS columns per chunk, see
// adaln_internal.hpp).  Element (tile t, quantity q: 0 = sum dy,
// 1 = sum dy*xhat, column d):
__device__ __forceinline__ int64_t pidx(int64_t tiles_alloc, int64_t t, int q, int d) {
  return ((static_cast<int64_t>(d / PCOLS) * tiles_alloc + t) * 2 + q) * PCOLS + (d % PCOLS);
}


// ---------------------------------------------------------------------------
// vectorised forward
// ---------------------------------------------------------------------------
// Grid: one workgroup per chunk of `rows_per_wg` consecutive rows.
// LDS: 2 buffers x [slots][RIF][groups] x (mean, M2).

template <int DT, int VPT, int RIF, int NTMAX = VEC_MAX_NT>
__global__ void __launch_bounds__(NTMAX)
fwd_vec_kernel(const uint4* __restrict__ x, const uint4* __restrict__ shift,
               const uint4* __restrict__ scale, float eps, RowMap rm, int V, int D, int lpr,
               int64_t rows_per_wg, uint4* __restrict__ y, float* __restrict__ mean,
               float* __restrict__ rstd) {
  using E = Elem<DT>;
  constexpr int EPV = E::EPV;
  extern __shared__ float2 lds_f2[];

  const int tid = threadIdx.x;
  const int nslots = blockDim.x / lpr;
  const int slot = tid / lpr;
  const int lane = tid - slot * lpr;
  const int unit = reduce_unit(lpr);
  const int groups = lpr / unit;          // LDS partials per row
  const int group = lane / unit;
  const bool leader = (lane % unit) == 0;
  const int buf_stride = nslots * RIF * groups;

  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t r_end = min(rm.R, r_begin + rows_per_wg);
  const int64_t rows_per_iter = static_cast<int64_t>(nslots) * RIF;
  const float inv_d = 1.0f / static_cast<float>(D);
  constexpr float n_lane = static_cast<float>(VPT * EPV);

  float sc1[VPT][EPV], sh[VPT][EPV];
  int64_t cur_lo = 0, cur_hi = 0;     // rows of the sample whose modulation is loaded
  auto load_mod = [&](int64_t r) {    // unpacked 1 + scale and shift of row r's sample
    const int64_t b = sample_of_row(rm, r);
    cur_lo = rm.offsets ? clamp_row(rm.offsets[b], rm.R) : b * rm.N;
    cur_hi = rm.offsets ? clamp_row(rm.offsets[b + 1], rm.R) : cur_lo + rm.N;
    const uint4* scp = scale + b * V + lane;
    const uint4* shp = shift + b * V + lane;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      E::unpack(scp[j * lpr], sc1[j]);
      E::unpack(shp[j * lpr], sh[j]);
#pragma unroll
      for (int k = 0; k < EPV; ++k) sc1[j][k] += 1.0f;
    }
  };
  uint4 xv[RIF][VPT];
  int64_t row[RIF];
  bool valid[RIF];
  auto load_x = [&](int64_t base) {
#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      row[i] = base + static_cast<int64_t>(slot) * RIF + i;
      valid[i] = row[i] < r_end;
      const uint4* xr = x + row[i] * V + lane;
#pragma unroll
      for (int j = 0; j < VPT; ++j) xv[i][j] = valid[i] ? load_stream(xr + j * lpr) : make_uint4(0, 0, 0, 0);
    }
  };
  // One iteration after its rows were requested; `it` picks the LDS buffer.
  auto process = [&](int it) {
    // per-lane two-pass (mean, M2), then the fixed-order merge across lanes
    float m[RIF], s[RIF];
#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        float f[EPV];
        E::unpack(xv[i][j], f);
#pragma unroll
        for (int k = 0; k < EPV; ++k) acc += f[k];
      }
      const float ml = div_count(acc, n_lane, 1.0f / n_lane);
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        float f[EPV];
        E::unpack(xv[i][j], f);
#pragma unroll
        for (int k = 0; k < EPV; ++k) { const float d = f[k] - ml; sq += d * d; }
      }
      m[i] = ml; s[i] = sq;
      chan_reduce_unit(m[i], s[i], n_lane, unit);
    }
    if (groups > 1) {
      float2* buf = lds_f2 + (it & 1) * buf_stride;
      if (leader) {
#pragma unroll
        for (int i = 0; i < RIF; ++i) buf[(slot * RIF + i) * groups + group] = make_float2(m[i], s[i]);
      }
      __syncthreads();
      const float n_unit = n_lane * static_cast<float>(unit);
#pragma unroll
      for (int i = 0; i < RIF; ++i) {
        const float2* p = buf + (slot * RIF + i) * groups;
        float2 v = p[0];
        float mm = v.x, ss = v.y, nn = n_unit;
        for (int g = 1; g < groups; ++g) { v = p[g]; chan_merge(mm, ss, nn, v.x, v.y, n_unit); }
        m[i] = mm; s[i] = ss;
      }
    }

#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      if (!valid[i]) continue;
      const float rs = 1.0f / sqrtf(s[i] * inv_d + eps);
      if (lane == 0) { mean[row[i]] = m[i]; rstd[row[i]] = rs; }
      if (row[i] >= cur_hi || row[i] < cur_lo) load_mod(row[i]);
      uint4* yr = y + row[i] * V + lane;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        float f[EPV];
        E::unpack(xv[i][j], f);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float xh = (f[k] - m[i]) * rs;      // (x - mean) * rstd
          f[k] = xh * sc1[j][k] + sh[j][k];
        }
        store_stream(yr + j * lpr, E::pack(f));
      }
    }
    };

  if constexpr (RIF > 1) {
    // Two rows per slot: typically one iteration per workgroup, so the first
    // rows and their sample's modulation are requested together (one memory
    // round trip instead of two; r_begin < R).
    load_x(r_begin);
    load_mod(r_begin);
    process(0);
    int it = 1;
    for (int64_t base = r_begin + rows_per_iter; base < r_end; base += rows_per_iter, ++it) {
      load_x(base);
      process(it);
    }
  } else {
    int it = 0;
    for (int64_t base = r_begin; base < r_end; base += rows_per_iter, ++it) {
      load_x(base);
      process(it);
    }
  }
}

// ---------------------------------------------------------------------------
// persistent forward, one wave per row
// ---------------------------------------------------------------------------
// For rows of 64 x VPT 16-byte vectors: a row is one wave (lane l holds
// vectors l, l + 64, ...), so its statistics need no LDS and no barrier.  A
// fixed grid of `active` waves (four per workgroup, about one workgroup per
// CU) walks the rows grid-stride: wave g takes rows g, g + active, ..., so
// every wave gets the same number of rows give or take one and the chip
// sweeps memory in a narrow window.  Each wave loads its next row while it
// reduces and writes the current one; the two row buffers alternate
// (unrolled by two) so no register copy waits on the prefetch.  Measured on
// MI355X: a plain copy of a 18900 x 5120 bf16 tensor runs best with ~16-20 KB
// of loads in flight per CU (6.2-6.4 TB/s) and slower with more, which is what
// this grid is shaped by; in a warm fwd+bwd step it ties the slot kernel on
// the video shape and is ~1% faster on D = 3072.
constexpr int WAVE_NT = 256;            // four waves per workgroup
constexpr int WAVE_MAX_VPT = 10;
constexpr int WAVE_MAX_ROWS = 32;       // beyond this many rows per wave the slot kernel wins

template <int DT, int VPT>
__global__ void __launch_bounds__(WAVE_NT)
fwd_wave_kernel(const uint4* __restrict__ x, const uint4* __restrict__ shift,
                const uint4* __restrict__ scale, float eps, RowMap rm, int D, int64_t active,
                uint4* __restrict__ y, float* __restrict__ mean, float* __restrict__ rstd) {
  using E = Elem<DT>;
  constexpr int EPV = E::EPV;
  constexpr int V = 64 * VPT;               // vectors per row
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (gw >= active) return;
  const int lane = threadIdx.x & 63;
  const int64_t last = rm.R - 1;
  const float inv_d = 1.0f / static_cast<float>(D);
  constexpr float n_lane = static_cast<float>(VPT * EPV);
  // Where the next row's loads are issued.  Wide rows (8 or more vectors per
  // lane) issue them right after the row sum, before the pass over the
  // squared deviations: that pass is long enough to delay the request, and
  // more so while the engine clock is low (first milliseconds of sustained
  // load).  Video shape, D = 5120, 20 steps after 5 warm-up steps: forward
  // 67.9 against 70.0-70.6 us, step 5,490-5,532 against 5,433-5,490 GB/s
  // over three interleaved runs; tied at the settled clock (67.4 against
  // 67.2 us).  Narrower rows keep the later point: D = 3072 forward 23.4
  // against 24.3 us.
  constexpr bool EARLY_PREFETCH = VPT >= 8;

  uint4 sc[VPT], sh[VPT];                   // the current sample's modulation, as stored
  int64_t cur_lo = 0, cur_hi = 0;
  // Past the last row the prefetch loads the last row again (always in
  // bounds) and nothing uses it: the loads are unconditional so the
  // compiler's wait counts stay exact and the prefetch stays in flight.
  auto load_row = [&](uint4 (&dst)[VPT], int64_t r) {
    const uint4* xr = x + (r < last ? r : last) * V + lane;
#pragma unroll
    for (int j = 0; j < VPT; ++j) dst[j] = load_stream(xr + j * 64);
  };
  auto step = [&](uint4 (&cur)[VPT], uint4 (&nxt)[VPT], int64_t r) {
    if (r >= cur_hi || r < cur_lo) {
      const int64_t b = sample_of_row(rm, r);
      cur_lo = rm.offsets ? clamp_row(rm.offsets[b], rm.R) : b * rm.N;
      cur_hi = rm.offsets ? clamp_row(rm.offsets[b + 1], rm.R) : cur_lo + rm.N;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        sc[j] = scale[b * V + lane + j * 64];
        sh[j] = shift[b * V + lane + j * 64];
      }
      // vmcnt(0): the reload settles inside its branch, so the common path
      // reaches the join with only the row loads and stores outstanding
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) acc = E::accumulate(cur[j], acc);
    const float ml = div_count(acc, n_lane, 1.0f / n_lane);
    if constexpr (EARLY_PREFETCH) {
      __builtin_amdgcn_sched_barrier(0);
      load_row(nxt, r + active);
      __builtin_amdgcn_sched_barrier(0);
    }
    float f[VPT][EPV];
#pragma unroll
    for (int j = 0; j < VPT; ++j) E::unpack(cur[j], f[j]);
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
      for (int k = 0; k < EPV; ++k) { const float d = f[j][k] - ml; sq += d * d; }
    float m = ml, s = sq;
    // Otherwise the next row's loads go out here, once this row's own pass
    // over its registers is done, and stay in flight through the reduction
    // and the output.
    if constexpr (!EARLY_PREFETCH) {
      __builtin_amdgcn_sched_barrier(0);
      load_row(nxt, r + active);
      __builtin_amdgcn_sched_barrier(0);
    }
    chan_reduce_wave(m, s, n_lane);
    const float rs = 1.0f / sqrtf(s * inv_d + eps);
    if (lane == 0) { mean[r] = m; rstd[r] = rs; }
    uint4* yr = y + r * V + lane;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      float a[EPV], h[EPV], o[EPV];
      E::unpack(sc[j], a);
      E::unpack(sh[j], h);
      // (x - mean) first: exact when x is near the mean (constant rows have
      // rstd = eps^-1/2, where x*rstd - mean*rstd would lose the digits)
#pragma unroll
      for (int k = 0; k < EPV; ++k) o[k] = __builtin_fmaf((f[j][k] - m) * rs, a[k] + 1.0f, h[k]);
      store_stream(yr + j * 64, E::pack(o));
    }
  };

  // The first row is peeled off so that every entry into the loop finds the
  // same memory operations outstanding (a prefetch into xb, then the stores):
  // otherwise the compiler merges the entry path into the loop head and
  // waits for everything there.
  uint4 xa[VPT], xb[VPT];
  load_row(xa, gw);
  step(xa, xb, gw);                         // gw < active <= R
  for (int64_t row = gw + active; row < rm.R; row += 2 * active) {
    step(xb, xa, row);
    if (row + active >= rm.R) break;
    step(xa, xb, row + active);
  }
}

// ---------------------------------------------------------------------------
// vectorised backward row pass
// ---------------------------------------------------------------------------
// Grid: one workgroup per tile (a run of rows inside one sample).
// LDS: 2 buffers x [slots][RIF][groups] x (sum g, sum g*xhat), then, when a
// workgroup holds several slots, [slots][D] floats for the slot combine.
// COLS = false compiles out the column partials: dx only (the first pass of
// the two-pass backward).
template <int DT, int VPT, int RIF, int NTMAX = VEC_MAX_NT, bool COLS = true, bool PACKED = false>
__global__ void __launch_bounds__(NTMAX)
bwd_vec_kernel(const uint4* __restrict__ dy, const uint4* __restrict__ x,
               const uint4* __restrict__ scale, const float* __restrict__ mean,
               const float* __restrict__ rstd, RowMap rm, Tiling tl, int V, int D, int lpr,
               float* __restrict__ partial, uint4* __restrict__ dx) {
  using E = Elem<DT>;
  constexpr int EPV = E::EPV;
  extern __shared__ float2 lds_f2[];

  const int64_t t = blockIdx.x;
  int64_t b, first, step, count;
  if (!tile_rows_of<PACKED>(rm, tl, t, b, first, step, count)) return;   // spare packed workgroup

  const int tid = threadIdx.x;
  const int nslots = blockDim.x / lpr;
  const int slot = tid / lpr;
  const int lane = tid - slot * lpr;
  const int unit = reduce_unit(lpr);
  const int groups = lpr / unit;
  const int group = lane / unit;
  const bool leader = (lane % unit) == 0;
  const int buf_stride = nslots * RIF * groups;
  const float inv_d = 1.0f / static_cast<float>(D);

  // The modulation row, requested first and unpacked after the first rows
  // are requested (below).
  uint4 sc_raw[VPT];
  {
    const uint4* scp = scale + b * V + lane;
#pragma unroll
    for (int j = 0; j < VPT; ++j) sc_raw[j] = scp[j * lpr];
  }
  float scl[VPT][EPV];
  float acc_h[VPT][EPV], acc_s[VPT][EPV];   // column partials of dy and dy*xhat
#pragma unroll
  for (int j = 0; j < VPT; ++j)
#pragma unroll
    for (int k = 0; k < EPV; ++k) { acc_h[j][k] = 0.f; acc_s[j][k] = 0.f; }

  // One iteration's rows: this slot takes tile rows m = base + slot*RIF + i.
  // Rows past the tile's end load the tile's first row instead (always
  // valid) and are then ignored.
  uint4 xv[RIF][VPT], gv[RIF][VPT];
  float mu[RIF], rs[RIF];
  auto load_rows = [&](int64_t base, uint4 (&xa)[RIF][VPT], uint4 (&ga)[RIF][VPT], float (&ma)[RIF],
                       float (&ra)[RIF]) {
#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      const int64_t m = base + static_cast<int64_t>(slot) * RIF + i;
      const int64_t rr = m < count ? first + m * step : first;
      ma[i] = mean[rr];
      ra[i] = rstd[rr];
      const uint4* xr = x + rr * V + lane;
      const uint4* gr = dy + rr * V + lane;
#pragma unroll
      for (int j = 0; j < VPT; ++j) { xa[i][j] = load_stream(xr + j * lpr); ga[i][j] = load_stream(gr + j * lpr); }
    }
  };

  const int64_t rows_per_iter = static_cast<int64_t>(nslots) * RIF;
  // One loop iteration after its rows were requested; `it` picks the LDS buffer.
  auto process = [&](int64_t base, int it) {

    float sg[RIF], sgx[RIF];
#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        float fx[EPV], fg[EPV];
        E::unpack(xv[i][j], fx);
        E::unpack(gv[i][j], fg);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float xh = (fx[k] - mu[i]) * rs[i];
          const float g = grad_g(fg[k], scl[j][k]);
          a += g;
          c = __builtin_fmaf(g, xh, c);
        }
      }
      sg[i] = sum_unit(a, unit);
      sgx[i] = sum_unit(c, unit);
    }
    if (groups > 1) {
      float2* buf = lds_f2 + (it & 1) * buf_stride;
      if (leader) {
#pragma unroll
        for (int i = 0; i < RIF; ++i) buf[(slot * RIF + i) * groups + group] = make_float2(sg[i], sgx[i]);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < RIF; ++i) {
        const float2* p = buf + (slot * RIF + i) * groups;
        float2 v = p[0];
        float a = v.x, c = v.y;
        for (int g = 1; g < groups; ++g) { v = p[g]; a += v.x; c += v.y; }
        sg[i] = a; sgx[i] = c;
      }
    }

#pragma unroll
    for (int i = 0; i < RIF; ++i) {
      const int64_t m = base + static_cast<int64_t>(slot) * RIF + i;
      if (m >= count) continue;
      const int64_t row = first + m * step;
      const RowGrad rg(sg[i], sgx[i], rs[i], inv_d);
      uint4* dxr = dx + row * V + lane;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        float fx[EPV], fg[EPV], out[EPV];
        E::unpack(xv[i][j], fx);
        E::unpack(gv[i][j], fg);
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          const float xh = (fx[k] - mu[i]) * rs[i];
          out[k] = rg.dx(grad_g(fg[k], scl[j][k]), xh);
          if (COLS) {
            acc_h[j][k] += fg[k];
            acc_s[j][k] = __builtin_fmaf(fg[k], xh, acc_s[j][k]);
          }
        }
        store_stream(dxr + j * lpr, E::pack(out));
      }
    }
  };
  // The first iteration is peeled: its rows are requested before the
  // modulation row is unpacked, so the two share one memory round trip (a
  // tile has at least one row).
  load_rows(0, xv, gv, mu, rs);
  __builtin_amdgcn_sched_barrier(0);   // every first-row load ahead of the wait below
#pragma unroll
  for (int j = 0; j < VPT; ++j) E::unpack(sc_raw[j], scl[j]);
  process(0, 0);
  int it = 1;
  for (int64_t base = rows_per_iter; base < count; base += rows_per_iter, ++it) {
    load_rows(base, xv, gv, mu, rs);
    process(base, it);
  }
  if (!COLS) return;

  // tile partials, chunk-major (see pidx)
  const int64_t TA = tl.tiles_alloc;
  if (nslots == 1) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int col = (j * lpr + lane) * EPV;
#pragma unroll
      for (int k = 0; k < EPV; k += 4) {
        *reinterpret_cast<float4*>(partial + pidx(TA, t, 0, col + k)) =
            make_float4(acc_h[j][k], acc_h[j][k + 1], acc_h[j][k + 2], acc_h[j][k + 3]);
        *reinterpret_cast<float4*>(partial + pidx(TA, t, 1, col + k)) =
            make_float4(acc_s[j][k], acc_s[j][k + 1], acc_s[j][k + 2], acc_s[j][k + 3]);
      }
    }
  } else {
    // Several slots: for each quantity, every slot stores its column sums to
    // LDS, then each thread adds a 4-column group over the slots in slot order
    // and writes the tile partial.  Two barriers per quantity, however many
    // slots.  A slot's D sums are stored as EPV/4 planes of V float4s (plane
    // h holds columns 4h..4h+3 of every 16-byte vector), so the lanes of a
    // wave store and load consecutive float4s: no LDS bank conflicts.
    float* comb = reinterpret_cast<float*>(lds_f2 + 2 * buf_stride);
    const int d4 = D / 4;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __syncthreads();                 // the reduction buffers / previous quantity are done
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int v = j * lpr + lane;
        const float* a = q == 0 ? acc_h[j] : acc_s[j];
#pragma unroll
        for (int h = 0; h < EPV / 4; ++h)
          *reinterpret_cast<float4*>(comb + slot * D + (h * V + v) * 4) =
              make_float4(a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]);
      }
      __syncthreads();
      for (int i = tid; i < d4; i += blockDim.x) {
        float4 v = *reinterpret_cast<const float4*>(comb + i * 4);
        for (int sl = 1; sl < nslots; ++sl) {
          const float4 w = *reinterpret_cast<const float4*>(comb + sl * D + i * 4);
          v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        const int h = i / V;
        const int col = (i - h * V) * EPV + h * 4;
        *reinterpret_cast<float4*>(partial + pidx(TA, t, q, col)) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward row pass for rows of whole waves
// ---------------------------------------------------------------------------
// Rows of W whole waves (LPR = 64*W lanes = the workgroup, VPT vectors per
// lane), one row at a time per workgroup, one workgroup per tile.  Per
// element: d = x - mean, xhat = d*rstd, g = dy*(1+scale) with one rounding
// (fma(dy, scale, dy)), the row sums of g and g*xhat, the column partials of
// dy and dy*xhat; after the row sums, dx = rstd*((g - a) - xhat*c) from the
// xhat and g kept in registers.  The row sums reach the wave's last lane
// through DPP (row broadcasts), the waves' sums meet in LDS and every lane
// adds them in wave order: one barrier per row, fixed order, bitwise
// repeatable.  The wave sums equal the slot kernel's butterfly sums bit for
// bit (the same pairs are added, only the operand order of commutative adds
// differs), so both kernels give the same dx for the same row.
//
// Against the slot kernel (which recomputes xhat and g from the stored row in
// its output pass) this takes about 290 instead of 350 instructions per row
// and lane at D = 5120 bf16, and it keeps its speed when the engine clock
// drops: on MI355X the clock falls to 1.6-1.8 GHz for ~2-20 ms after a
// sustained load starts (deeper the more ALU work per byte the kernels do),
// and there the video backward call takes ~106-108 us against ~114-118 us for
// the slot kernel (104-105 against 102 us at the settled 2.4 GHz).
// COLS = false leaves out the column partials (dx only: the first pass of the
// two-pass backward).

// Sum over a wave into its last lane (other lanes hold partial sums).
__device__ __forceinline__ float sum_to_last_lane(float v) {
  v = v + partner16<0>(v);
  v = v + partner16<1>(v);
  v = v + partner16<2>(v);
  v = v + partner16<3>(v);                  // every lane: its 16-lane row's sum
  // rows 1 and 3 add rows 0 and 2 (lane 15 of the row below), then rows 2 and
  // 3 add lane 31: lane 63 = (row3 + row2) + (row1 + row0)
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

constexpr int ROW_MAX_WAVES = VEC_MAX_NT / 64;

template <int DT, int VPT, bool COLS = true, bool PACKED = false>
__global__ void __launch_bounds__(VEC_MAX_NT)
bwd_row_kernel(const uint4* __restrict__ dy, const uint4* __restrict__ x,
               const uint4* __restrict__ scale, const float* __restrict__ mean,
               const float* __restrict__ rstd, RowMap rm, Tiling tl, int D,
               float* __restrict__ partial, uint4* __restrict__ dx) {
  using E = Elem<DT>;
  constexpr int EPV = E::EPV;
  const int LPR = blockDim.x;               // the row's lanes: W whole waves
  const int W = LPR >> 6;
  const int V = LPR * VPT;
  __shared__ float2 red[2][ROW_MAX_WAVES];

  const int64_t t = blockIdx.x;
  int64_t b, first, step, count;
  if (!tile_rows_of<PACKED>(rm, tl, t, b, first, step, count)) return;   // spare packed workgroup
  const int lane = threadIdx.x;
  const int wave = lane >> 6;
  const float inv_d = 1.0f / static_cast<float>(D);

  // the sample's scale, unpacked once (g = fma(dy, scale, dy))
  const uint4* mod = scale + b * V + lane;
  float scl[VPT][EPV];
#pragma unroll
  for (int j = 0; j < VPT; ++j) E::unpack(mod[j * LPR], scl[j]);
  float acc_h[VPT][EPV], acc_s[VPT][EPV];   // column partials of dy and dy*xhat
#pragma unroll
  for (int j = 0; j < VPT; ++j)
#pragma unroll
    for (int k = 0; k < EPV; ++k) { acc_h[j][k] = 0.f; acc_s[j][k] = 0.f; }

  const int64_t adv = step * V;             // vectors from one of the tile's rows to the next
  const uint4* xp = x + first * V + lane;
  const uint4* gp = dy + first * V + lane;
  uint4* dp = dx + first * V + lane;

  uint4 xv[VPT], gv[VPT];
  for (int64_t m = 0; m < count; ++m) {
    float mu, rs;
    {
      // The statistics go through vector loads (the offset is made opaque
      // in a vector register), issued with the row's own loads; as scalar
      // loads they would be waited for by the barrier's LDS wait.
      int64_t o = m * step;
      asm volatile("" : "+v"(o));
      mu = mean[first + o];
      rs = rstd[first + o];
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        xv[j] = load_stream(xp + m * adv + j * LPR);
        gv[j] = load_stream(gp + m * adv + j * LPR);
      }
    }
    float xh[VPT][EPV], g[VPT][EPV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      float d[EPV], fg[EPV];
      Center<DT>::apply(xv[j], -mu, d);
      E::unpack(gv[j], fg);
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        xh[j][k] = d[k] * rs;
        g[j][k] = grad_g(fg[k], scl[j][k]);
        s1 += g[j][k];
        s2 = __builtin_fmaf(g[j][k], xh[j][k], s2);
        if (COLS) {
          acc_h[j][k] += fg[k];
          acc_s[j][k] = __builtin_fmaf(fg[k], xh[j][k], acc_s[j][k]);
        }
      }
    }
    float a, c;
    if (W == 1) {
      a = sum_wave(s1);
      c = sum_wave(s2);
    } else {
      const int par = static_cast<int>(m & 1);
      s1 = sum_to_last_lane(s1);
      s2 = sum_to_last_lane(s2);
      if ((lane & 63) == 63) red[par][wave] = make_float2(s1, s2);
      __syncthreads();
      float2 v = red[par][0];
      a = v.x; c = v.y;
      for (int w = 1; w < W; ++w) { v = red[par][w]; a += v.x; c += v.y; }
    }
    const RowGrad rg(a, c, rs, inv_d);
    uint4* dr = dp + m * adv;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      float o[EPV];
#pragma unroll
      for (int k = 0; k < EPV; ++k) o[k] = rg.dx(g[j][k], xh[j][k]);
      store_stream(dr + j * LPR, E::pack(o));
    }
  }
  if constexpr (!COLS) return;

  // tile partials, chunk-major (see pidx)
  const int64_t TA = tl.tiles_alloc;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int col = (j * LPR + lane) * EPV;
#pragma unroll
    for (int k = 0; k < EPV; k += 4) {
      *reinterpret_cast<float4*>(partial + pidx(TA, t, 0, col + k)) =
          make_float4(acc_h[j][k], acc_h[j][k + 1], acc_h[j][k + 2], acc_h[j][k + 3]);
      *reinterpret_cast<float4*>(partial + pidx(TA, t, 1, col + k)) =
          make_float4(acc_s[j][k], acc_s[j][k + 1], acc_s[j][k + 2], acc_s[j][k + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// two-pass backward, second pass: D-tile column partials
// ---------------------------------------------------------------------------
// The backward's gradient reduction as the AdaptiveLoad summary lays it out
// (section 2.B, backward bullet): after a separate dx pass, a grid of
// (n_tile, d_tile) workgroups reads dy and x again; each thread is pinned to
// one 16-byte vector of columns and adds sum(dy) and sum(dy*xhat) down the
// rows of its tile, so the 64 lanes of a wave read one contiguous 1 KiB span
// of a row.  It writes the same chunk-major tile partials as the fused row
// pass, which gets them without the second read of dy and x; the two paths
// exist side by side to measure what the fusion saves.
// Grid: (tiles, ceil(V/64)); 256 threads = 4 waves.  Wave w adds the tile's
// rows w, w+4, w+8, ... in ascending order (DT_UNROLL rows' loads in flight),
// then the four wave sums are added in wave order.
constexpr int DT_WAVES = 4;
constexpr int DT_UNROLL = 4;

template <int DT>
__global__ void __launch_bounds__(64 * DT_WAVES)
dtile_cols_kernel(const uint4* __restrict__ dy, const uint4* __restrict__ x,
                  const float* __restrict__ mean, const float* __restrict__ rstd, RowMap rm,
                  Tiling tl, int V, float* __restrict__ partial) {
  using E = Elem<DT>;
  constexpr int EPV = E::EPV;
  __shared__ float red[DT_WAVES - 1][64][2 * EPV];
  const int64_t t = blockIdx.x;
  int64_t b, first, step, count;
  if (!tile_rows_of<false>(rm, tl, t, b, first, step, count)) return;   // dense batches only
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int v = blockIdx.y * 64 + lane;
  const bool on = v < V;

  float ah[EPV], as[EPV];
#pragma unroll
  for (int k = 0; k < EPV; ++k) { ah[k] = 0.f; as[k] = 0.f; }
  auto add_row = [&](const uint4& xv, const uint4& gv, float mu, float rs) {
    float fx[EPV], fg[EPV];
    E::unpack(xv, fx);
    E::unpack(gv, fg);
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const float xh = (fx[k] - mu) * rs;
      ah[k] += fg[k];
      as[k] += fg[k] * xh;
    }
  };
  if (on) {
    int64_t m = w;
    for (; m + (DT_UNROLL - 1) * DT_WAVES < count; m += DT_UNROLL * DT_WAVES) {
      uint4 xv[DT_UNROLL], gv[DT_UNROLL];
      float mu[DT_UNROLL], rs[DT_UNROLL];
#pragma unroll
      for (int u = 0; u < DT_UNROLL; ++u) {
        const int64_t row = first + (m + u * DT_WAVES) * step;
        mu[u] = mean[row];
        rs[u] = rstd[row];
        xv[u] = load_stream(x + row * V + v);
        gv[u] = load_stream(dy + row * V + v);
      }
#pragma unroll
      for (int u = 0; u < DT_UNROLL; ++u) add_row(xv[u], gv[u], mu[u], rs[u]);
    }
    for (; m < count; m += DT_WAVES) {
      const int64_t row = first + m * step;
      add_row(load_stream(x + row * V + v), load_stream(dy + row * V + v), mean[row], rstd[row]);
    }
  }
  if (w > 0) {
#pragma unroll
    for (int k = 0; k < EPV; ++k) { red[w - 1][lane][k] = ah[k]; red[w - 1][lane][EPV + k] = as[k]; }
  }
  __syncthreads();
  if (w == 0 && on) {
#pragma unroll
    for (int q = 0; q < DT_WAVES - 1; ++q)
#pragma unroll
      for (int k = 0; k < EPV; ++k) { ah[k] += red[q][lane][k]; as[k] += red[q][lane][EPV + k]; }
    const int64_t TA = tl.tiles_alloc;
    const int col = v * EPV;
#pragma unroll
    for (int k = 0; k < EPV; k += 4) {
      *reinterpret_cast<float4*>(partial + pidx(TA, t, 0, col + k)) =
          make_float4(ah[k], ah[k + 1], ah[k + 2], ah[k + 3]);
      *reinterpret_cast<float4*>(partial + pidx(TA, t, 1, col + k)) =
          make_float4(as[k], as[k + 1], as[k + 2], as[k + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// general kernels (any D, any alignment): scalar accesses, re-reads from cache
// ---------------------------------------------------------------------------
constexpr int GEN_NT = 256;

// Sum over the workgroup in a fixed order; every thread returns the same bits.
// `red` holds GEN_NT/64 floats; the caller alternates between two buffers.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = sum_unit(v, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < GEN_NT / 64; ++i) s += red[i];
  return s;
}

template <int DT>
__global__ void __launch_bounds__(GEN_NT)
fwd_gen_kernel(const void* __restrict__ x, const void* __restrict__ shift,
               const void* __restrict__ scale, float eps, RowMap rm, int D,
               int64_t rows_per_wg, void* __restrict__ y, float* __restrict__ mean,
               float* __restrict__ rstd) {
  using E = Elem<DT>;
  __shared__ float red[4][GEN_NT / 64];
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t r_end = min(rm.R, r_begin + rows_per_wg);
  int k = 0;
  for (int64_t r = r_begin; r < r_end; ++r) {
    const int64_t base = r * D;
    float a = 0.f;
    for (int d = threadIdx.x; d < D; d += GEN_NT) a += E::load1(x, base + d);
    const float mu = block_sum(a, red[(k++) & 3]) / static_cast<float>(D);
    float q = 0.f;
    for (int d = threadIdx.x; d < D; d += GEN_NT) { const float t = E::load1(x, base + d) - mu; q += t * t; }
    const float var = block_sum(q, red[(k++) & 3]) / static_cast<float>(D);
    const float rs = 1.0f / sqrtf(var + eps);
    if (threadIdx.x == 0) { mean[r] = mu; rstd[r] = rs; }
    const int64_t b = sample_of_row(rm, r);
    for (int d = threadIdx.x; d < D; d += GEN_NT) {
      const float xh = (E::load1(x, base + d) - mu) * rs;
      E::store1(y, base + d, xh * (1.0f + E::load1(scale, b * D + d)) + E::load1(shift, b * D + d));
    }
  }
}

// One workgroup per tile; column partials accumulate in the tile's slice of
// `partial`, each column owned by one thread for the whole tile.
template <int DT, bool PACKED>
__global__ void __launch_bounds__(GEN_NT)
bwd_gen_kernel(const void* __restrict__ dy, const void* __restrict__ x,
               const void* __restrict__ scale, const float* __restrict__ mean,
               const float* __restrict__ rstd, RowMap rm, Tiling tl, int D,
               float* __restrict__ partial, void* __restrict__ dx) {
  using E = Elem<DT>;
  __shared__ float red[4][GEN_NT / 64];
  const int64_t t = blockIdx.x;
  int64_t b, first, step, count;
  if (!tile_rows_of<PACKED>(rm, tl, t, b, first, step, count)) return;   // spare packed workgroup
  const int64_t TA = tl.tiles_alloc;
  for (int d = threadIdx.x; d < D; d += GEN_NT) {
    partial[pidx(TA, t, 0, d)] = 0.f;
    partial[pidx(TA, t, 1, d)] = 0.f;
  }
  const float inv_d = 1.0f / static_cast<float>(D);
  int k = 0;
  for (int64_t m = 0; m < count; ++m) {
    const int64_t r = first + m * step;
    const int64_t base = r * D;
    const float mu = mean[r], rs = rstd[r];
    float a = 0.f, c = 0.f;
    for (int d = threadIdx.x; d < D; d += GEN_NT) {
      const float xh = (E::load1(x, base + d) - mu) * rs;
      const float g = grad_g(E::load1(dy, base + d), E::load1(scale, b * D + d));
      a += g; c = __builtin_fmaf(g, xh, c);
    }
    a = block_sum(a, red[(k++) & 3]);
    c = block_sum(c, red[(k++) & 3]);
    const RowGrad rg(a, c, rs, inv_d);
    for (int d = threadIdx.x; d < D; d += GEN_NT) {
      const float xh = (E::load1(x, base + d) - mu) * rs;
      const float gy = E::load1(dy, base + d);
      E::store1(dx, base + d, rg.dx(grad_g(gy, E::load1(scale, b * D + d)), xh));
      partial[pidx(TA, t, 0, d)] += gy;
      partial[pidx(TA, t, 1, d)] = __builtin_fmaf(gy, xh, partial[pidx(TA, t, 1, d)]);
    }
  }
}

// ---------------------------------------------------------------------------
// finish: dshift[b,d] / dscale[b,d] = sum of sample b's tile partials
// ---------------------------------------------------------------------------
// Both variants add the tiles in an order fixed by the shape and the CU count
// alone, entirely in fp64, and round the result once to the output type, which is the template's DT: the I/O type, or F32 for callers that
// want fp32 column sums whatever the I/O type.  Bitwise repeatable, no
// atomics.  Measured alternatives on MI355X (video shape) and why they lost:
// one thread walking all tiles of its column (49 us, latency-bound); a
// cooperative grid sync (about 30 us per sync); a last-arriving-workgroup
// hand-off inside one kernel (46 us: each workgroup's device-scope release
// fence writes back its XCD's L2); groups-then-samples in two kernels (13 us).

// Tiles [t0, t1) of sample b (b uniform over the workgroup; every thread
// calls this).
__device__ __forceinline__ void sample_tiles(const RowMap& rm, const Tiling& tl, int64_t b,
                                             int64_t& t0, int64_t& t1) {
  if (rm.offsets == nullptr) {
    const int64_t tps = (rm.N + tl.tile_rows - 1) / tl.tile_rows;
    t0 = b * tps; t1 = t0 + tps;
  } else if (tl.tile_start == nullptr) {
    const WaveTiles w = wave_tile_table(rm, tl);
    t0 = lane_value(w.excl, static_cast<int>(b));
    t1 = lane_value(w.incl, static_cast<int>(b));
  } else {
    t0 = tl.tile_start[b]; t1 = tl.tile_start[b + 1];
  }
}

// Few samples: one 256-thread workgroup per (sample, 16-column chunk).  Thread
// (slice, lane) adds tiles slice, slice + 64, ... (ascending, 8 per round of
// loads, as many rounds as the sample has tiles) for 4 adjacent columns in
// fp64; the
// 64 slice sums are then added in a fixed two-level order (run r adds slices
// r, r+8, ..., r+56, then the 8 run sums are added in run order), still in
// fp64, so the only rounding of a column sum is the final one.  320
// workgroups on the video shape, every load issued up front over one
// contiguous run of partials: about one memory round trip.  The LDS arrays
// are component-major with consecutive lanes on consecutive doubles.
constexpr int NARROW_LANES = PCOLS / 4;                  // float4 lanes per chunk
constexpr int NARROW_SLICES = 256 / NARROW_LANES;        // 64
constexpr int NARROW_PER = 8;                            // tiles per slice
constexpr int NARROW_MAX_SAMPLES = 16;

template <int DT>
__global__ void __launch_bounds__(256)
finish_narrow_kernel(const float* __restrict__ partial, RowMap rm, Tiling tl, int D,
                     int col_blocks, void* __restrict__ dscale, void* __restrict__ dshift) {
  using E = Elem<DT>;
  constexpr int LANES = NARROW_LANES, NSLICE = NARROW_SLICES, PER = NARROW_PER;
  constexpr int RUNS = NSLICE / 8;
  constexpr int SPLANE = NSLICE * LANES;    // doubles per component plane of the slice sums
  __shared__ double sl_h[4][SPLANE];        // per-slice sums, component-major
  __shared__ double sl_s[4][SPLANE];
  // each component's plane of run sums is padded by 4 doubles so that the 32
  // threads of the last step, one per (component, quantity, lane), read
  // distinct banks
  constexpr int RUN_PLANE = RUNS * LANES + 4;
  __shared__ double run_h[4][RUN_PLANE];
  __shared__ double run_s[4][RUN_PLANE];
  const int64_t b = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - static_cast<int>(b * col_blocks);
  const int lane = threadIdx.x % LANES;
  const int slice = threadIdx.x / LANES;
  const int d = cb * PCOLS + lane * 4;
  int64_t t0, t1;
  sample_tiles(rm, tl, b, t0, t1);
  const bool col_ok = d < D;          // D % 4 == 0: the lane's 4 columns are all in or all out
  const float* base = partial + pidx(tl.tiles_alloc, 0, 0, cb * PCOLS) + lane * 4;

  double h[4] = {0.0, 0.0, 0.0, 0.0}, sc[4] = {0.0, 0.0, 0.0, 0.0};
  // PER tiles of the slice per round (their loads issued together); one
  // round covers NSLICE * PER = 512 tiles, more rounds follow in order
  for (int64_t r0 = t0; r0 < t1; r0 += NSLICE * PER) {
    float4 vh[PER], vs[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int64_t t = r0 + slice + u * NSLICE;
      if (col_ok && t < t1) {
        vh[u] = *reinterpret_cast<const float4*>(base + t * 2 * PCOLS);
        vs[u] = *reinterpret_cast<const float4*>(base + t * 2 * PCOLS + PCOLS);
      } else {
        vh[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        vs[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      h[0] += vh[u].x; h[1] += vh[u].y; h[2] += vh[u].z; h[3] += vh[u].w;
      sc[0] += vs[u].x; sc[1] += vs[u].y; sc[2] += vs[u].z; sc[3] += vs[u].w;
    }
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sl_h[w][slice * LANES + lane] = h[w];
    sl_s[w][slice * LANES + lane] = sc[w];
  }
  __syncthreads();
  if (slice < RUNS) {
    double a[4] = {0.0, 0.0, 0.0, 0.0}, c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < NSLICE / RUNS; ++q) {
      const int i = (slice + q * RUNS) * LANES + lane;
#pragma unroll
      for (int w = 0; w < 4; ++w) { a[w] += sl_h[w][i]; c[w] += sl_s[w][i]; }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      run_h[w][slice * LANES + lane] = a[w];
      run_s[w][slice * LANES + lane] = c[w];
    }
  }
  __syncthreads();
  // one output per thread: slices 0-3 add component `slice` of the shift
  // sums, slices 4-7 that of the scale sums, the runs in run order
  if (slice < 8 && col_ok) {
    const int w = slice & 3;
    const double* run = slice < 4 ? run_h[w] : run_s[w];
    double a = 0.0;
#pragma unroll
    for (int q = 0; q < RUNS; ++q) a += run[q * LANES + lane];
    E::store_sum(slice < 4 ? dshift : dscale, b * D + d + w, a);
  }
}

// Any number of samples and tiles, any D: one 256-thread workgroup per
// (sample, 64 columns); slice k adds tiles k, k+4, ... in ascending order
// (8 loads in flight per thread), then the 4 slices are added in ascending
// order.  Used for many-sample packed batches, whose samples have few tiles.
constexpr int TILES_COLS = 64;
constexpr int TILES_SLICES = 4;

template <int DT>
__global__ void __launch_bounds__(TILES_COLS * TILES_SLICES)
finish_tiles_kernel(const float* __restrict__ partial, RowMap rm, Tiling tl, int D, int col_blocks,
                    void* __restrict__ dscale, void* __restrict__ dshift) {
  using E = Elem<DT>;
  __shared__ double sh_h[TILES_SLICES][TILES_COLS];
  __shared__ double sh_s[TILES_SLICES][TILES_COLS];
  const int64_t b = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - static_cast<int>(b * col_blocks);
  const int lane = threadIdx.x % TILES_COLS;
  const int slice = threadIdx.x / TILES_COLS;
  const int d = cb * TILES_COLS + lane;
  int64_t t0, t1;
  sample_tiles(rm, tl, b, t0, t1);
  const int64_t TA = tl.tiles_alloc;
  double h = 0.0, s = 0.0;
  if (d < D) {
    const float* ph = partial + pidx(TA, 0, 0, d);     // tile t at ph[t * 2 * PCOLS]
    int64_t t = t0 + slice;
    for (; t + 7 * TILES_SLICES < t1; t += 8 * TILES_SLICES) {
      float vh[8], vs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        vh[u] = ph[(t + u * TILES_SLICES) * 2 * PCOLS];
        vs[u] = ph[(t + u * TILES_SLICES) * 2 * PCOLS + PCOLS];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) { h += static_cast<double>(vh[u]); s += static_cast<double>(vs[u]); }
    }
    for (; t < t1; t += TILES_SLICES) {
      h += static_cast<double>(ph[t * 2 * PCOLS]);
      s += static_cast<double>(ph[t * 2 * PCOLS + PCOLS]);
    }
  }
  sh_h[slice][lane] = h;
  sh_s[slice][lane] = s;
  __syncthreads();
  // slice 0 finishes the shift sums, slice 1 the scale sums
  if (slice < 2 && d < D) {
    const double (*sh)[TILES_COLS] = slice == 0 ? sh_h : sh_s;
    double v = sh[0][lane];
#pragma unroll
    for (int k = 1; k < TILES_SLICES; ++k) v += sh[k][lane];
    E::store_sum(slice == 0 ? dshift : dscale, b * D + d, v);
  }
}

// ---------------------------------------------------------------------------
// varlen prologue: tile_start[b] = sum_{c<b} ceil(rows_c / tile_rows)
// ---------------------------------------------------------------------------
constexpr int PRO_NT = 1024;

__global__ void __launch_bounds__(PRO_NT)
varlen_tiles_kernel(const int64_t* __restrict__ offsets, int64_t B, int64_t R, int64_t tile_rows,
                    int64_t tiles_alloc, int64_t* __restrict__ tile_start) {
  __shared__ int64_t scan[PRO_NT];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < B; base += PRO_NT) {
    const int64_t b = base + threadIdx.x;
    int64_t cnt = 0;
    if (b < B) {
      const int64_t n = clamped_span(offsets[b], offsets[b + 1], R).n;
      cnt = n > 0 ? (n + tile_rows - 1) / tile_rows : 0;
    }
    scan[threadIdx.x] = cnt;
    __syncthreads();
    // Hillis-Steele inclusive scan over the chunk
    for (int off = 1; off < PRO_NT; off <<= 1) {
      const int64_t v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    // exclusive, capped at the partials' tile capacity (reached only by a
    // malformed table whose samples overlap)
    if (b < B) tile_start[b] = min(carry + scan[threadIdx.x] - cnt, tiles_alloc);
    __syncthreads();
    if (threadIdx.x == PRO_NT - 1) carry += scan[PRO_NT - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_start[B] = min(carry, tiles_alloc);
}


// ---------------------------------------------------------------------------
// plans and launchers
// ---------------------------------------------------------------------------
// Forward grid: many short-lived workgroups keep the rows in flight inside a
// narrow window of memory; about 128 per CU, but at least two iterations each
// at one row per slot (measured with streaming accesses: video shape 73 us at
// two rows per workgroup against 76 at one; mixed-length batch at D = 3072
// 498 us at 128 per CU against 514 at 64 and 540 at 32).  At two rows per
// slot one iteration is enough (DiT, D = 1152: 8.1 us against 11.5 at two).
constexpr int FWD_WG_PER_CU = 128;
constexpr int FWD_MIN_ITERS = 2;

template <int DT, int VPT, int RIF>
static hipError_t fwd_vec_launch(const void* x, const void* shift, const void* scale, float eps,
                                 const RowMap& rm, int64_t D, const VecPlan& vp, int num_cu,
                                 hipStream_t stream, void* y, float* mean, float* rstd) {
  constexpr int EPV = Elem<DT>::EPV;
  const int V = static_cast<int>(D / EPV);
  const int nslots = vp.nt / vp.lpr;
  const size_t lds = vec_lds_bytes(vp, D, false);
  const int64_t per_iter = static_cast<int64_t>(nslots) * RIF;
  const int64_t target = static_cast<int64_t>(num_cu) * FWD_WG_PER_CU;
  int64_t rows_per_wg = (rm.R + target - 1) / target;
  rows_per_wg = ((rows_per_wg + per_iter - 1) / per_iter) * per_iter;
  const int64_t min_iters = RIF > 1 ? 1 : FWD_MIN_ITERS;
  if (rows_per_wg < min_iters * per_iter) rows_per_wg = min_iters * per_iter;
  const int64_t grid = (rm.R + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((fwd_vec_kernel<DT, VPT, RIF>), dim3(static_cast<unsigned>(grid)),
                     dim3(vp.nt), lds, stream, static_cast<const uint4*>(x),
                     static_cast<const uint4*>(shift), static_cast<const uint4*>(scale), eps, rm, V,
                     static_cast<int>(D), vp.lpr, rows_per_wg, static_cast<uint4*>(y), mean, rstd);
  return hipGetLastError();
}

// Backward row kernel launch: rows of vp.lpr lanes (whole waves, one row slot
// per workgroup), one workgroup per tile.
template <int DT, int VPT, bool COLS>
static hipError_t bwd_row_launch(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd, const RowMap& rm,
                                 int64_t D, const VecPlan& vp, const Tiling& tl, float* partial,
                                 hipStream_t stream, void* dx) {
#define ADALN_ROW_LAUNCH(P)                                                                        \
  hipLaunchKernelGGL((bwd_row_kernel<DT, VPT, COLS, P>), dim3(static_cast<unsigned>(tl.tiles_max)), \
                     dim3(vp.lpr), 0, stream, static_cast<const uint4*>(dy),                      \
                     static_cast<const uint4*>(x), static_cast<const uint4*>(scale), mean, rstd, rm, \
                     tl, static_cast<int>(D), partial, static_cast<uint4*>(dx))
  if constexpr (COLS) {        // dx-only passes (the two-pass backward) take dense batches only
    if (rm.offsets != nullptr) {
      ADALN_ROW_LAUNCH(true);
      return hipGetLastError();
    }
  }
  ADALN_ROW_LAUNCH(false);
#undef ADALN_ROW_LAUNCH
  return hipGetLastError();
}

template <int DT, int VPT, bool COLS = true>
static hipError_t bwd_vec_launch(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd, const RowMap& rm,
                                 int64_t D, const VecPlan& vp, const Tiling& tl, float* partial,
                                 hipStream_t stream, void* dx) {
  constexpr int EPV = Elem<DT>::EPV;
  constexpr int RIF = BWD_RIF;
  const int V = static_cast<int>(D / EPV);
  const size_t lds = vec_lds_bytes(vp, D, true);
#define ADALN_VEC_LAUNCH(P)                                                                         \
  hipLaunchKernelGGL((bwd_vec_kernel<DT, VPT, RIF, VEC_MAX_NT, COLS, P>),                          \
                     dim3(static_cast<unsigned>(tl.tiles_max)), dim3(vp.nt), lds, stream,          \
                     static_cast<const uint4*>(dy), static_cast<const uint4*>(x),                  \
                     static_cast<const uint4*>(scale), mean, rstd, rm, tl, V, static_cast<int>(D), \
                     vp.lpr, partial, static_cast<uint4*>(dx))
  if constexpr (COLS) {        // dx-only passes (the two-pass backward) take dense batches only
    if (rm.offsets != nullptr) {
      ADALN_VEC_LAUNCH(true);
      return hipGetLastError();
    }
  }
  ADALN_VEC_LAUNCH(false);
#undef ADALN_VEC_LAUNCH
  return hipGetLastError();
}

// Vectors per lane for the persistent forward: a row of 64 x VPT vectors with
// VPT <= WAVE_MAX_VPT, else 0 (the slot kernel).  Measured in a warm fwd+bwd
// step, the persistent kernel gains on such rows (MMDiT, D = 3072: 83.4
// against 84.4 us per step) or ties (video, D = 5120: 170.8 against 171.0),
// while rows of 16 or 32 lanes, several per wave, were faster on the slot
// kernel (DiT, D = 1152: 31.5 against 32.0 us per step).
static int wave_vpt(int dtype, int64_t D) {
  const int epv = dtype == BF16 ? 8 : 4;
  if (D <= 0 || D % epv != 0) return 0;
  const int64_t V = D / epv;
  return (V % 64 == 0 && V / 64 <= WAVE_MAX_VPT) ? static_cast<int>(V / 64) : 0;
}

template <int DT>
static hipError_t fwd_wave_launch(const void* x, const void* shift, const void* scale, float eps,
                                  const RowMap& rm, int64_t D, int vpt, int64_t active,
                                  hipStream_t stream, void* y, float* mean, float* rstd) {
  const int64_t grid = (active + WAVE_NT / 64 - 1) / (WAVE_NT / 64);
#define ADALN_WAVE_CASE(N)                                                                          \
  case N:                                                                                          \
    hipLaunchKernelGGL((fwd_wave_kernel<DT, N>), dim3(static_cast<unsigned>(grid)), dim3(WAVE_NT), \
                       0, stream, static_cast<const uint4*>(x), static_cast<const uint4*>(shift),  \
                       static_cast<const uint4*>(scale), eps, rm, static_cast<int>(D), active,     \
                       static_cast<uint4*>(y), mean, rstd);                                        \
    break;
  switch (vpt) {
    ADALN_WAVE_CASE(1) ADALN_WAVE_CASE(2) ADALN_WAVE_CASE(3) ADALN_WAVE_CASE(4) ADALN_WAVE_CASE(5)
    ADALN_WAVE_CASE(6) ADALN_WAVE_CASE(7) ADALN_WAVE_CASE(8) ADALN_WAVE_CASE(9) ADALN_WAVE_CASE(10)
    default: return hipErrorInvalidValue;
  }
#undef ADALN_WAVE_CASE
  return hipGetLastError();
}

template <int DT>
static hipError_t fwd_dispatch(const void* x, const void* shift, const void* scale, float eps,
                               const RowMap& rm, int64_t D, bool vec, const VecPlan& vp,
                               int num_cu, hipStream_t stream, void* y, float* mean, float* rstd) {
  if (vec) {
    // The persistent wave kernel when each of ~4 waves per CU gets at most
    // WAVE_MAX_ROWS rows; the active wave count is trimmed so the rows divide
    // as evenly as possible.
    const int wvpt = wave_vpt(DT, D);
    if (wvpt > 0) {
      const int64_t cap = static_cast<int64_t>(num_cu) * (WAVE_NT / 64);
      const int64_t per = (rm.R + cap - 1) / cap;
      if (per <= WAVE_MAX_ROWS) {
        const int64_t active = (rm.R + per - 1) / per;
        return fwd_wave_launch<DT>(x, shift, scale, eps, rm, D, wvpt, active, stream, y, mean, rstd);
      }
    }
    static_assert(FWD_RIF2_MAX_VPT == 3, "two-row slots are instantiated for VPT 1..3");
    const bool two = vp.rif == 2 && vp.vpt <= FWD_RIF2_MAX_VPT;
    if (vp.rif != 1 && !two) return hipErrorInvalidValue;
    switch (vp.vpt) {
      case 1: return two ? fwd_vec_launch<DT, 1, 2>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd)
                         : fwd_vec_launch<DT, 1, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 2: return two ? fwd_vec_launch<DT, 2, 2>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd)
                         : fwd_vec_launch<DT, 2, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 3: return two ? fwd_vec_launch<DT, 3, 2>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd)
                         : fwd_vec_launch<DT, 3, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 4: return fwd_vec_launch<DT, 4, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 5: return fwd_vec_launch<DT, 5, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 6: return fwd_vec_launch<DT, 6, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 7: return fwd_vec_launch<DT, 7, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      case 8: return fwd_vec_launch<DT, 8, 1>(x, shift, scale, eps, rm, D, vp, num_cu, stream, y, mean, rstd);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t target = static_cast<int64_t>(num_cu) * 8;
  const int64_t rows_per_wg = (rm.R + target - 1) / target;
  const int64_t grid = (rm.R + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((fwd_gen_kernel<DT>), dim3(static_cast<unsigned>(grid)), dim3(GEN_NT), 0,
                     stream, x, shift, scale, eps, rm, static_cast<int>(D), rows_per_wg, y, mean,
                     rstd);
  return hipGetLastError();
}

// The vectorised backward row pass (dx, and the tile partials when COLS):
// the row kernel for rows of whole waves, else the slot kernel.  The fused
// and the two-pass backward both come through here, so their dx is the same.
template <int DT, bool COLS>
static hipError_t bwd_rows(const void* dy, const void* x, const void* scale, const float* mean,
                           const float* rstd, const RowMap& rm, int64_t D, const VecPlan& vp,
                           const Tiling& tl, float* partial, hipStream_t stream, void* dx) {
  const bool row = vp.nt == vp.lpr && vp.lpr % 64 == 0;
#define ADALN_ROWS_CASE(N)                                                                         \
  case N:                                                                                          \
    return row ? bwd_row_launch<DT, N, COLS>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial,    \
                                             stream, dx)                                           \
               : bwd_vec_launch<DT, N, COLS>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial,    \
                                             stream, dx);
  switch (vp.vpt) {
    ADALN_ROWS_CASE(1) ADALN_ROWS_CASE(2) ADALN_ROWS_CASE(3) ADALN_ROWS_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef ADALN_ROWS_CASE
}

template <int DT>
static hipError_t bwd_gen_launch(const void* dy, const void* x, const void* scale,
                                 const float* mean, const float* rstd, const RowMap& rm,
                                 int64_t D, const Tiling& tl, float* partial, hipStream_t stream,
                                 void* dx) {
  if (rm.offsets != nullptr)
    hipLaunchKernelGGL((bwd_gen_kernel<DT, true>), dim3(static_cast<unsigned>(tl.tiles_max)),
                       dim3(GEN_NT), 0, stream, dy, x, scale, mean, rstd, rm, tl,
                       static_cast<int>(D), partial, dx);
  else
    hipLaunchKernelGGL((bwd_gen_kernel<DT, false>), dim3(static_cast<unsigned>(tl.tiles_max)),
                       dim3(GEN_NT), 0, stream, dy, x, scale, mean, rstd, rm, tl,
                       static_cast<int>(D), partial, dx);
  return hipGetLastError();
}

template <int DT>
static hipError_t finish_launch(const RowMap& rm, int64_t D, const Tiling& tl,
                                const float* partial, hipStream_t stream, void* dscale,
                                void* dshift);

// The packed batch's tile table: batches of at most PACKED_FEW_SAMPLES
// samples rebuild it wave by wave inside the kernels (tile_start = nullptr
// tells them so), larger ones get it from the prologue kernel.
static hipError_t varlen_tile_table(const RowMap& rm, Tiling& tl, hipStream_t stream) {
  if (rm.offsets == nullptr) return hipSuccess;
  if (rm.B <= PACKED_FEW_SAMPLES) {
    tl.tile_start = nullptr;
    return hipSuccess;
  }
  hipLaunchKernelGGL(varlen_tiles_kernel, dim3(1), dim3(PRO_NT), 0, stream, rm.offsets, rm.B,
                     rm.R, tl.tile_rows, tl.tiles_alloc, tl.tile_start);
  return hipGetLastError();
}

template <int DT>
static hipError_t bwd_dispatch(const void* dy, const void* x, const void* scale,
                               const float* mean, const float* rstd, const RowMap& rm, int64_t D,
                               bool vec, const VecPlan& vp, const Tiling& tl_in, float* partial,
                               hipStream_t stream, void* dx, void* dscale, void* dshift,
                               bool sums_f32) {
  Tiling tl = tl_in;
  hipError_t e = varlen_tile_table(rm, tl, stream);
  if (e != hipSuccess) return e;
  if (rm.R > 0 && tl.tiles_max > 0) {
    e = vec ? bwd_rows<DT, true>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial, stream, dx)
            : bwd_gen_launch<DT>(dy, x, scale, mean, rstd, rm, D, tl, partial, stream, dx);
    if (e != hipSuccess) return e;
  }
  return sums_f32 ? finish_launch<F32>(rm, D, tl, partial, stream, dscale, dshift)
                  : finish_launch<DT>(rm, D, tl, partial, stream, dscale, dshift);
}

// finish: the narrow kernel for few samples (any number of tiles each), else
// one workgroup per (sample, 64 columns)
template <int DT>
static hipError_t finish_launch(const RowMap& rm, int64_t D, const Tiling& tl,
                                const float* partial, hipStream_t stream, void* dscale,
                                void* dshift) {
  if (D % 4 == 0 && rm.B <= NARROW_MAX_SAMPLES) {
    const int col_blocks = static_cast<int>((D + PCOLS - 1) / PCOLS);
    hipLaunchKernelGGL((finish_narrow_kernel<DT>), dim3(static_cast<unsigned>(rm.B * col_blocks)),
                       dim3(256), 0, stream, partial, rm, tl, static_cast<int>(D), col_blocks,
                       dscale, dshift);
  } else {
    const int col_blocks = static_cast<int>((D + TILES_COLS - 1) / TILES_COLS);
    hipLaunchKernelGGL((finish_tiles_kernel<DT>), dim3(static_cast<unsigned>(rm.B * col_blocks)),
                       dim3(TILES_COLS * TILES_SLICES), 0, stream, partial, rm, tl,
                       static_cast<int>(D), col_blocks, dscale, dshift);
  }
  return hipGetLastError();
}

// Two-pass backward (vectorised shapes only): dx rows, then D-tile column
// partials over contiguous sequence chunks, then the same finish.
template <int DT>
static hipError_t bwd_twopass_dispatch(const void* dy, const void* x, const void* scale,
                                       const float* mean, const float* rstd, const RowMap& rm,
                                       int64_t D, const VecPlan& vp, const Tiling& tl_in,
                                       float* partial, hipStream_t stream, void* dx,
                                       void* dscale, void* dshift) {
  if (rm.offsets != nullptr) return hipErrorInvalidValue;   // dense batches only
  const Tiling& tl = tl_in;
  hipError_t e = hipSuccess;
  if (rm.R > 0 && tl.tiles_max > 0) {
    e = bwd_rows<DT, false>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial, stream, dx);
    if (e != hipSuccess) return e;
    const int V = static_cast<int>(D / Elem<DT>::EPV);
    Tiling chunks = tl;
    chunks.interleave = 0;
    hipLaunchKernelGGL((dtile_cols_kernel<DT>),
                       dim3(static_cast<unsigned>(tl.tiles_max), static_cast<unsigned>((V + 63) / 64)),
                       dim3(64 * DT_WAVES), 0, stream, static_cast<const uint4*>(dy),
                       static_cast<const uint4*>(x), mean, rstd, rm, chunks, V, partial);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return finish_launch<DT>(rm, D, tl, partial, stream, dscale, dshift);
}

hipError_t launch_fwd(int dtype, const void* x, const void* shift, const void* scale, float eps,
                      const RowMap& rm, int64_t D, bool vec, const VecPlan& vp, int num_cu,
                      hipStream_t stream, void* y, float* mean, float* rstd) {
  if (rm.R == 0) return hipSuccess;
  return dtype == BF16
             ? fwd_dispatch<BF16>(x, shift, scale, eps, rm, D, vec, vp, num_cu, stream, y, mean, rstd)
             : fwd_dispatch<F32>(x, shift, scale, eps, rm, D, vec, vp, num_cu, stream, y, mean, rstd);
}

hipError_t launch_bwd_twopass(int dtype, const void* dy, const void* x, const void* scale,
                              const float* mean, const float* rstd, const RowMap& rm, int64_t D,
                              const VecPlan& vp, const Tiling& tl, float* partial,
                              hipStream_t stream, void* dx, void* dscale, void* dshift) {
  return dtype == BF16
             ? bwd_twopass_dispatch<BF16>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial, stream, dx, dscale, dshift)
             : bwd_twopass_dispatch<F32>(dy, x, scale, mean, rstd, rm, D, vp, tl, partial, stream, dx, dscale, dshift);
}

hipError_t launch_bwd(int dtype, const void* dy, const void* x, const void* scale,
                      const float* mean, const float* rstd, const RowMap& rm, int64_t D,
                      bool vec, const VecPlan& vp, const Tiling& tl, float* partial,
                      hipStream_t stream, void* dx, void* dscale, void* dshift, bool sums_f32) {
  return dtype == BF16
             ? bwd_dispatch<BF16>(dy, x, scale, mean, rstd, rm, D, vec, vp, tl, partial, stream, dx, dscale, dshift, sums_f32)
             : bwd_dispatch<F32>(dy, x, scale, mean, rstd, rm, D, vec, vp, tl, partial, stream, dx, dscale, dshift, sums_f32);
}

}  // namespace adaln
