// Device building blocks for the gfx950 GDN kernels: MFMA wrappers, the
// register-resident tile conventions, and small wave-level helpers.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16, and eight chained
// v_mfma_f32_16x16x4_f32 for the fp32 path).  With lane l, r = l % 16, q = l / 16:
//   * a 16x16 fp32 accumulator tile holds element (row 4q+i, col r) in slot i;
//   * an A operand ("frag") holds row r of A and 8 values of the contraction
//     index, element e; a B operand holds column r of B and 8 values, element e;
//     A's (q, e) meets B's (q, e) in the product.
// A 32-wide contraction step therefore pairs A[row][phys(q,e)] with
// B[phys(q,e)][col] for any bijection phys; we always use phys(q,e) = 8q + e,
// which makes every LDS fragment read 8 contiguous elements.
//
// Register-resident operands.  A result tile can feed the next product as its B
// operand without leaving registers if the result's rows are numbered so that
// (tile 2s+e/4, slot e%4) of lane group q is contraction index 32s + 8q + e.  So
// every row dimension that is later contracted (chunk rows, key dimension)
// lives in "tile order": slot i of lane group q in tile t is physical row
//     prow(t, 4q+i),  prow(t, r) = 32*(t/2) + 8*(r/4) + 4*(t%2) + r%4.
// An A operand that produces tile t must then supply, in lane row r, the
// source row prow(t, r).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int prow(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}
// Inverse of prow: the tile-order slot 16 t + r that holds physical row R.  Tiles
// staged in LDS in this order make every fragment read touch 16 consecutive LDS
// rows, which (with a row stride of 8 mod 32 dwords) is free of bank conflicts.
__host__ __device__ constexpr int tord(int R) {
  return 16 * (2 * (R >> 5) + ((R >> 2) & 1)) + 4 * ((R & 31) >> 3) + (R & 3);
}

template <typename E>
struct Mma;

template <>
struct Mma<bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 run(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // B operand of contraction step s from result tiles 2s (lo) and 2s+1 (hi)
  static __device__ __forceinline__ frag pack(const f32x4& lo, const f32x4& hi) {
    frag r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
  }
};

template <>
struct Mma<float> {
  typedef f32x8 frag;
  static __device__ __forceinline__ f32x4 run(const frag& a, const frag& b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ frag pack(const f32x4& lo, const f32x4& hi) {
    frag r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
};

// Fragment read from a row-major LDS matrix: row `row`, columns kbase+8q .. +7.
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag lds_frag(const E* base, int stride, int row,
                                                          int kbase, int q) {
  return *reinterpret_cast<const typename Mma<E>::frag*>(base + row * stride + kbase + 8 * q);
}

// Column read of a row-major LDS matrix M: for the lane with index j inside its
// 16-lane group, returns M[row0 + i][colmap(j)], i = 0..3, where the 16 columns
// of a group form four runs of four, colmap(j) = base(j / 4) + j % 4, base()
// 4-element aligned.  Every lane of a group passes the same row0.
//   own_col    = colmap(j) of this lane (used by the fp32 form)
//   supply_col = base(j % 4)  (used by the bf16 form)
// bf16: one ds_read_b64_tr_b16.  Inside a 16-lane group, lane j receives element
// j % 4 of the 8-byte chunks addressed by lanes 4i + j / 4 (i = 0..3), so lane j'
// addresses M[row0 + j'/4][base(j'%4)].  fp32: four plain reads.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 col_read4(const bf16* M, int stride, int row0, int own_col,
                                           int supply_col) {
  (void)own_col;
  const int j = threadIdx.x & 15;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const bf16* addr = M + (row0 + (j >> 2)) * stride + supply_col;
  const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(addr));
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __uint_as_float(((uint32_t)(uint16_t)raw[i]) << 16);
  return r;
}

__device__ __forceinline__ f32x4 col_read4(const float* M, int stride, int row0, int own_col,
                                           int supply_col) {
  (void)supply_col;
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = M[(row0 + i) * stride + own_col];
  return r;
}

// Same column read returning the raw storage elements (to build MFMA operands).
__device__ __forceinline__ i16x4 col_read4_raw(const bf16* M, int stride, int row0, int own_col,
                                               int supply_col) {
  (void)own_col;
  const int j = threadIdx.x & 15;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const bf16* addr = M + (row0 + (j >> 2)) * stride + supply_col;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(addr));
}

// A/B operand of one 32-wide contraction step whose 8 elements are column reads
// at rows row_lo .. row_lo+3 (elements 0-3) and row_hi .. row_hi+3 (elements 4-7).
__device__ __forceinline__ bf16x8 col_frag(const bf16* M, int stride, int row_lo, int row_hi,
                                           int own_col, int supply_col) {
  const i16x4 lo = col_read4_raw(M, stride, row_lo, own_col, supply_col);
  const i16x4 hi = col_read4_raw(M, stride, row_hi, own_col, supply_col);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x8 col_frag(const float* M, int stride, int row_lo, int row_hi,
                                          int own_col, int supply_col) {
  (void)supply_col;
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = M[(row_lo + i) * stride + own_col];
    r[4 + i] = M[(row_hi + i) * stride + own_col];
  }
  return r;
}

// Stores 8 consecutive elements: lo = elements 0..3, hi = 4..7 (raw storage).
__device__ __forceinline__ void store8(bf16* dst, i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  *reinterpret_cast<i16x8*>(dst) = v;
}
__device__ __forceinline__ void store8(float* dst, f32x4 lo, f32x4 hi) {
  reinterpret_cast<f32x4*>(dst)[0] = lo;
  reinterpret_cast<f32x4*>(dst)[1] = hi;
}
__device__ __forceinline__ i16x4 col_read4_storage(const bf16* M, int stride, int row0, int own_col,
                                                   int supply_col) {
  return col_read4_raw(M, stride, row0, own_col, supply_col);
}
__device__ __forceinline__ f32x4 col_read4_storage(const float* M, int stride, int row0,
                                                   int own_col, int supply_col) {
  return col_read4(M, stride, row0, own_col, supply_col);
}

// The bf16 residuals x - bf16(x) of the eight values Mma<bf16>::pack(lo, hi) rounds:
// an operand carried as the pair (pack, pack_residual) keeps about 16 significant
// bits, at the cost of a second product.
__device__ __forceinline__ bf16x8 pack_residual(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (bf16)(lo[i] - (float)(bf16)lo[i]);
    r[4 + i] = (bf16)(hi[i] - (float)(bf16)hi[i]);
  }
  return r;
}
// Four fp32 values as four bf16 (round to nearest even) in two dwords.
__device__ __forceinline__ uint2 pack_bf16x4(const f32x4& v) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (bf16)v[i];
  return __builtin_bit_cast(uint2, b);
}

// Four consecutive elements of one row from fp32: 8 bytes (bf16) or 16 bytes (fp32).
__device__ __forceinline__ void store4(bf16* dst, const f32x4& v) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4*>(dst) = b;
}
__device__ __forceinline__ void store4(float* dst, const f32x4& v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ float load_scalar(const void* p, int64_t i, bool is_bf16) {
  return is_bf16 ? (float)reinterpret_cast<const bf16*>(p)[i] : reinterpret_cast<const float*>(p)[i];
}

__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Fragment-ordered storage of a DK x DK bf16 matrix used as MFMA A operands (the
// merge's M): the 16-byte operand of lane l = 16 q + r for row tile rt and
// contraction step s (row 16 rt + r, columns 32 s + 8 q .. +7) sits at element
// ((rt * DK/32 + s) * 64 + l) * 8, so one wave's operand load is 1 KB contiguous.
template <int DK>
__device__ __forceinline__ int64_t mfrag_offset(int row, int col) {
  return ((int64_t)((row >> 4) * (DK / 32) + (col >> 5)) * 64 + 16 * ((col & 31) >> 3) + (row & 15)) * 8 +
         (col & 7);
}

// Accumulator-ordered storage of a DK x dv fp32 matrix read as 16x16 MFMA D tiles
// (the merge's S*): lane l = 16 q + r of row tile rt, column tile ct holds rows
// 16 rt + 4 q + i (i = 0..3) of column 16 ct + r, at float ((ct * DK/16 + rt) * 64
// + l) * 4 + i, so one tile is a 1 KB contiguous 16-byte-per-lane load.
template <int DK>
__device__ __forceinline__ int64_t sfrag_offset(int row, int col) {
  return ((int64_t)((col >> 4) * (DK / 16) + (row >> 4)) * 64 + 16 * ((row & 15) >> 2) + (col & 15)) * 4 +
         (row & 3);
}

// Inclusive prefix sum over the 64 lanes of a wave without LDS traffic: DPP row
// shifts scan each 16-lane row (lanes without a source add 0), then the row totals
// are carried with v_readlane.
__device__ __forceinline__ float wave_inclusive_scan_dpp(float x) {
  const int lane = threadIdx.x & 63;
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = lane >> 4;
  const float c1 = r0, c2 = r0 + r1, c3 = r0 + r1 + r2;
  return x + (row == 0 ? 0.f : row == 1 ? c1 : row == 2 ? c2 : c3);
}

// Order-preserving float <-> uint encoding (for atomic max of floats); 0 is
// below every encoded float and marks "unset".
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Smallest admissible lookback window (chunks) of (sequence, head) nh from the
// gate-scan maxima; 0 if none.  The 16 maxima are loaded at once (64 bytes, 16-byte
// aligned) and searched in registers: a load per candidate behind the early exit
// would cost one memory latency per window length tried.
__device__ __forceinline__ int window_of(const uint32_t* best, int nh, int nch, int wmax,
                                         float thr) {
  static_assert(kWindowMaxCap == 16, "one 64-byte row of maxima per (sequence, head)");
  const uint4* row = reinterpret_cast<const uint4*>(best + (int64_t)nh * kWindowMaxCap);
  uint32_t u[kWindowMaxCap];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 x = row[i];
    u[4 * i] = x.x; u[4 * i + 1] = x.y; u[4 * i + 2] = x.z; u[4 * i + 3] = x.w;
  }
  const int lim = min(wmax, nch);
  int found = 0;
#pragma unroll
  for (int w = kWindowMaxCap; w >= 1; --w)   // the smallest admissible w wins
    if (w <= lim && u[w - 1] != 0u && from_ordered_bits(u[w - 1]) <= thr) found = w;
  return found;
}

// Largest gate sum over every run of w consecutive chunks (w = 1..wmax) of one
// (sequence, head), from its chunk gate sums csum[(chunk0 + c) * H + h], computed by a
// whole workgroup of NT threads (every thread must call it).  sums: LDS scratch of
// cap floats (cap > kWindowMaxCap); red: LDS scratch of NT / 64 * kWindowMaxCap
// floats.  Thread t < kWindowMaxCap returns the maximum for w = t + 1 (-inf: no run
// of that length); the other threads return -inf.
//
// The 16 per-lane maxima are reduced over the wave by a halving butterfly: at the
// exchange with lane ^ d (d = 32, 16, 8, 4) a lane keeps half of its windows (the
// upper half if bit d of its lane is set) and sends the other half, so the wave
// needs 8 + 4 + 2 + 1 + 2 shuffles instead of 16 x 6; afterwards lanes 4w .. 4w+3
// hold window w + 1.
template <int NT>
__device__ float block_run_max(const float* csum, int64_t chunk0, int nch, int H, int h, int wmax,
                               float* sums, int cap, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pass = cap - kWindowMaxCap;   // run starts per pass
  float mx[kWindowMaxCap];
#pragma unroll
  for (int w = 0; w < kWindowMaxCap; ++w) mx[w] = -INFINITY;
  for (int cs = 0; cs < nch; cs += pass) {
    __syncthreads();   // the previous pass (or the caller) is done with sums[]
    for (int i = tid; i < pass + wmax - 1; i += NT) {
      const int c = cs + i;
      sums[i] = c < nch ? csum[(chunk0 + c) * H + h] : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < pass; i += NT) {
      const int c = cs + i;
      float acc = 0.f;
#pragma unroll
      for (int w = 1; w <= kWindowMaxCap; ++w) {
        if (w <= wmax) {
          acc += sums[i + w - 1];
          if (c + w <= nch) mx[w - 1] = fmaxf(mx[w - 1], acc);
        }
      }
    }
  }
  // halving butterfly over the wave (see above)
#pragma unroll
  for (int half = kWindowMaxCap / 2, d = 32; half >= 1; half >>= 1, d >>= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int k = 0; k < half; ++k) {
      const float send = upper ? mx[k] : mx[k + half];
      const float keep = upper ? mx[k + half] : mx[k];
      mx[k] = fmaxf(keep, __shfl_xor(send, d, 64));
    }
  }
  float v = mx[0];
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  if ((lane & 3) == 0) red[wave * kWindowMaxCap + (lane >> 2)] = v;
  __syncthreads();
  v = -INFINITY;
  if (tid < kWindowMaxCap) {
    v = red[tid];
#pragma unroll
    for (int k = 1; k < NT / 64; ++k) v = fmaxf(v, red[k * kWindowMaxCap + tid]);
  }
  return v;
}

// Sequence n's token range and first global chunk.
struct SeqInfo {
  int64_t tok0;    // first token (flattened over B*T)
  int len;         // tokens in the sequence
  int64_t chunk0;  // global index of its first chunk
};

__device__ __forceinline__ SeqInfo seq_info(int n, const int32_t* cu, const int32_t* chunk_off,
                                            int64_t T) {
  SeqInfo s;
  if (cu) {
    s.tok0 = cu[n];
    s.len = cu[n + 1] - cu[n];
    s.chunk0 = chunk_off[n];
  } else {
    s.tok0 = (int64_t)n * T;
    s.len = (int)T;
    s.chunk0 = (int64_t)n * ((T + kChunk - 1) / kChunk);
  }
  return s;
}

// Sequence owning global chunk `cg` (binary search over chunk offsets).
__device__ __forceinline__ int seq_of_chunk(int64_t cg, const int32_t* chunk_off, int N,
                                            int64_t T) {
  if (!chunk_off) return (int)(cg / ((T + kChunk - 1) / kChunk));
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= cg) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace gdn
