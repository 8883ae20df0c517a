// Step 1 of the chunked WY form on gfx950: per (chunk, head), the gated,
// beta-scaled Gram matrix of the chunk's keys and the inverse of its unit
// lower-triangular completion.
//
// FlashQLA talk transcript (tokendh.com), chunked-WY section: form K K^T inside
// each chunk and invert the C x C matrix; kernel-cut section: this inverse is a
// kernel of its own so that the sequence-parallel pass can reuse it; algebraic-
// rewrites section: Gamma is formed in log space, Gamma_rs = exp(G_r - G_s).
//
//   A = strict_lower(diag(beta) K K^T * Gamma),   T = (I + A)^{-1}
//
// Mapping: one wave per (chunk, head), four heads of one chunk per workgroup, no
// workgroup barriers (waves exchange data only through their own LDS slice).
// The key rows go straight from HBM into MFMA operand registers; the Gram tiles
// run on v_mfma_f32_16x16x32_bf16 (fp32 path: 16x16x4_f32).  With 16x16 blocks
// A_ij, T_ij of A and T:
//   * T_ii = (I + A_ii)^{-1} by forward substitution in fp32, lane = (block, column);
//   * the rest by two doubling levels of 16x16x16 MFMA products (fp32 inputs: fp32
//     MFMA; bf16 inputs: bf16 MFMA, fp32 accumulation),
//       T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22,
//       [T_20 T_21; T_30 T_31] = -[T_22 0; T_32 T_33] A[32:, :32] [T_00 0; T_10 T_11].
// Register-resident products.  In accumulator ("D") layout lane (r, q) holds
// X[4q+i][r] in slot i.  Feeding slot e of X^T's D tile as the A operand and slot e
// of Y's D tile as the B operand of four chained 16x16x4 MFMAs contracts index
// 4q+e, so D(X^T), D(Y) -> D(XY), and with the operands swapped D(Y), D(X^T) ->
// D((XY)^T).  Off-diagonal Gram tiles are therefore formed transposed (K_j K_i^T,
// gated with the roles of rows and columns exchanged), and T's final blocks come
// out transposed, i.e. with four consecutive columns of one row per lane, which is
// what the row-major store wants.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

template <typename E, int DK>
struct InvCfg {
  static constexpr int NS = DK / 32;                           // Gram contraction steps
  static constexpr int OS = kChunk + (sizeof(E) == 2 ? 8 : 4);  // staged T row stride (elements)
  static constexpr int ABS = 260;   // block stride of the staged diagonal A blocks (floats)
  static constexpr int TCS = 20;    // column stride of the staged diagonal T blocks (floats)
  static constexpr int TBS = 16 * TCS;
  static constexpr int WORK = 4 * ABS + 4 * TBS;              // A and T diagonal blocks
  static constexpr int OUT = kChunk * OS * (int)sizeof(E) / 4;  // staged T (aliases WORK)
  static constexpr int UNION = WORK > OUT ? WORK : OUT;
  static constexpr int PER_WAVE = 2 * kChunk + UNION;          // floats of LDS per wave
};

// D(X^T), D(Y), acc -> acc + D(X Y) for 16x16 blocks (see the header comment).  fp32
// inputs: four chained v_mfma_f32_16x16x4_f32 (fp32 products, the fp32 path's 1e-5
// accuracy).  bf16 inputs: one v_mfma_f32_16x16x16_bf16 on the operands rounded to
// bf16 (the four slots of a D tile are exactly that MFMA's four contraction
// elements); T leaves this kernel in bf16, whose rounding is of the same size.
template <typename E>
__device__ __forceinline__ f32x4 mm16(const f32x4& xt, const f32x4& y, f32x4 acc) {
  if constexpr (sizeof(E) == 2) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 a = __builtin_bit_cast(i16x4, pack_bf16x4(xt));
    const i16x4 b = __builtin_bit_cast(i16x4, pack_bf16x4(y));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[e], y[e], acc, 0, 0, 0);
    return acc;
  }
}

// Orders this wave's LDS accesses across lanes (LDS executes a wave's operations in
// issue order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename E>
__device__ __forceinline__ typename Mma<E>::frag load_frag(const E* src, bool ok) {
  typename Mma<E>::frag f;
  if (ok) {
    f = *reinterpret_cast<const typename Mma<E>::frag*>(src);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (E)0.f;
  }
  return f;
}

}  // namespace

// full = 0: the upper-right 32 x 32 quadrant of T (zero) is not written; the fused
// forward never reads it.
template <typename E, int DK>
__global__ __launch_bounds__(256) void chunk_inverse_kernel(Problem p, E* __restrict__ tout,
                                                             float* __restrict__ csum, int full) {
  using Cfg = InvCfg<E, DK>;
  using M = Mma<E>;
  using frag = typename M::frag;
  constexpr int NS = Cfg::NS, OS = Cfg::OS, ABS = Cfg::ABS, TCS = Cfg::TCS, TBS = Cfg::TBS;
  __shared__ __align__(16) float lds[4 * Cfg::PER_WAVE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int HG = (p.H + 3) / 4;
  const int64_t cg = blockIdx.x / HG;
  const int h = (int)(blockIdx.x % HG) * 4 + wave;
  if (h >= p.H) return;   // whole wave: no workgroup barrier follows
  const int n = seq_of_chunk(cg, p.chunk_off, p.N, p.T);
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int c = (int)(cg - si.chunk0);
  const int64_t r0 = si.tok0 + (int64_t)c * kChunk;
  const int len = min(kChunk, si.len - c * kChunk);

  float* sG = lds + wave * Cfg::PER_WAVE;   // chunk-local cumulative gate, per row
  float* sB = sG + kChunk;                  // beta, per row
  float* sAd = sB + kChunk;                 // diagonal A blocks, row-major, stride 16
  float* sTd = sAd + 4 * ABS;               // diagonal T blocks, column-major, stride TCS
  E* sOut = reinterpret_cast<E*>(sAd);      // staged T, row-major (after sAd/sTd are read)

  // ---- key rows -> operand registers: tile a, step s, lane (r, q): row 16a+r, cols 32s+8q..+7
  const E* K = reinterpret_cast<const E*>(p.k) + (r0 * p.H + h) * DK;
  const int64_t krow = (int64_t)p.H * DK;
  frag kf[4][NS];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kf[a][s] = load_frag<E>(K + (16 * a + r) * krow + 32 * s + 8 * q, 16 * a + r < len);

  {
    float gv = 0.f, bv = 0.f;
    if (lane < len) {
      gv = p.g[(r0 + lane) * p.H + h];
      bv = load_scalar(p.beta, (r0 + lane) * p.H + h, p.beta_bf16);
    }
    const float G = wave_inclusive_scan(gv);
    sG[lane] = G;
    sB[lane] = bv;
    if (csum && lane == kChunk - 1) csum[cg * p.H + h] = G;   // chunk gate sum for the gate scan
  }

  // ---- Gram tiles: diagonal (a, a) and transposed off-diagonal (b, a), b < a
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 gd[4], go[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    gd[a] = zero4;
#pragma unroll
    for (int s = 0; s < NS; ++s) gd[a] = M::run(kf[a][s], kf[a][s], gd[a]);
#pragma unroll
    for (int b = 0; b < a; ++b) {
      go[a][b] = zero4;
#pragma unroll
      for (int s = 0; s < NS; ++s) go[a][b] = M::run(kf[b][s], kf[a][s], go[a][b]);
    }
  }
  wave_lds_sync();

  // ---- gate and mask: A[m][k] = beta_m exp(G_m - G_k) (K K^T)[m][k], k < m
  float Gc[4], Bc[4];
  f32x4 Gr[4], Br[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    Gc[a] = sG[16 * a + r];
    Bc[a] = sB[16 * a + r];
    Gr[a] = *reinterpret_cast<const f32x4*>(sG + 16 * a + 4 * q);
    Br[a] = *reinterpret_cast<const f32x4*>(sB + 16 * a + 4 * q);
  }
  f32x4 At[4][4];   // At[a][b] = D(A_ab^T), b < a
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      sAd[a * ABS + m * 16 + r] = r < m ? Br[a][i] * fast_exp(Gr[a][i] - Gc[a]) * gd[a][i] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < a; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) At[a][b][i] = Bc[a] * fast_exp(Gc[a] - Gr[b][i]) * go[a][b][i];
  }
  wave_lds_sync();

  // ---- T_bb = (I + A_bb)^{-1}: lane (r, q) solves column r of block q
  {
    const float* arow = sAd + q * ABS;
    float x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      float acc = (m == r) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < (m + 3) / 4; ++j) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(arow + m * 16 + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * j + e < m) acc -= a4[e] * x[4 * j + e];
      }
      x[m] = acc;
    }
    float* tcol = sTd + q * TBS + r * TCS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = {x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
      *reinterpret_cast<f32x4*>(tcol + 4 * j) = v;
    }
  }
  wave_lds_sync();
  f32x4 Td[4], TdT[4];   // D(T_aa), D(T_aa^T)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    Td[a] = *reinterpret_cast<const f32x4*>(sTd + a * TBS + r * TCS + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) TdT[a][i] = sTd[a * TBS + (4 * q + i) * TCS + r];
  }
  wave_lds_sync();

  // ---- doubling levels (D(.) of each block; "T" suffix = transposed block)
  const f32x4 R10 = mm16<E>(At[1][0], Td[0], zero4);
  const f32x4 T10 = -mm16<E>(TdT[1], R10, zero4);
  const f32x4 T10T = -mm16<E>(R10, TdT[1], zero4);
  const f32x4 R32 = mm16<E>(At[3][2], Td[2], zero4);
  const f32x4 T32T = -mm16<E>(R32, TdT[3], zero4);
  const f32x4 R20 = mm16<E>(At[2][1], T10, mm16<E>(At[2][0], Td[0], zero4));
  const f32x4 R21 = mm16<E>(At[2][1], Td[1], zero4);
  const f32x4 R30 = mm16<E>(At[3][1], T10, mm16<E>(At[3][0], Td[0], zero4));
  const f32x4 R31 = mm16<E>(At[3][1], Td[1], zero4);
  const f32x4 T20T = -mm16<E>(R20, TdT[2], zero4);
  const f32x4 T21T = -mm16<E>(R21, TdT[2], zero4);
  const f32x4 T30T = -mm16<E>(R30, TdT[3], mm16<E>(R20, T32T, zero4));
  const f32x4 T31T = -mm16<E>(R31, TdT[3], mm16<E>(R21, T32T, zero4));

  // ---- stage T row-major (lane (r, q) of block (a, b): row 16a+r, cols 16b+4q..+3)
  auto put = [&](int a, int b, const f32x4& v) { store4(sOut + (16 * a + r) * OS + 16 * b + 4 * q, v); };
#pragma unroll
  for (int a = 0; a < 4; ++a) put(a, a, TdT[a]);
  put(1, 0, T10T);
  put(2, 0, T20T);
  put(2, 1, T21T);
  put(3, 0, T30T);
  put(3, 1, T31T);
  put(3, 2, T32T);
  wave_lds_sync();

  // ---- coalesced 16-byte stores; blocks above the diagonal are zero
  constexpr int EPV = 16 / (int)sizeof(E);
  constexpr int SPR = kChunk / EPV;   // 16-byte segments per row
  E* dst = tout + ((int64_t)cg * p.H + h) * (kChunk * kChunk);
#pragma unroll
  for (int j = 0; j < kChunk * SPR / 64; ++j) {
    const int idx = 64 * j + lane, row = idx / SPR, seg = idx % SPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (seg * EPV < 16 * (row / 16 + 1)) v = *reinterpret_cast<const u32x4*>(sOut + row * OS + seg * EPV);
    if (full || row >= kChunk / 2 || seg * EPV < kChunk / 2)
      *reinterpret_cast<u32x4*>(dst + row * kChunk + seg * EPV) = v;
  }
}

__global__ void chunk_offsets_kernel(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ off) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int32_t acc = 0;
    off[0] = 0;
    for (int n = 0; n < N; ++n) {
      acc += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
      off[n + 1] = acc;
    }
  }
}

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s) {
  chunk_offsets_kernel<<<1, 64, 0, s>>>(cu, N, chunk_off);
  return hipGetLastError();
}

hipError_t launch_chunk_inverse(const Problem& p, void* t_out, float* csum, bool full, hipStream_t s,
                                KernelEvents ev) {
  const int64_t blocks = p.total_chunks * ((p.H + 3) / 4);
  if (blocks == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (blocks > kMaxDispatchItems / 256) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (p.qkv_bf16) {
    if (p.dk == 128)
      hipExtLaunchKernelGGL(chunk_inverse_kernel<bf16, 128>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, p,
                            (bf16*)t_out, csum, full ? 1 : 0);
    else
      hipExtLaunchKernelGGL(chunk_inverse_kernel<bf16, 64>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, p,
                            (bf16*)t_out, csum, full ? 1 : 0);
  } else {
    if (p.dk == 128)
      hipExtLaunchKernelGGL(chunk_inverse_kernel<float, 128>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, p,
                            (float*)t_out, csum, full ? 1 : 0);
    else
      hipExtLaunchKernelGGL(chunk_inverse_kernel<float, 64>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, p,
                            (float*)t_out, csum, full ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace gdn
