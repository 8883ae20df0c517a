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
// Mapping: one 256-thread workgroup per (chunk, head).  The Gram matrix runs on
// MFMA (wave w owns row tile w, bf16 or fp32 operands, fp32 accumulation).  The
// inverse is computed in fp32 in LDS: the four 16x16 diagonal blocks by forward
// substitution (one lane per column), then two doubling levels
//     [D0 0; X D1]^-1 off-diagonal = -D1 A10 D0            (16 -> 32)
//     [X0 0; Y X1]^-1 off-diagonal = -X1 A[32:,:32] X0     (32 -> 64)
// and T is written in the storage dtype, row-major 64 x 64 per (chunk, head).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename E, int DK>
__global__ __launch_bounds__(256) void chunk_inverse_kernel(Problem p, E* __restrict__ tout) {
  constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
  constexpr int KS = DK + PAD;       // padded row stride of the key tile (elements)
  constexpr int AS = 65;             // fp32 stride of A and T
  constexpr int VPR = DK * (int)sizeof(E) / 16;
  constexpr int EPV = 16 / (int)sizeof(E);
  __shared__ __align__(16) E sK[64 * KS];
  __shared__ float sA[64 * AS];
  __shared__ float sT[64 * AS];
  __shared__ float sG[64], sB[64];
  float* sR = reinterpret_cast<float*>(sK);  // scratch once the Gram matrix is done
  static_assert(sizeof(sK) >= 32 * 33 * sizeof(float), "scratch alias too small");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t cg = blockIdx.x;
  const int h = blockIdx.y;
  const int n = seq_of_chunk(cg, p.chunk_off, p.N, p.T);
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int c = (int)(cg - si.chunk0);
  const int64_t r0 = si.tok0 + (int64_t)c * kChunk;
  const int len = min(kChunk, si.len - c * kChunk);
  const E* K = reinterpret_cast<const E*>(p.k);

  for (int i = tid; i < 64 * VPR; i += 256) {
    const int r = i / VPR, cv = i % VPR;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < len) val = *reinterpret_cast<const u32x4*>(K + ((r0 + r) * p.H + h) * DK + cv * EPV);
    *reinterpret_cast<u32x4*>(sK + r * KS + cv * EPV) = val;
  }
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (lane < len) {
      gv = p.g[(r0 + lane) * p.H + h];
      bv = load_scalar(p.beta, (r0 + lane) * p.H + h, p.beta_bf16);
    }
    sG[lane] = wave_inclusive_scan(gv);
    sB[lane] = bv;
  }
  __syncthreads();

  // Gram matrix, row tile = wave; mask before exp.
  {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (v <= wave) {
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          acc = Mma<E>::run(lds_frag(sK, KS, 16 * wave + r, 32 * s, q),
                            lds_frag(sK, KS, 16 * v + r, 32 * s, q), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * q + i, col = 16 * v + r;
        float val = 0.f;
        if (col < row) val = sB[row] * fast_exp(sG[row] - sG[col]) * acc[i];
        sA[row * AS + col] = val;
      }
    }
  }
  __syncthreads();

  // Diagonal blocks: lane = 16*b + column.
  if (wave == 0) {
    const int b = lane >> 4, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float acc = (rr == cc) ? 1.f : 0.f;
      const float* arow = sA + (16 * b + rr) * AS + 16 * b;
#pragma unroll
      for (int s = 0; s < rr; ++s) acc -= arow[s] * x[s];
      x[rr] = acc;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sT[(16 * b + rr) * AS + 16 * b + cc] = x[rr];
  }
  __syncthreads();

  // 16 -> 32: blocks (1,0) and (3,2):  T_i,i-1 = -D_i (A_i,i-1 D_i-1)
  for (int idx = tid; idx < 512; idx += 256) {
    const int which = idx >> 8, rr = (idx >> 4) & 15, cc = idx & 15;
    const int i = which ? 3 : 1, j = i - 1;
    const float* arow = sA + (16 * i + rr) * AS + 16 * j;
    float acc = 0.f;
    for (int s = cc; s < 16; ++s) acc += arow[s] * sT[(16 * j + s) * AS + 16 * j + cc];
    sR[which * 256 + rr * 16 + cc] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < 512; idx += 256) {
    const int which = idx >> 8, rr = (idx >> 4) & 15, cc = idx & 15;
    const int i = which ? 3 : 1, j = i - 1;
    const float* drow = sT + (16 * i + rr) * AS + 16 * i;
    float acc = 0.f;
    for (int s = 0; s <= rr; ++s) acc += drow[s] * sR[which * 256 + s * 16 + cc];
    sT[(16 * i + rr) * AS + 16 * j + cc] = -acc;
  }
  __syncthreads();

  // 32 -> 64: T[32:,:32] = -X1 (A[32:,:32] X0)
  for (int idx = tid; idx < 1024; idx += 256) {
    const int rr = idx >> 5, cc = idx & 31;
    const float* arow = sA + (32 + rr) * AS;
    float acc = 0.f;
    for (int s = cc; s < 32; ++s) acc += arow[s] * sT[s * AS + cc];
    sR[rr * 33 + cc] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < 1024; idx += 256) {
    const int rr = idx >> 5, cc = idx & 31;
    const float* xrow = sT + (32 + rr) * AS + 32;
    float acc = 0.f;
    for (int s = 0; s <= rr; ++s) acc += xrow[s] * sR[s * 33 + cc];
    sT[(32 + rr) * AS + cc] = -acc;
  }
  __syncthreads();

  E* dst = tout + ((int64_t)cg * p.H + h) * (kChunk * kChunk);
  for (int idx = tid; idx < kChunk * kChunk; idx += 256) {
    const int rr = idx >> 6, cc = idx & 63;
    dst[idx] = from_f32<E>(cc <= rr ? sT[rr * AS + cc] : 0.f);
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

hipError_t launch_chunk_inverse(const Problem& p, void* t_out, hipStream_t s) {
  if (p.total_chunks == 0) return hipSuccess;
  dim3 grid((unsigned)p.total_chunks, (unsigned)p.H);
  if (p.qkv_bf16) {
    if (p.dk == 128) chunk_inverse_kernel<bf16, 128><<<grid, 256, 0, s>>>(p, (bf16*)t_out);
    else chunk_inverse_kernel<bf16, 64><<<grid, 256, 0, s>>>(p, (bf16*)t_out);
  } else {
    if (p.dk == 128) chunk_inverse_kernel<float, 128><<<grid, 256, 0, s>>>(p, (float*)t_out);
    else chunk_inverse_kernel<float, 64><<<grid, 256, 0, s>>>(p, (float*)t_out);
  }
  return hipGetLastError();
}

}  // namespace gdn
