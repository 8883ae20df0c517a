// Backward of the chunked GDN forward on gfx950 for fp32 q / k / v (bf16 inputs take
// the MFMA kernels of chunk_bwd_mfma.hip): gradients of <dO, O> + <dhT, hT> with
// respect to q, k, v, g, beta and the initial state.
//
// FlashQLA talk transcript (tokendh.com): results and timeline sections (the
// backward keeps the forward's structure); algebraic-rewrites section (the K K^T
// gradient reaches K once, as (dB + dB^T) K, the A-side and transposed terms merged
// first).  The chunk algebra differentiated here, with h = S^T at a chunk's start,
// G the chunk-local cumsum of g, gamma = exp(G), Gamma_ij = exp(G_i - G_j) (j <= i),
// d = exp(G_n - G):
//
//   A = strict_lower(diag(beta) K K^T * Gamma),  T = (I + A)^{-1}
//   V' = V - diag(gamma) K h,  U = T diag(beta) V'
//   O = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)
//   h' = gamma_n h + (diag(d) K)^T U
//
// Taken backwards (dY = scale dO, dh' the carried state gradient):
//   dU   = diag(d) K dh' + P^T dY                    P = (Q K^T) * Gamma
//   dR   = T^T dU,  dV = diag(beta) dR,  dbeta += rowsum(dR * V')
//   dP   = lower(dY U^T),  dA = strict_lower(-dR U^T),  dB = diag(beta) dA * Gamma
//   dQ   = diag(gamma) dY h^T + (dP * Gamma) K
//   dK   = diag(d) U dh'^T + (dP * Gamma)^T Q - diag(gamma) dV h^T + (dB + dB^T) K
//   dh   = gamma_n dh' + Q^T diag(gamma) dY - K^T diag(gamma) dV
//   dG   from the Gamma, gamma, d and gamma_n terms; dg = reverse cumsum of dG.
//
// Mapping: one workgroup per (sequence, head, 32 value columns), walking the chunks
// in reverse and recomputing each chunk's intermediates from the state at its start.
// Those states come from the forward's checkpoint pass (fused_forward.hip, kCkpt:
// the fused forward's MFMA recurrence over whole sequences, storing the state at
// every chunk start), which runs first.
// dV and dh0 of its columns are final; dQ, dK, dbeta and dg are sums over all value
// columns, so each workgroup writes its share in fp32 and a second kernel adds the
// shares.  Arithmetic is plain fp32, the chunk's matrices in LDS, K, Q, V and dO
// read from global memory (L1/L2 resident within a chunk); operands come as runs of
// eight consecutive elements: every product gives each thread a run of eight
// outputs, or eight contraction terms, per load.  P = (Q K^T) * Gamma is formed
// once per chunk, so no exponential sits in an inner loop.  512 threads (eight waves,
// two per SIMD) per workgroup: 1024 spilled registers once the loops took runs of
// eight.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kBwdCols = kBwdColumnBlock;  // value columns per workgroup
constexpr int kBwdThreads = 512;
constexpr int NS = kChunk + 1;            // row stride (floats) of chunk x chunk LDS matrices
constexpr int CS = kBwdCols + 1;          // row stride of chunk x 32 and dk x 32 LDS matrices

template <typename E>
__device__ __forceinline__ float ldf(const E* p, int64_t i) { return (float)p[i]; }

// Eight consecutive elements as fp32 (p 16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void ld8(const bf16* p, float* o) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Sum over the 16 consecutive lanes of a row group (a row's partial sums).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace

template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void chunk_bwd_kernel(Problem p, BwdArgs a) {
  static_assert(kBwdCols == 32 && DK % 8 == 0, "thread mappings below");
  constexpr int D8 = DK / 8;             // runs of eight along dk
  __shared__ float sKK[kChunk * NS], sT[kChunk * NS], sQK[kChunk * NS], sM[kChunk * NS];
  __shared__ float sVp[kChunk * CS], sU[kChunk * CS];
  __shared__ float sdU[kChunk * CS], sdR[kChunk * CS];
  __shared__ float sH[DK * CS], sdH[DK * CS];
  __shared__ float sG[kChunk], sGam[kChunk], sD[kChunk], sBet[kChunk], sdG[kChunk], sDD[kChunk], sQhY[kChunk],
      sKhR[kChunk];
  __shared__ float sRed[kBwdThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = p.dv / kBwdCols;
  const int blk = (int)(blockIdx.x % nblk);
  const int64_t unit = blockIdx.x / nblk;
  if (unit >= a.units) return;   // whole workgroup
  // the unit: (sequence, head), or with a split (segment, head), segments numbered as
  // in the forward's split; [c_lo, c_hi) are its chunks
  int n, h, seg = 0, S = 1;
  int64_t sg0 = 0;
  if (a.seg_chunks > 0) {
    h = (int)(unit % p.H);
    const int64_t sg = unit / p.H;
    if (a.seg_off) {
      n = seq_of_chunk(sg, a.seg_off, p.N, 0);
      sg0 = a.seg_off[n];
      S = (int)(a.seg_off[n + 1] - sg0);
    } else {
      const int64_t segs = max((int64_t)1, ((p.T + kChunk - 1) / kChunk + a.seg_chunks - 1) / a.seg_chunks);
      n = (int)(sg / segs);
      sg0 = (int64_t)n * segs;
      S = (int)segs;
    }
    seg = (int)(sg - sg0);
  } else {
    n = (int)(unit / p.H);
    h = (int)(unit % p.H);
  }
  const bool chain = a.mode == kBwdChain;
  if (chain && seg == 0) return;   // the merge needs no offset of a first segment
  const int64_t nh = (int64_t)n * p.H + h;
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int c_lo = a.seg_chunks > 0 ? min(nch, seg * a.seg_chunks) : 0;
  const int c_hi = a.seg_chunks > 0 ? min(nch, (seg + 1) * a.seg_chunks) : nch;
  const int H = p.H, dv = p.dv, col0 = blk * kBwdCols;
  const int64_t rqk = (int64_t)H * DK, rv = (int64_t)H * dv;
  const E* Qg = reinterpret_cast<const E*>(p.q) + si.tok0 * rqk + (int64_t)h * DK;
  const E* Kg = reinterpret_cast<const E*>(p.k) + si.tok0 * rqk + (int64_t)h * DK;
  const E* Vg = reinterpret_cast<const E*>(p.v) + si.tok0 * rv + (int64_t)h * dv + col0;
  const E* DOg = reinterpret_cast<const E*>(a.d_o) + si.tok0 * rv + (int64_t)h * dv + col0;
  const float scale = p.scale;
  const int64_t tot = a.total_tokens;

  auto Krow = [&](int i) { return Kg + (int64_t)i * rqk; };
  auto Qrow = [&](int i) { return Qg + (int64_t)i * rqk; };
  auto DOrow = [&](int i) { return DOg + (int64_t)i * rv; };
  auto gam_ij = [&](int i, int j) { return expf(sG[i] - sG[j]); };   // j <= i
  int ct0 = 0;   // first token of the chunk being processed
  // eight K elements of chunk row i from dk column d; eight dO elements of row i from
  // value column c; one dO element (dO, not yet scaled)
  auto kld8 = [&](int i, int d, float* o) { ld8(Krow(ct0 + i) + d, o); };
  auto dold8 = [&](int i, int c, float* o) { ld8(DOrow(ct0 + i) + c, o); };
  auto dos = [&](int i, int c) { return ldf(DOg, (int64_t)(ct0 + i) * rv + c); };


  // ---- the chunk's gates, K K^T (lower), P = (Q K^T) * Gamma (lower),
  //      K h, A -> T, V', U (the forward quantities)
  auto recompute = [&](int t0, int len) {
    ct0 = t0;
    if (wave == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < len) {
        gv = p.g[(si.tok0 + t0 + lane) * H + h];
        bv = load_scalar(p.beta, (si.tok0 + t0 + lane) * H + h, p.beta_bf16);
      }
      const float G = wave_inclusive_scan(gv);
      sG[lane] = G;
      sBet[lane] = bv;
    }
    __syncthreads();
    if (tid < kChunk) {
      const float gl = sG[len > 0 ? len - 1 : 0];
      sGam[tid] = expf(sG[tid]);
      sD[tid] = expf(gl - sG[tid]);
    }
    for (int e = tid; e < len * len; e += kBwdThreads) {
      const int i = e / len, j = e % len;
      if (j <= i) {
        const E* qi = Qrow(t0 + i);
        float acc = 0.f, accq = 0.f;
#pragma unroll 2
        for (int d = 0; d < DK; d += 8) {
          float x[8], y[8], z[8];
          kld8(i, d, x);
          kld8(j, d, y);
          ld8(qi + d, z);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            acc += x[u] * y[u];
            accq += z[u] * y[u];
          }
        }
        sKK[i * NS + j] = acc;
        sQK[i * NS + j] = accq * gam_ij(i, j);
      }
    }
    // V' = V - diag(gamma) K h (the chain pass needs neither V' nor U)
    for (int e = tid; e < (chain ? 0 : len * kBwdCols); e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
#pragma unroll 2
      for (int d = 0; d < DK; d += 8) {
        float x[8];
        kld8(i, d, x);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += x[u] * sH[(d + u) * CS + j];
      }
      sVp[i * CS + j] = ldf(Vg, (int64_t)(t0 + i) * rv + j) - expf(sG[i]) * acc;
    }
    __syncthreads();
    // A (strict lower; zero elsewhere over the whole 64 x 64, rows past a partial
    // chunk's end included) into sM
    for (int e = tid; e < kChunk * kChunk; e += kBwdThreads) {
      const int i = e / kChunk, j = e % kChunk;
      sM[i * NS + j] = (j < i && i < len) ? sBet[i] * gam_ij(i, j) * sKK[i * NS + j] : 0.f;
    }
    __syncthreads();
    // T = (I + A)^{-1} by 16 x 16 blocks: the diagonal blocks by forward substitution
    // (one thread per (block, column)), then the blocks below the diagonal, by
    // distance from it: T_ab = -T_aa X, X = sum_{k=b}^{a-1} A_ak T_kb (sdU as scratch)
    if (tid < kChunk) {
      const int o = 16 * (tid >> 4), c = tid & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = r == c ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m)
          if (m >= c) v -= sM[(o + r) * NS + o + m] * x[m];
        x[r] = r >= c ? v : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(o + r) * NS + o + c] = x[r];
    }
    __syncthreads();
    for (int dist = 1; dist < 4; ++dist) {
      const int nb = 4 - dist;   // blocks (a, a - dist), a = dist .. 3
      for (int e = tid; e < nb * 256; e += kBwdThreads) {
        const int a16 = 16 * (dist + e / 256), r = (e >> 4) & 15, c = e & 15, b16 = a16 - 16 * dist;
        float acc = 0.f;
        for (int m = b16; m < a16; ++m) acc += sM[(a16 + r) * NS + m] * sT[m * NS + b16 + c];
        sdU[(a16 + r) * CS + c] = acc;
      }
      __syncthreads();
      for (int e = tid; e < nb * 256; e += kBwdThreads) {
        const int a16 = 16 * (dist + e / 256), r = (e >> 4) & 15, c = e & 15, b16 = a16 - 16 * dist;
        float acc = 0.f;
        for (int m = 0; m <= r; ++m) acc += sT[(a16 + r) * NS + a16 + m] * sdU[(a16 + m) * CS + c];
        sT[(a16 + r) * NS + b16 + c] = -acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < (chain ? 0 : len * kBwdCols); e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int m = 0; m <= i; ++m) acc += sT[i * NS + m] * sBet[m] * sVp[m * CS + j];
      sU[i * CS + j] = acc;
    }
    __syncthreads();
  };

  // the state at every chunk start: the forward's checkpoint pass wrote it
  // (fused_forward.hip, kCkpt; layout ckpt_offset)
  auto chk = [&](int c) { return a.hchk + ((si.chunk0 + c) * H + h) * (int64_t)DK * dv; };

  // ================= reverse sweep =================
  // the state gradient after the unit's last chunk: dhT for a sequence's last segment
  // (or a whole sequence), the merge's result for the other segments, zero in the
  // chain pass
  const int64_t gslot = bwd_slot(sg0, S, seg) * H + h;
  for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
    const int i = e / kBwdCols, j = e % kBwdCols;
    float x = 0.f;
    if (!chain) {
      if (seg == S - 1) x = a.dhT ? a.dhT[((int64_t)nh * DK + i) * dv + col0 + j] : 0.f;
      else x = a.seg_g[(gslot * DK + i) * dv + col0 + j];
    }
    sdH[i * CS + j] = x;
  }
  __syncthreads();
  for (int c = c_hi - 1; c >= c_lo; --c) {
    const int t0 = c * kChunk, len = min(kChunk, si.len - t0);
    const float* hc = chk(c);
    for (int e = tid; e < (chain ? 0 : DK / 4 * kBwdCols); e += kBwdThreads) {   // four rows of a column
      const int i4 = (e / kBwdCols) * 4, j = e % kBwdCols;
      const f32x4 x = *reinterpret_cast<const f32x4*>(hc + ckpt_offset(i4, col0 + j, dv));
#pragma unroll
      for (int u = 0; u < 4; ++u) sH[(i4 + u) * CS + j] = x[u];
    }
    __syncthreads();
    recompute(t0, len);
    const float gn = expf(sG[len - 1]);
    // K dh' (into sdR for now) and dd_i = sum_j U_ij (K dh')_ij
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
#pragma unroll 2
      for (int d = 0; d < DK; d += 8) {
        float x[8];
        kld8(i, d, x);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += x[u] * sdH[(d + u) * CS + j];
      }
      sdR[i * CS + j] = acc;
    }
    __syncthreads();
    // (16 lanes per row: the rows' reductions below are all split this way)
    for (int e = tid; e < (chain ? 0 : len * 16); e += kBwdThreads) {
      const int i = e >> 4, pp = e & 15;
      const float acc = row16_sum(sU[i * CS + pp] * sdR[i * CS + pp] + sU[i * CS + pp + 16] * sdR[i * CS + pp + 16]);
      if (pp == 0) sDD[i] = acc;
    }
    // dU = diag(d) K dh' + P^T dY: a thread owns columns j8 .. j8 + 7 of one row
    for (int e = tid; e < len * (kBwdCols / 8); e += kBwdThreads) {
      const int i = e / (kBwdCols / 8), j8 = (e % (kBwdCols / 8)) * 8;
      float acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = sD[i] * sdR[i * CS + j8 + u];
#pragma unroll 2
      for (int m = i; m < len; ++m) {
        float o[8];
        dold8(m, j8, o);
        const float pm = scale * sQK[m * NS + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += pm * o[u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sdU[i * CS + j8 + u] = acc[u];
    }
    __syncthreads();
    // dR = T^T dU;  dP = lower(dY U^T) into sM
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int m = i; m < len; ++m) acc += sT[m * NS + i] * sdU[m * CS + j];
      sdR[i * CS + j] = acc;
    }
    if (chain) {
      __syncthreads();   // dR, read by the state-gradient update below
    } else {
      for (int e = tid; e < len * len; e += kBwdThreads) {
        const int i = e / len, j = e % len;
        float acc = 0.f;
        if (j <= i) {
#pragma unroll 2
          for (int k8 = 0; k8 < kBwdCols; k8 += 8) {
            float o[8];
            dold8(i, k8, o);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += o[u] * sU[j * CS + k8 + u];
          }
          acc *= scale;
        }
        sM[i * NS + j] = acc;
      }
      __syncthreads();
      // dV = diag(beta) dR; the Gamma gradient of P: E_ij = dP_ij P_ij
      E* dVg = reinterpret_cast<E*>(a.dv) + si.tok0 * rv + (int64_t)h * dv + col0;
      for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
        const int i = e / kBwdCols, j = e % kBwdCols;
        dVg[(int64_t)(t0 + i) * rv + j] = (E)(sBet[i] * sdR[i * CS + j]);
      }
      for (int e = tid; e < len * 16; e += kBwdThreads) {
        const int i = e >> 4, pp = e & 15;
        float r = 0.f, cs = 0.f;
        for (int j = pp; j <= i; j += 16) r += sM[i * NS + j] * sQK[i * NS + j];
        for (int m = i + pp; m < len; m += 16) cs += sM[m * NS + i] * sQK[m * NS + i];
        const float v = row16_sum(r - cs);
        if (pp == 0) sdG[i] = v;
      }
      __syncthreads();
      // sQK <- dP * Gamma (lower);  then dA = strict_lower(-dR U^T) into sM
      for (int e = tid; e < len * len; e += kBwdThreads) {
        const int i = e / len, j = e % len;
        sQK[i * NS + j] = j <= i ? sM[i * NS + j] * gam_ij(i, j) : 0.f;
      }
      __syncthreads();
      for (int e = tid; e < len * len; e += kBwdThreads) {
        const int i = e / len, j = e % len;
        float acc = 0.f;
        if (j < i)
          for (int k2 = 0; k2 < kBwdCols; ++k2) acc -= sdR[i * CS + k2] * sU[j * CS + k2];
        sM[i * NS + j] = acc;
      }
      __syncthreads();
      // dbeta share: rowsum(dR * V') + sum_j dA_ij KK_ij Gamma_ij; the Gamma gradient of A
      for (int e = tid; e < len * 16; e += kBwdThreads) {
        const int i = e >> 4, pp = e & 15;
        float db = sdR[i * CS + pp] * sVp[i * CS + pp] + sdR[i * CS + pp + 16] * sVp[i * CS + pp + 16];
        float t = 0.f, cs = 0.f;
        for (int j = pp; j < i; j += 16) t += sM[i * NS + j] * sKK[i * NS + j] * gam_ij(i, j);
        for (int m = i + 1 + pp; m < len; m += 16) cs += sBet[m] * sM[m * NS + i] * sKK[m * NS + i] * gam_ij(m, i);
        db = row16_sum(db + t);
        const float dgA = row16_sum(sBet[i] * t - cs);
        if (pp == 0) {
          sdG[i] += dgA;
          a.dbeta_p[((int64_t)blk * tot + si.tok0 + t0 + i) * H + h] = db;
        }
      }
      __syncthreads();
      // sKK <- dB = diag(beta) dA * Gamma (strict lower; zero elsewhere)
      for (int e = tid; e < len * len; e += kBwdThreads) {
        const int i = e / len, j = e % len;
        sKK[i * NS + j] = j < i ? sBet[i] * sM[i * NS + j] * gam_ij(i, j) : 0.f;
      }
      __syncthreads();
      // shares of dQ and dK (the K K^T gradient enters as (dB + dB^T) K, merged); a
      // thread owns columns d8 .. d8 + 7 of one row.  The Y = Q h part of gamma's
      // gradient, sum_j (Q h)_ij dY_ij = sum_d Q_id (dY h^T)_id, is summed on the side.
      for (int e = tid; e < len * D8; e += kBwdThreads) {
        const int i = e / D8, d8 = (e % D8) * 8;
        float hdy[8], udh[8], rvh[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) hdy[u] = udh[u] = rvh[u] = 0.f;
#pragma unroll 2
        for (int j = 0; j < kBwdCols; ++j) {
          const float dy = scale * dos(i, j);
          const float uu = sU[i * CS + j], rr = sBet[i] * sdR[i * CS + j];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float hv = sH[(d8 + u) * CS + j];
            hdy[u] += dy * hv;
            udh[u] += uu * sdH[(d8 + u) * CS + j];
            rvh[u] += rr * hv;
          }
        }
        float dq[8], dk[8], qi[8], ki[8];
        ld8(Qrow(t0 + i) + d8, qi);
        kld8(i, d8, ki);
        float qhy = 0.f, khr = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          qhy += qi[u] * hdy[u];
          khr += ki[u] * rvh[u];
          dq[u] = sGam[i] * hdy[u];
          dk[u] = sD[i] * udh[u] - sGam[i] * rvh[u];
        }
#pragma unroll 1
        for (int m = 0; m < len; ++m) {
          float km[8], qm[8];
          kld8(m, d8, km);
          ld8(Qrow(t0 + m) + d8, qm);
          const float pq = sQK[i * NS + m];                      // zero for m > i
          const float pk = m >= i ? sQK[m * NS + i] : 0.f;
          const float bb = sKK[i * NS + m] + sKK[m * NS + i];    // dB strict lower, zero elsewhere
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            dq[u] += pq * km[u];
            dk[u] += pk * qm[u] + bb * km[u];
          }
        }
        const int64_t o = (((int64_t)blk * tot + si.tok0 + t0 + i) * H + h) * DK + d8;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a.dq_p[o + u] = dq[u];
          a.dk_p[o + u] = dk[u];
        }
        // the D8 threads of row i are consecutive lanes of one wave
#pragma unroll
        for (int off = D8 / 2; off >= 1; off >>= 1) {
          qhy += __shfl_xor(qhy, off, 64);
          khr += __shfl_xor(khr, off, 64);
        }
        if (d8 == 0) {
          sQhY[i] = qhy;
          sKhR[i] = khr;
        }
      }
      // gamma_n's gradient: <h, dh'> over this block's columns (workgroup reduction)
      float part = 0.f;
      for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
        const int i = e / kBwdCols, j = e % kBwdCols;
        part += sH[i * CS + j] * sdH[i * CS + j];
      }
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      if (lane == 0) sRed[wave] = part;
      __syncthreads();
      // the gamma and d gradients into dG
      // (the K h part of gamma's gradient, beta_i sum_j dR_ij (K h)_ij =
      // sum_d K_id (beta_i dR h^T)_id, was summed with the dK shares)
      if (tid < len) sdG[tid] += (sQhY[tid] - sKhR[tid]) * sGam[tid] - sDD[tid] * sD[tid];
      __syncthreads();
      // gamma_n's and d's gradients into the last row, then dg = reverse cumsum of dG
      if (wave == 0) {
        float x = (lane < len ? sDD[lane] * sD[lane] : 0.f) + (lane < kBwdThreads / 64 ? sRed[lane] * gn : 0.f);
        for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
        const float gv = lane < len ? sdG[lane] + (lane == len - 1 ? x : 0.f) : 0.f;
        const float pre = wave_inclusive_scan(gv);
        const float total = __shfl(pre, 63, 64);
        if (lane < len) a.dg_p[((int64_t)blk * tot + si.tok0 + t0 + lane) * H + h] = total - pre + gv;
      }
    }
    // dh = gamma_n dh' + Q^T diag(gamma) dY - K^T diag(gamma beta) dR (in place): a
    // thread owns rows i8 .. i8 + 7 of one column
    for (int e = tid; e < D8 * kBwdCols; e += kBwdThreads) {
      const int i8 = (e / kBwdCols) * 8, j = e % kBwdCols;
      float acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = gn * sdH[(i8 + u) * CS + j];
#pragma unroll 1
      for (int m = 0; m < len; ++m) {
        float qv[8], kv[8];
        ld8(Qrow(t0 + m) + i8, qv);
        kld8(m, i8, kv);
        const float ay = sGam[m] * scale * dos(m, j);
        const float ar = sGam[m] * sBet[m] * sdR[m * CS + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += qv[u] * ay - kv[u] * ar;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sdH[(i8 + u) * CS + j] = acc[u];
    }
    __syncthreads();
  }
  if (chain) {
    // the state gradient at the segment's start from a zero one at its end: the merge's
    // offset for this segment (accumulator-tile order, as the forward's S*)
    float* dst = a.seg_b + gslot * (int64_t)DK * dv;
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      dst[sfrag_offset<DK>(i, col0 + j)] = sdH[i * CS + j];
    }
  } else if (a.dh0 && seg == 0) {
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      a.dh0[((int64_t)nh * DK + i) * dv + col0 + j] = sdH[i * CS + j];
    }
  }
}

// dq, dk, dbeta, dg: the sum of the value-column blocks' shares, in the output dtypes.
template <typename E, typename EB>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int64_t tot, int H, int DK, int nblk) {
  const int64_t n_qk = tot * H * DK, n_s = tot * H;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n_qk; e += (int64_t)gridDim.x * 256) {
    float q = 0.f, k = 0.f;
    for (int b = 0; b < nblk; ++b) {
      q += a.dq_p[b * n_qk + e];
      k += a.dk_p[b * n_qk + e];
    }
    reinterpret_cast<E*>(a.dq)[e] = (E)q;
    reinterpret_cast<E*>(a.dk)[e] = (E)k;
    if (e < n_s) {
      float bsum = 0.f, gsum = 0.f;
      for (int b = 0; b < nblk; ++b) {
        bsum += a.dbeta_p[b * n_s + e];
        gsum += a.dg_p[b * n_s + e];
      }
      reinterpret_cast<EB*>(a.dbeta)[e] = (EB)bsum;
      a.dg[e] = gsum;
    }
  }
}

template <typename E, int DK>
static hipError_t launch_bwd_dk(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  const int nblk = p.dv / kBwdCols;
  const int64_t wgs = a.units * nblk;
  if (wgs > kMaxDispatchItems / kBwdThreads) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL(chunk_bwd_kernel<E, DK>, dim3((unsigned)wgs), dim3(kBwdThreads), 0, s, ev.start,
                        a.mode == kBwdChain ? ev.stop : nullptr, 0, p, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (a.mode == kBwdChain) return hipSuccess;   // no shares to add
  const int64_t n_qk = a.total_tokens * p.H * DK;
  const int64_t blocks = std::min<int64_t>((n_qk + 255) / 256, 65536);
  if (p.beta_bf16)
    hipExtLaunchKernelGGL((bwd_reduce_kernel<E, bf16>), dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s,
                          nullptr, ev.stop, 0, a, a.total_tokens, p.H, DK, nblk);
  else
    hipExtLaunchKernelGGL((bwd_reduce_kernel<E, float>), dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s,
                          nullptr, ev.stop, 0, a, a.total_tokens, p.H, DK, nblk);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  if (a.units == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (p.dv % kBwdCols != 0 || p.qkv_bf16) return hipErrorInvalidValue;   // bf16: chunk_bwd_mfma.hip
  return p.dk == 128 ? launch_bwd_dk<float, 128>(p, a, s, ev) : launch_bwd_dk<float, 64>(p, a, s, ev);
}

}  // namespace gdn
