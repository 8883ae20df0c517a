// Backward of the chunked GDN forward on gfx950: gradients of <dO, O> + <dhT, hT>
// with respect to q, k, v, g, beta and the initial state.
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
// Mapping: one workgroup per (sequence, head, 32 value columns).  The state columns
// are independent in the forward, so each workgroup runs the forward over its
// sequence first (the state at every chunk start goes to a checkpoint buffer), then
// the chunks in reverse, recomputing each chunk's intermediates from its checkpoint.
// dV and dh0 of its columns are final; dQ, dK, dbeta and dg are sums over all value
// columns, so each workgroup writes its share in fp32 and a second kernel adds the
// shares.  Arithmetic is plain fp32 (inputs converted on load), one thread per output
// element of each product, the chunk's matrices in LDS and K, Q, V, dO read from
// global memory (L1/L2 resident within a chunk).  1024 threads per workgroup: the
// products' inner loops wait on those reads, and 16 waves hide 2.5x more of the
// latency than 4 (Qwen-like shape: 90 ms with 256 threads, 54 with 512, 36 with 1024).
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kBwdCols = kBwdColumnBlock;  // value columns per workgroup
constexpr int kBwdThreads = 1024;
constexpr int NS = kChunk + 1;            // row stride (floats) of chunk x chunk LDS matrices
constexpr int CS = kBwdCols + 1;          // row stride of chunk x 32 and dk x 32 LDS matrices

template <typename E>
__device__ __forceinline__ float ldf(const E* p, int64_t i) { return (float)p[i]; }

}  // namespace

template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void chunk_bwd_kernel(Problem p, BwdArgs a) {
  __shared__ float sKK[kChunk * NS], sT[kChunk * NS], sQK[kChunk * NS], sM[kChunk * NS];
  __shared__ float sKh[kChunk * CS], sQh[kChunk * CS], sVp[kChunk * CS], sU[kChunk * CS];
  __shared__ float sdU[kChunk * CS], sdR[kChunk * CS];
  __shared__ float sH[DK * CS], sdH[DK * CS];
  __shared__ float sG[kChunk], sGam[kChunk], sD[kChunk], sBet[kChunk], sdG[kChunk], sDD[kChunk];
  __shared__ float sRed[kBwdThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = p.dv / kBwdCols;
  const int blk = (int)(blockIdx.x % nblk);
  const int64_t nh = blockIdx.x / nblk;
  if (nh >= (int64_t)p.N * p.H) return;   // whole workgroup
  const int n = (int)(nh / p.H), h = (int)(nh % p.H);
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int H = p.H, dv = p.dv, col0 = blk * kBwdCols;
  const int64_t rqk = (int64_t)H * DK, rv = (int64_t)H * dv;
  const E* Qg = reinterpret_cast<const E*>(p.q) + si.tok0 * rqk + (int64_t)h * DK;
  const E* Kg = reinterpret_cast<const E*>(p.k) + si.tok0 * rqk + (int64_t)h * DK;
  const E* Vg = reinterpret_cast<const E*>(p.v) + si.tok0 * rv + (int64_t)h * dv + col0;
  const E* DOg = reinterpret_cast<const E*>(a.d_o) + si.tok0 * rv + (int64_t)h * dv + col0;
  const float scale = p.scale;
  const int64_t tot = a.total_tokens;

  auto Kv = [&](int i, int d) { return ldf(Kg, (int64_t)i * rqk + d); };
  auto Qv = [&](int i, int d) { return ldf(Qg, (int64_t)i * rqk + d); };
  auto gam_ij = [&](int i, int j) { return expf(sG[i] - sG[j]); };   // j <= i

  // ---- the chunk's gates, K K^T (lower), K h, A -> T, V', U (the forward quantities)
  auto recompute = [&](int t0, int len, bool for_backward) {
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
        float acc = 0.f, accq = 0.f;
        for (int d = 0; d < DK; ++d) {
          const float kj = Kv(t0 + j, d);
          acc += Kv(t0 + i, d) * kj;
          if (for_backward) accq += Qv(t0 + i, d) * kj;
        }
        sKK[i * NS + j] = acc;
        if (for_backward) sQK[i * NS + j] = accq;
      }
    }
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f, accq = 0.f;
      for (int d = 0; d < DK; ++d) {
        const float hv = sH[d * CS + j];
        acc += Kv(t0 + i, d) * hv;
        if (for_backward) accq += Qv(t0 + i, d) * hv;
      }
      sKh[i * CS + j] = acc;
      if (for_backward) sQh[i * CS + j] = accq;
    }
    __syncthreads();
    // A (strict lower) into sM, then T = (I + A)^{-1}: thread j solves column j
    for (int e = tid; e < len * len; e += kBwdThreads) {
      const int i = e / len, j = e % len;
      sM[i * NS + j] = j < i ? sBet[i] * gam_ij(i, j) * sKK[i * NS + j] : 0.f;
    }
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      sVp[i * CS + j] = ldf(Vg, (int64_t)(t0 + i) * rv + j) - sGam[i] * sKh[i * CS + j];
    }
    __syncthreads();
    if (tid < len) {
      const int j = tid;
      for (int i = 0; i < len; ++i) {
        float x = i == j ? 1.f : 0.f;
        if (i > j)
          for (int m = j; m < i; ++m) x -= sM[i * NS + m] * sT[m * NS + j];
        sT[i * NS + j] = x;
      }
    }
    __syncthreads();
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int m = 0; m <= i; ++m) acc += sT[i * NS + m] * sBet[m] * sVp[m * CS + j];
      sU[i * CS + j] = acc;
    }
    __syncthreads();
  };

  auto chk = [&](int c) { return a.hchk + (((si.chunk0 + c) * H + h) * (int64_t)DK) * dv + col0; };

  // ================= forward sweep: the state at every chunk start =================
  for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
    const int i = e / kBwdCols, j = e % kBwdCols;
    sH[i * CS + j] = p.h0 ? p.h0[((int64_t)nh * DK + i) * dv + col0 + j] : 0.f;
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * kChunk, len = min(kChunk, si.len - t0);
    float* hc = chk(c);
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      hc[(int64_t)i * dv + j] = sH[i * CS + j];
    }
    recompute(t0, len, false);
    const float gn = expf(sG[len - 1]);
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int m = 0; m < len; ++m) acc += sD[m] * Kv(t0 + m, i) * sU[m * CS + j];
      sH[i * CS + j] = gn * sH[i * CS + j] + acc;
    }
    __syncthreads();
  }

  // ================= reverse sweep =================
  for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
    const int i = e / kBwdCols, j = e % kBwdCols;
    sdH[i * CS + j] = a.dhT ? a.dhT[((int64_t)nh * DK + i) * dv + col0 + j] : 0.f;
  }
  __syncthreads();
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * kChunk, len = min(kChunk, si.len - t0);
    const float* hc = chk(c);
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      sH[i * CS + j] = hc[(int64_t)i * dv + j];
    }
    __syncthreads();
    recompute(t0, len, true);
    const float gn = expf(sG[len - 1]);
    auto dY = [&](int i, int j) { return scale * ldf(DOg, (int64_t)(t0 + i) * rv + j); };
    // K dh' (into sdR for now) and dd_i = sum_j U_ij (K dh')_ij
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int d = 0; d < DK; ++d) acc += Kv(t0 + i, d) * sdH[d * CS + j];
      sdR[i * CS + j] = acc;
    }
    __syncthreads();
    if (tid < len) {
      float acc = 0.f;
      for (int j = 0; j < kBwdCols; ++j) acc += sU[tid * CS + j] * sdR[tid * CS + j];
      sDD[tid] = acc;
    }
    // dU = diag(d) K dh' + P^T dY,  P_mi = QK_mi Gamma_mi (i <= m)
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = sD[i] * sdR[i * CS + j];
      for (int m = i; m < len; ++m) acc += sQK[m * NS + i] * gam_ij(m, i) * dY(m, j);
      sdU[i * CS + j] = acc;
    }
    __syncthreads();
    // dR = T^T dU;  dP = lower(dY U^T) into sM
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = 0.f;
      for (int m = i; m < len; ++m) acc += sT[m * NS + i] * sdU[m * CS + j];
      sdR[i * CS + j] = acc;
    }
    for (int e = tid; e < len * len; e += kBwdThreads) {
      const int i = e / len, j = e % len;
      float acc = 0.f;
      if (j <= i)
        for (int k2 = 0; k2 < kBwdCols; ++k2) acc += dY(i, k2) * sU[j * CS + k2];
      sM[i * NS + j] = acc;
    }
    __syncthreads();
    // dV = diag(beta) dR; the Gamma gradient of P: E_ij = dP_ij QK_ij Gamma_ij
    E* dVg = reinterpret_cast<E*>(a.dv) + si.tok0 * rv + (int64_t)h * dv + col0;
    for (int e = tid; e < len * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      dVg[(int64_t)(t0 + i) * rv + j] = (E)(sBet[i] * sdR[i * CS + j]);
    }
    if (tid < len) {
      const int i = tid;
      float r = 0.f, cs = 0.f;
      for (int j = 0; j <= i; ++j) r += sM[i * NS + j] * sQK[i * NS + j] * gam_ij(i, j);
      for (int m = i; m < len; ++m) cs += sM[m * NS + i] * sQK[m * NS + i] * gam_ij(m, i);
      sdG[i] = r - cs;
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
    if (tid < len) {
      const int i = tid;
      float db = 0.f;
      for (int j = 0; j < kBwdCols; ++j) db += sdR[i * CS + j] * sVp[i * CS + j];
      float r = 0.f, cs = 0.f;
      for (int j = 0; j < i; ++j) {
        const float t = sM[i * NS + j] * sKK[i * NS + j] * gam_ij(i, j);
        db += t;
        r += sBet[i] * t;
      }
      for (int m = i + 1; m < len; ++m) cs += sBet[m] * sM[m * NS + i] * sKK[m * NS + i] * gam_ij(m, i);
      sdG[i] += r - cs;
      a.dbeta_p[((int64_t)blk * tot + si.tok0 + t0 + i) * H + h] = db;
    }
    __syncthreads();
    // sKK <- dB = diag(beta) dA * Gamma (strict lower; zero elsewhere)
    for (int e = tid; e < len * len; e += kBwdThreads) {
      const int i = e / len, j = e % len;
      sKK[i * NS + j] = j < i ? sBet[i] * sM[i * NS + j] * gam_ij(i, j) : 0.f;
    }
    __syncthreads();
    // shares of dQ and dK (the K K^T gradient enters as (dB + dB^T) K, merged)
    for (int e = tid; e < len * DK; e += kBwdThreads) {
      const int i = e / DK, d = e % DK;
      float dq = 0.f, dk = 0.f, hdy = 0.f, udh = 0.f, rvh = 0.f;
      for (int j = 0; j < kBwdCols; ++j) {
        const float hv = sH[d * CS + j];
        hdy += dY(i, j) * hv;
        udh += sU[i * CS + j] * sdH[d * CS + j];
        rvh += sBet[i] * sdR[i * CS + j] * hv;
      }
      dq = sGam[i] * hdy;
      dk = sD[i] * udh - sGam[i] * rvh;
      for (int m = 0; m < len; ++m) {
        const float km = Kv(t0 + m, d);
        if (m <= i) dq += sQK[i * NS + m] * km;
        if (m >= i) dk += sQK[m * NS + i] * Qv(t0 + m, d);
        dk += (sKK[i * NS + m] + sKK[m * NS + i]) * km;
      }
      const int64_t o = (((int64_t)blk * tot + si.tok0 + t0 + i) * H + h) * DK + d;
      a.dq_p[o] = dq;
      a.dk_p[o] = dk;
    }
    // gamma_n's gradient: <h, dh'> over this block's columns (workgroup reduction)
    float part = 0.f;
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      part += sH[i * CS + j] * sdH[i * CS + j];
    }
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) sRed[wave] = part;
    // the gamma and d gradients into dG
    if (tid < len) {
      const int i = tid;
      float dgam = 0.f;
      for (int j = 0; j < kBwdCols; ++j)
        dgam += sQh[i * CS + j] * dY(i, j) - sBet[i] * sdR[i * CS + j] * sKh[i * CS + j];
      sdG[i] += dgam * sGam[i] - sDD[i] * sD[i];
    }
    __syncthreads();
    if (tid == 0) {
      float dgn = 0.f, ddd = 0.f;
      for (int w = 0; w < kBwdThreads / 64; ++w) dgn += sRed[w];
      for (int m = 0; m < len; ++m) ddd += sDD[m] * sD[m];
      sdG[len - 1] += ddd + dgn * gn;
    }
    __syncthreads();
    // dg share = reverse cumsum of dG over the chunk
    if (tid < len) {
      float acc = 0.f;
      for (int m = tid; m < len; ++m) acc += sdG[m];
      a.dg_p[((int64_t)blk * tot + si.tok0 + t0 + tid) * H + h] = acc;
    }
    // dh = gamma_n dh' + Q^T diag(gamma) dY - K^T diag(gamma beta) dR (in place)
    for (int e = tid; e < DK * kBwdCols; e += kBwdThreads) {
      const int i = e / kBwdCols, j = e % kBwdCols;
      float acc = gn * sdH[i * CS + j];
      for (int m = 0; m < len; ++m)
        acc += sGam[m] * (Qv(t0 + m, i) * dY(m, j) - Kv(t0 + m, i) * sBet[m] * sdR[m * CS + j]);
      sdH[i * CS + j] = acc;
    }
    __syncthreads();
  }
  if (a.dh0) {
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
  const int64_t wgs = (int64_t)p.N * p.H * nblk;
  if (wgs > kMaxDispatchItems / kBwdThreads) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL(chunk_bwd_kernel<E, DK>, dim3((unsigned)wgs), dim3(kBwdThreads), 0, s, ev.start, nullptr,
                        0, p, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
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
  if (a.total_tokens == 0 && (int64_t)p.N * p.H == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (p.dv % kBwdCols != 0) return hipErrorInvalidValue;
  if (p.qkv_bf16)
    return p.dk == 128 ? launch_bwd_dk<bf16, 128>(p, a, s, ev) : launch_bwd_dk<bf16, 64>(p, a, s, ev);
  return p.dk == 128 ? launch_bwd_dk<float, 128>(p, a, s, ev) : launch_bwd_dk<float, 64>(p, a, s, ev);
}

}  // namespace gdn
