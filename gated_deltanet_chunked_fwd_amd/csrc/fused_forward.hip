// Steps 2-4 of the chunked WY form, fused, on gfx950: per (sequence, head,
// value-column block, segment) a workgroup walks the chunks in order with the
// state resident in registers, and writes only O and the final state.
//
// FlashQLA talk transcript (tokendh.com): chunked-WY section (W/U projections,
// chunk-serial state recurrence, output from the state); pain-points section
// (W, U and S must not round-trip through HBM); algebraic-rewrites section
// (forward merge: form "V minus S" first, then apply gamma).  With h = S^T the
// state at chunk start, G the chunk-local cumsum of g, gamma = exp(G),
// Gamma_rs = exp(G_r - G_s) (r >= s) and T from step 1:
//
//   V' = V - diag(gamma) K h                      (merged W/U form)
//   U  = T diag(beta) V'
//   O  = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)
//   h <- gamma_last h + (diag(exp(G_last - G)) K)^T U
//
// Mapping.  256 threads = 4 waves; each wave owns NCW value columns of h for
// all dk rows, as 16x16 fp32 accumulator tiles in "tile order" (see
// gdn_device.h), so h, V' and U feed the next MFMA directly from registers.
// Each chunk's K, Q, K~^T (decay-scaled, transposed), T, P = (QK^T)*Gamma and
// the wave's V columns are staged in LDS and read as MFMA A operands.  The
// value columns are independent: only T and P are shared between them.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename E, int DK, int NCW>
struct FwdCfg {
  static constexpr int NWAVES = 4;
  static constexpr int BV = NWAVES * NCW;   // value columns per workgroup
  static constexpr int NCT = NCW / 16;      // column tiles per wave
  static constexpr int NKT = DK / 16;       // dk tiles of the state
  static constexpr int NKS = DK / 32;       // contraction steps over dk
  static constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
  static constexpr int KS = DK + PAD;       // row stride of sK, sQ
  static constexpr int CS = kChunk + PAD;   // row stride of sKt, sT, sP
  static constexpr int VS = BV + PAD;       // row stride of sV
  static constexpr int EPV = 16 / (int)sizeof(E);
};

template <typename E, int DK, int NCW>
__global__ __launch_bounds__(256) void fused_forward_kernel(Problem p, FwdPlan plan) {
  using Cfg = FwdCfg<E, DK, NCW>;
  using M = Mma<E>;
  using frag = typename M::frag;
  constexpr int BV = Cfg::BV, NCT = Cfg::NCT, NKT = Cfg::NKT, NKS = Cfg::NKS;
  constexpr int KS = Cfg::KS, CS = Cfg::CS, VS = Cfg::VS, EPV = Cfg::EPV;

  __shared__ __align__(16) E sK[kChunk * KS];
  __shared__ __align__(16) E sQ[kChunk * KS];
  __shared__ __align__(16) E sKt[DK * CS];
  __shared__ __align__(16) E sT[kChunk * CS];
  __shared__ __align__(16) E sP[kChunk * CS];
  __shared__ __align__(16) E sV[kChunk * VS];
  __shared__ float sGraw[kChunk], sBraw[kChunk];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int H = p.H, dv = p.dv;
  const int col0 = blockIdx.y * BV;        // first value column of the workgroup
  const int wcol = wave * NCW;             // wave's first column inside the block

  const int64_t unit = blockIdx.x;
  const int h = (int)(unit % H);
  const int64_t sg = unit / H;             // global segment index
  int n, seg;
  if (plan.seg_off) {
    n = seq_of_chunk(sg, plan.seg_off, p.N, 0);
    seg = (int)(sg - plan.seg_off[n]);
  } else {
    const int64_t nch_all = (p.T + kChunk - 1) / kChunk;
    const int64_t segs = (nch_all + plan.seg_chunks - 1) / plan.seg_chunks;
    n = (int)(sg / (segs > 0 ? segs : 1));
    seg = (int)(sg - (int64_t)n * segs);
  }
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int c_begin = seg * plan.seg_chunks;
  const int c_end = min(nch, c_begin + plan.seg_chunks);

  const E* Q = reinterpret_cast<const E*>(p.q);
  const E* K = reinterpret_cast<const E*>(p.k);
  const E* V = reinterpret_cast<const E*>(p.v);
  const E* Tm = reinterpret_cast<const E*>(plan.Tmat);
  E* O = reinterpret_cast<E*>(p.o);

  // ---- initial state
  f32x4 hs[NKT][NCT];
  const int64_t st_off = ((int64_t)n * H + h) * DK * dv;
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hs[t][ct][i] = (p.h0 && seg == 0)
                           ? p.h0[st_off + (int64_t)prow(t, 4 * q + i) * dv + col0 + wcol + ct * 16 + r16]
                           : 0.f;

  for (int c = c_begin; c < c_end; ++c) {
    const int64_t r0 = si.tok0 + (int64_t)c * kChunk;
    const int len = min(kChunk, si.len - c * kChunk);

    // ---- stage the chunk in LDS (rows past the end are zero)
    {
      constexpr int VPR = DK / EPV;
      for (int i = tid; i < kChunk * VPR; i += 256) {
        const int r = i / VPR, cv = i % VPR;
        u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (r < len) {
          const int64_t off = ((r0 + r) * H + h) * DK + cv * EPV;
          kv = *reinterpret_cast<const u32x4*>(K + off);
          qv = *reinterpret_cast<const u32x4*>(Q + off);
        }
        *reinterpret_cast<u32x4*>(sK + r * KS + cv * EPV) = kv;
        *reinterpret_cast<u32x4*>(sQ + r * KS + cv * EPV) = qv;
      }
      constexpr int VPRV = BV / EPV;
      for (int i = tid; i < kChunk * VPRV; i += 256) {
        const int r = i / VPRV, cv = i % VPRV;
        u32x4 vv = {0u, 0u, 0u, 0u};
        if (r < len) vv = *reinterpret_cast<const u32x4*>(V + ((r0 + r) * H + h) * dv + col0 + cv * EPV);
        *reinterpret_cast<u32x4*>(sV + r * VS + cv * EPV) = vv;
      }
      constexpr int VPRT = kChunk / EPV;
      const E* tsrc = Tm + ((si.chunk0 + c) * H + h) * (int64_t)(kChunk * kChunk);
      for (int i = tid; i < kChunk * VPRT; i += 256) {
        const int r = i / VPRT, cv = i % VPRT;
        *reinterpret_cast<u32x4*>(sT + r * CS + cv * EPV) =
            *reinterpret_cast<const u32x4*>(tsrc + r * kChunk + cv * EPV);
      }
      if (wave == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < len) {
          gv = p.g[(r0 + lane) * H + h];
          bv = load_scalar(p.beta, (r0 + lane) * H + h, p.beta_bf16);
        }
        sGraw[lane] = gv;
        sBraw[lane] = bv;
      }
    }
    __syncthreads();

    // ---- gates (every wave keeps its own copy; lane = chunk row)
    const float G = wave_inclusive_scan(sGraw[lane]);
    const float Glast = __shfl(G, 63, 64);
    const float gam_l = fast_exp(G);
    const float dec_l = fast_exp(Glast - G);
    const float gC = fast_exp(Glast);
    const float bet_l = sBraw[lane];

    // ---- K~^T: decay-scaled, transposed keys (wave w handles dk groups of 8)
#pragma unroll
    for (int jj = 0; jj < DK / 32; ++jj) {
      const int j = wave * (DK / 32) + jj;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sKt[(8 * j + e) * CS + lane] = from_f32<E>(to_f32(sK[lane * KS + 8 * j + e]) * dec_l);
    }
    // ---- P = (Q K^T) * Gamma, row tile = wave (natural row order)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (v <= wave) {
#pragma unroll
        for (int s = 0; s < NKS; ++s)
          acc = M::run(lds_frag(sQ, KS, 16 * wave + r16, 32 * s, q),
                       lds_frag(sK, KS, 16 * v + r16, 32 * s, q), acc);
      }
      const int col = 16 * v + r16;
      const float Gcol = __shfl(G, col, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * q + i;
        const float Grow = __shfl(G, row, 64);
        const float val = (col <= row) ? acc[i] * fast_exp(Grow - Gcol) : 0.f;
        sP[row * CS + col] = from_f32<E>(val);
      }
    }
    // per-row gate values in tile order
    float gam_r[4][4], bet_r[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gam_r[u][i] = __shfl(gam_l, prow(u, 4 * q + i), 64);
        bet_r[u][i] = __shfl(bet_l, prow(u, 4 * q + i), 64);
      }
    __syncthreads();

    // ---- X = K h, Y = Q h
    f32x4 X[4][NCT], Y[4][NCT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        X[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        Y[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      frag hb[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) hb[ct] = M::pack(hs[2 * s][ct], hs[2 * s + 1][ct]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const frag aK = lds_frag(sK, KS, prow(u, r16), 32 * s, q);
        const frag aQ = lds_frag(sQ, KS, prow(u, r16), 32 * s, q);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          X[u][ct] = M::run(aK, hb[ct], X[u][ct]);
          Y[u][ct] = M::run(aQ, hb[ct], Y[u][ct]);
        }
      }
    }
    // ---- W = diag(beta) (V - diag(gamma) X), in place
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = prow(u, 4 * q + i);
          const float vv = to_f32(sV[row * VS + wcol + ct * 16 + r16]);
          X[u][ct][i] = bet_r[u][i] * (vv - gam_r[u][i] * X[u][ct][i]);
        }
    // ---- U = T W (T lower triangular: row tiles 0,1 need contraction step 0 only)
    frag wb[2][NCT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) wb[s][ct] = M::pack(X[2 * s][ct], X[2 * s + 1][ct]);
    f32x4 U[4][NCT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) U[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= (u >> 1); ++s) {
        const frag aT = lds_frag(sT, CS, prow(u, r16), 32 * s, q);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) U[u][ct] = M::run(aT, wb[s][ct], U[u][ct]);
      }
    }
    frag ub[2][NCT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) ub[s][ct] = M::pack(U[2 * s][ct], U[2 * s + 1][ct]);
    // ---- O = scale (diag(gamma) Y + P U)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[u][ct][i] *= gam_r[u][i];
#pragma unroll
      for (int s = 0; s <= (u >> 1); ++s) {
        const frag aP = lds_frag(sP, CS, prow(u, r16), 32 * s, q);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Y[u][ct] = M::run(aP, ub[s][ct], Y[u][ct]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = prow(u, 4 * q + i);
        if (row < len) {
          E* dst = O + ((r0 + row) * H + h) * dv + col0 + wcol + r16;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) dst[ct * 16] = from_f32<E>(p.scale * Y[u][ct][i]);
        }
      }
    }
    // ---- h <- gamma_last h + K~^T U
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) hs[t][ct] *= gC;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const frag aKt = lds_frag(sKt, CS, prow(t, r16), 32 * s, q);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) hs[t][ct] = M::run(aKt, ub[s][ct], hs[t][ct]);
      }
    }
    __syncthreads();
  }

  if (p.hT) {
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p.hT[st_off + (int64_t)prow(t, 4 * q + i) * dv + col0 + wcol + ct * 16 + r16] = hs[t][ct][i];
  }
}

template <typename E, int DK>
static void launch_dk(const Problem& p, const FwdPlan& plan, hipStream_t s) {
  if constexpr (sizeof(E) == 2) {  // fp32 tiles only fit LDS at 64 columns per workgroup
    if (p.dv % 128 == 0) {
      dim3 grid((unsigned)plan.units, (unsigned)(p.dv / 128));
      fused_forward_kernel<E, DK, 32><<<grid, 256, 0, s>>>(p, plan);
      return;
    }
  }
  dim3 grid((unsigned)plan.units, (unsigned)(p.dv / 64));
  fused_forward_kernel<E, DK, 16><<<grid, 256, 0, s>>>(p, plan);
}

hipError_t launch_fused_forward(const Problem& p, const FwdPlan& plan, hipStream_t s) {
  if (plan.units == 0) return hipSuccess;
  if (p.qkv_bf16) {
    if (p.dk == 128) launch_dk<bf16, 128>(p, plan, s);
    else launch_dk<bf16, 64>(p, plan, s);
  } else {
    if (p.dk == 128) launch_dk<float, 128>(p, plan, s);
    else launch_dk<float, 64>(p, plan, s);
  }
  return hipGetLastError();
}

}  // namespace gdn
