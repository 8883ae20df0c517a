// Backward of the chunked GDN forward on gfx950 for bf16 q / k / v: bf16 MFMA
// products with fp32 accumulation, in two kernels.
//
// FlashQLA talk transcript (tokendh.com): results and timeline sections (the
// backward keeps the forward's chunked structure); algebraic-rewrites section (the
// K K^T gradient reaches K once, as (dB + dB^T) K).  The chunk algebra is the
// forward's, with h = S^T the state at the chunk's start, G the chunk-local cumsum
// of g, gamma = exp(G), Gamma_ij = exp(G_i - G_j) (j <= i), d = exp(G_n - G),
// gamma_n = exp(G_n) (G_n: the chunk's last row):
//
//   A = strict_lower(diag(beta) K K^T * Gamma),  T = (I + A)^{-1}
//   V' = V - diag(gamma) K h,  U = T diag(beta) V',  P = (Q K^T) * Gamma (j <= i)
//   O = scale (diag(gamma) Q h + P U),  h' = gamma_n h + K^T diag(d) U
//
// 1. bwd_dh_kernel: the state-gradient chain, serial over a sequence's chunks from
//    last to first, per (sequence or segment, head, 32 value columns).  With dh' the
//    gradient of the state after the chunk and dY = scale dO:
//      X' = K dh',  dU = diag(d) X' + P^T dY,  dR = T^T dU,  dV = diag(beta) dR
//      dh = gamma_n dh' + Q^T diag(gamma) dY - K^T diag(gamma) dV
//    dV is final; dh' of every chunk goes to a checkpoint (fp32), the gradient at the
//    sequence's start to dh0.  It needs no forward state: only K, Q, dO, T and gates.
// 2. bwd_grads_kernel: every (chunk, head) on its own, from the forward's state h at
//    the chunk's start and the chain's dh' at its end:
//      dP = lower(dY U^T),  dA = strict_lower(-dR U^T),  dB = diag(beta) dA * Gamma
//      dQ = diag(gamma) dY h^T + (dP * Gamma) K
//      dK = diag(d) U dh'^T + (dP * Gamma)^T Q - diag(gamma) dV h^T + (dB + dB^T) K
//      dbeta_i = sum_c dR_ic V'_ic + sum_j dA_ij (K K^T)_ij Gamma_ij
//      dG_i (per row, from every place G enters):
//        Gamma in P and A:  + sum_j dP_ij P_ij - sum_j dP_ji P_ji  (and the same with dA, A)
//        gamma in V' and O: + sum_d K_id (-gamma_i dV h^T)_id + sum_d Q_id (gamma_i dY h^T)_id
//        d in the update:   - d_i sum_c X'_ic U_ic, and the sum over i of d_i sum_c X'_ic U_ic
//                           plus gamma_n <h, dh'> to the last row (G_n)
//      dg = the reverse cumulative sum of dG inside the chunk.
//    dQ and dK contract over all value columns inside one workgroup, so they are
//    written once, in bf16, with no partial sums.
//
// Every product is v_mfma_f32_16x16x32_bf16 on operands read from LDS: a matrix is
// stored row-major with natural rows, and an operand whose contraction index runs
// along a row is a 16-byte read (op_rows), one whose contraction runs down a column a
// transposing read (op_cols, ds_read_b64_tr_b16).  Accumulator tiles: lane l = 16 q
// + r holds (row 4 q + i, column r) in slot i.  Rows past a partial chunk's end
// are zero in K, Q, dO and V, and their g and beta are zero, so they contribute
// nothing; the chunk inverse leaves them the identity.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

using Mb = Mma<bf16>;
using frag = bf16x8;

// A or B operand of one 32-wide contraction step, index (the operand's row for A,
// column for B) idx0 + r, contraction k0 + 8 q + e:
//   op_rows: from a matrix stored [index][contraction] (16-byte read);
//   op_cols: from a matrix stored [contraction][index] (transposing read).
__device__ __forceinline__ frag op_rows(const bf16* m, int stride, int idx0, int k0) {
  const int l = threadIdx.x & 63;
  return *reinterpret_cast<const frag*>(m + (idx0 + (l & 15)) * stride + k0 + 8 * (l >> 4));
}
__device__ __forceinline__ frag op_cols(const bf16* m, int stride, int k0, int idx0) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  return col_frag(m, stride, k0 + 8 * q, k0 + 8 * q + 4, idx0 + r, idx0 + 4 * (r & 3));
}

// The ten 16 x 16 blocks (a, b), b <= a, of a lower-triangular 64 x 64 chunk matrix.
__device__ __forceinline__ void tri_block(int k, int& a, int& b) {
  a = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
  b = k - (a * (a + 1)) / 2;
}

// Sum over the 16 lanes of a lane group (one accumulator row's columns).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float beta_at(const void* beta, int64_t i, bool is_bf16) {
  return is_bf16 ? (float)reinterpret_cast<const bf16*>(beta)[i] : reinterpret_cast<const float*>(beta)[i];
}

// (sequence, head, segment) of a backward unit (segments as in the forward's split:
// seg_off for packed input, else the same count for every sequence).
struct BwdUnit {
  int n, h, seg, S;
  int64_t sg0;
};
__device__ __forceinline__ BwdUnit bwd_unit(const Problem& p, const BwdArgs& a, int64_t unit) {
  BwdUnit u;
  u.seg = 0;
  u.S = 1;
  u.sg0 = 0;
  if (a.seg_chunks > 0) {
    u.h = (int)(unit % p.H);
    const int64_t sg = unit / p.H;
    if (a.seg_off) {
      u.n = seq_of_chunk(sg, a.seg_off, p.N, 0);
      u.sg0 = a.seg_off[u.n];
      u.S = (int)(a.seg_off[u.n + 1] - u.sg0);
    } else {
      const int64_t segs = max((int64_t)1, ((p.T + kChunk - 1) / kChunk + a.seg_chunks - 1) / a.seg_chunks);
      u.n = (int)(sg / segs);
      u.sg0 = (int64_t)u.n * segs;
      u.S = (int)segs;
    }
    u.seg = (int)(sg - u.sg0);
  } else {
    u.n = (int)(unit / p.H);
    u.h = (int)(unit % p.H);
  }
  return u;
}

// Workgroup barrier for LDS data: this wave's LDS accesses complete, then s_barrier.
// Unlike __syncthreads it does not wait for the wave's outstanding global stores (no
// data written to global memory is read back inside these kernels).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kDhCols = 32;     // value columns per chain workgroup
constexpr int kDhThreads = 256;
constexpr int kGrThreads = 512;
constexpr int kTS = 80;         // row stride (elements) of 64 x 64 LDS matrices: rows
                                // 8 (mod 32) dwords apart, as every LDS matrix here

}  // namespace

// ============================ 1. the state-gradient chain ============================
// Workgroup = (unit, 32 value columns), four waves.  Wave w owns row tile w of every
// 64 x 32 chunk result and dk rows [DK/4 w, DK/4 (w+1)) of the state gradient (in
// fp32 registers; a bf16 copy in LDS feeds X').  One chunk ahead, every thread loads
// its share of the next chunk's K, Q, dO and T rows into registers.
template <int DK>
__global__ __launch_bounds__(kDhThreads) void bwd_dh_kernel(Problem p, BwdArgs a) {
  constexpr int BV = kDhCols, NT = kDhThreads;
  constexpr int KS = DK + 16, TS = kTS, VS = BV + 16, HS = BV + 16;
  constexpr int NKS = DK / 32;       // contraction steps over dk
  constexpr int NKP = DK / 32;       // 16-byte pieces of K (and of Q) per thread and chunk
  constexpr int NRT = DK / 64;       // state row tiles per wave
  __shared__ __align__(16) bf16 sK[kChunk * KS], sQ[kChunk * KS], sT[kChunk * TS], sP[kChunk * TS];
  __shared__ __align__(16) bf16 sDO[kChunk * VS], sGY[kChunk * VS], sDU[kChunk * VS], sGV[kChunk * VS],
      sDV[kChunk * VS];
  __shared__ __align__(16) bf16 sH[DK * HS];
  __shared__ float sG[kChunk], sGam[kChunk], sD[kChunk], sBet[kChunk];
  __shared__ float sHD[NT / 64];

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware numbering: the column blocks of one unit share blockIdx mod 8, so they
  // run on one XCD and share its L2 for K, Q and T
  const int nblk = p.dv / BV;
  const uint32_t bid = blockIdx.x, rest = bid >> 3;
  const int blk = (int)(rest % (uint32_t)nblk);
  const int64_t unit = (int64_t)(rest / (uint32_t)nblk) * 8 + (bid & 7u);
  if (unit >= a.units) return;
  const BwdUnit U = bwd_unit(p, a, unit);
  const bool chain = a.mode == kBwdChain;
  if (chain && U.seg == 0) return;   // the merge needs no offset of a first segment
  const int h = U.h, H = p.H, dv = p.dv, col0 = blk * BV;
  const int64_t nh = (int64_t)U.n * H + h;
  const SeqInfo si = seq_info(U.n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int c_lo = a.seg_chunks > 0 ? min(nch, U.seg * a.seg_chunks) : 0;
  const int c_hi = a.seg_chunks > 0 ? min(nch, (U.seg + 1) * a.seg_chunks) : nch;
  const int64_t rqk = (int64_t)H * DK, rv = (int64_t)H * dv;
  const bf16* Kg = reinterpret_cast<const bf16*>(p.k) + si.tok0 * rqk + (int64_t)h * DK;
  const bf16* Qg = reinterpret_cast<const bf16*>(p.q) + si.tok0 * rqk + (int64_t)h * DK;
  const bf16* DOg = reinterpret_cast<const bf16*>(a.d_o) + si.tok0 * rv + (int64_t)h * dv + col0;
  bf16* DVg = reinterpret_cast<bf16*>(a.dv) + si.tok0 * rv + (int64_t)h * dv + col0;
  const bf16* Tg = reinterpret_cast<const bf16*>(a.tmat);
  const float* Gg = p.g + si.tok0 * H + h;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // P's blocks above the diagonal stay zero (only the lower ones are rewritten)
  for (int e = tid; e < kChunk * TS / 8; e += NT) reinterpret_cast<u32x4*>(sP)[e] = z4;

  // ---- the state gradient after the unit's last chunk: dhT for a sequence's last
  //      segment (or a whole sequence), the merge's result for the other segments,
  //      zero in the chain pass
  const int64_t gslot = bwd_slot(U.sg0, U.S, U.seg) * H + h;
  f32x4 dh[NRT][2];
#pragma unroll
  for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * (NRT * w + tt) + 4 * q + i, c = 16 * j + r;
        float x = 0.f;
        if (!chain) {
          if (U.seg == U.S - 1) x = a.dhT ? a.dhT[(nh * DK + d) * dv + col0 + c] : 0.f;
          else x = a.seg_g[(gslot * DK + d) * dv + col0 + c];
        }
        dh[tt][j][i] = x;
        sH[d * HS + c] = (bf16)x;
      }

  // ---- one chunk's inputs, loaded into registers a chunk ahead (the forward state at
  //      the chunk's start, for gamma_n <h, dh'>, in the layout of this lane's dh')
  u32x4 pk[NKP], pq[NKP], po, pt[2];
  f32x4 ph[NRT][2];
  float pg = 0.f, pb = 0.f;
  auto load = [&](int c) {
    const int len = min(kChunk, si.len - c * kChunk);
    const int64_t t0 = (int64_t)c * kChunk;
#pragma unroll
    for (int k = 0; k < NKP; ++k) {
      const int idx = tid + NT * k, row = idx / (DK / 8), cp = idx % (DK / 8);
      const int64_t off = (t0 + row) * rqk + cp * 8;
      pk[k] = row < len ? *reinterpret_cast<const u32x4*>(Kg + off) : z4;
      pq[k] = row < len ? *reinterpret_cast<const u32x4*>(Qg + off) : z4;
    }
    {
      const int row = tid >> 2, cp = tid & 3;
      po = row < len ? *reinterpret_cast<const u32x4*>(DOg + (t0 + row) * rv + cp * 8) : z4;
    }
    const bf16* Tc = Tg + ((si.chunk0 + c) * H + h) * (int64_t)(kChunk * kChunk);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid + NT * k, row = idx >> 3, cp = idx & 7;
      pt[k] = *reinterpret_cast<const u32x4*>(Tc + row * kChunk + cp * 8);
    }
    if (w == 0) {
      pg = lane < len ? Gg[(t0 + lane) * H] : 0.f;
      pb = lane < len ? beta_at(p.beta, (si.tok0 + t0 + lane) * H + h, p.beta_bf16) : 0.f;
    }
    if (!chain) {
      const float* hc = a.hchk + ((si.chunk0 + c) * H + h) * (int64_t)DK * dv;
#pragma unroll
      for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          ph[tt][j] = *reinterpret_cast<const f32x4*>(hc + ckpt_offset(16 * (NRT * w + tt) + 4 * q, col0 + 16 * j + r, dv));
    }
  };
  // dV of chunk c (16-byte stores of the rows inside the chunk) from sDV; the
  // checkpoint of the state gradient after chunk c from the registers, as its bf16
  // transpose as a hi + lo pair (hi block, then lo block; four keys of one value column
  // per 8-byte store); this wave's share of
  // gamma_n <h, dh'> into sHD (hd: this lane's <h, dh'> terms, formed at the top of the
  // step; the workgroup's sum is written at the next step)
  auto store_dv = [&](int c) {
    const int len = min(kChunk, si.len - c * kChunk);
    const int row = tid >> 2, cp = tid & 3;
    if (row < len)
      *reinterpret_cast<u32x4*>(DVg + ((int64_t)c * kChunk + row) * rv + cp * 8) =
          *reinterpret_cast<const u32x4*>(sDV + row * VS + cp * 8);
  };
  auto store_ckpt = [&](int c, float hd) {
    bf16* ck = reinterpret_cast<bf16*>(a.dhchk) + ((si.chunk0 + c) * H + h) * (int64_t)2 * DK * dv;
#pragma unroll
    for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t at = (int64_t)(col0 + 16 * j + r) * DK + 16 * (NRT * w + tt) + 4 * q;
        const uint2 hi = pack_bf16x4(dh[tt][j]);
        *reinterpret_cast<uint2*>(ck + at) = hi;
        const bf16x4 hb = __builtin_bit_cast(bf16x4, hi);
        f32x4 lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = dh[tt][j][i] - (float)hb[i];
        *reinterpret_cast<uint2*>(ck + (int64_t)DK * dv + at) = pack_bf16x4(lo);
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hd += __shfl_xor(hd, off, 64);
    if (lane == 0) sHD[w] = fast_exp(sG[kChunk - 1]) * hd;
  };
  // the workgroup's gamma_n <h, dh'> of chunk c, once sHD is complete
  auto store_gnh = [&](int c) {
    if (tid == 0) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < NT / 64; ++k) s += sHD[k];
      a.gnh[((si.chunk0 + c) * H + h) * nblk + blk] = s;
    }
  };
  if (c_hi > c_lo) load(c_hi - 1);
  lds_barrier();

  for (int c = c_hi - 1; c >= c_lo; --c) {
    if (!chain && c + 1 < c_hi) store_gnh(c + 1);
    // ---- this chunk into LDS; the gates (wave 0); the next chunk's loads
#pragma unroll
    for (int k = 0; k < NKP; ++k) {
      const int idx = tid + NT * k, row = idx / (DK / 8), cp = idx % (DK / 8);
      *reinterpret_cast<u32x4*>(sK + row * KS + cp * 8) = pk[k];
      *reinterpret_cast<u32x4*>(sQ + row * KS + cp * 8) = pq[k];
    }
    *reinterpret_cast<u32x4*>(sDO + (tid >> 2) * VS + (tid & 3) * 8) = po;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid + NT * k;
      *reinterpret_cast<u32x4*>(sT + (idx >> 3) * TS + (idx & 7) * 8) = pt[k];
    }
    if (w == 0) {
      const float G = wave_inclusive_scan_dpp(pg);
      const float Gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
      sG[lane] = G;
      sGam[lane] = fast_exp(G);
      sD[lane] = fast_exp(Gn - G);
      sBet[lane] = pb;
    }
    // <h, dh'> of this chunk, before the next chunk's loads take ph
    float hdc = 0.f;
    if (!chain) {
#pragma unroll
      for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) hdc += ph[tt][j][i] * dh[tt][j][i];
    }
    if (c > c_lo) load(c - 1);
    lds_barrier();

    // ---- P = (Q K^T) * Gamma (lower blocks); gamma * scale * dO; X' = K dh'
    for (int k = w; k < 10; k += 4) {
      int ba, bb;
      tri_block(k, ba, bb);
      f32x4 acc = zero4;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc = Mb::run(op_rows(sQ, KS, 16 * ba, 32 * ks), op_rows(sK, KS, 16 * bb, 32 * ks), acc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = 16 * ba + 4 * q + s, j = 16 * bb + r;
        sP[i * TS + j] = (bf16)(j <= i ? acc[s] * fast_exp(sG[i] - sG[j]) : 0.f);
      }
    }
    {
      const int row = tid >> 2, cp = tid & 3;
      const float f = sGam[row] * p.scale;
      const frag x = *reinterpret_cast<const frag*>(sDO + row * VS + cp * 8);
      frag y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (bf16)((float)x[e] * f);
      *reinterpret_cast<frag*>(sGY + row * VS + cp * 8) = y;
    }
    f32x4 X[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      X[j] = zero4;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        X[j] = Mb::run(op_rows(sK, KS, 16 * w, 32 * ks), op_cols(sH, HS, 32 * ks, 16 * j), X[j]);
    }
    lds_barrier();

    // ---- dU = diag(d) X' + scale P^T dO (P^T is upper triangular)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 acc = zero4;
      for (int ks = w >> 1; ks < 2; ++ks)
        acc = Mb::run(op_cols(sP, TS, 32 * ks, 16 * w), op_cols(sDO, VS, 32 * ks, 16 * j), acc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = 16 * w + 4 * q + s;
        sDU[i * VS + 16 * j + r] = (bf16)(sD[i] * X[j][s] + p.scale * acc[s]);
      }
    }
    lds_barrier();

    // ---- dR = T^T dU, dV = diag(beta) dR
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 acc = zero4;
      for (int ks = w >> 1; ks < 2; ++ks)
        acc = Mb::run(op_cols(sT, TS, 32 * ks, 16 * w), op_cols(sDU, VS, 32 * ks, 16 * j), acc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = 16 * w + 4 * q + s;
        const float dvv = sBet[i] * acc[s];
        sDV[i * VS + 16 * j + r] = (bf16)dvv;
        sGV[i * VS + 16 * j + r] = (bf16)(-sGam[i] * dvv);
      }
    }
    lds_barrier();

    if (!chain) {
      store_dv(c);
      store_ckpt(c, hdc);
    }
    // ---- dh <- gamma_n dh' + Q^T (gamma dY) - K^T (gamma dV)
    const float gn = fast_exp(sG[kChunk - 1]);
#pragma unroll
    for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = NRT * w + tt;
        f32x4 acc = dh[tt][j] * gn;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc = Mb::run(op_cols(sQ, KS, 32 * ks, 16 * t), op_cols(sGY, VS, 32 * ks, 16 * j), acc);
          acc = Mb::run(op_cols(sK, KS, 32 * ks, 16 * t), op_cols(sGV, VS, 32 * ks, 16 * j), acc);
        }
        dh[tt][j] = acc;
#pragma unroll
        for (int s = 0; s < 4; ++s) sH[(16 * t + 4 * q + s) * HS + 16 * j + r] = (bf16)acc[s];
      }
    lds_barrier();
  }

  if (!chain && c_hi > c_lo) store_gnh(c_lo);
  if (chain) {
    // the state gradient at the segment's start from a zero one at its end: the merge's
    // offset for this segment (accumulator-tile order, as the forward's S*)
    float* dst = a.seg_b + gslot * (int64_t)DK * dv;
#pragma unroll
    for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[sfrag_offset<DK>(16 * (NRT * w + tt) + 4 * q + i, col0 + 16 * j + r)] = dh[tt][j][i];
  } else if (a.dh0 && U.seg == 0) {
#pragma unroll
    for (int tt = 0; tt < NRT; ++tt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dh0[(nh * DK + 16 * (NRT * w + tt) + 4 * q + i) * dv + col0 + 16 * j + r] = dh[tt][j][i];
  }
}

// ========================= 2. the gradients of every chunk =========================
// Workgroup = (chunk, head), eight waves.  Wave w owns row tile u = w % 4 of the
// 64 x dv and 64 x dk results, column tiles [NJ (w / 4), NJ (w / 4 + 1)), and the
// lower 64 x 64 blocks w and w + 8, the same tiles in every product so that the row
// sums of dbeta and dG pair registers lane by lane.
template <int DK, int DV>
__global__ __launch_bounds__(kGrThreads) void bwd_grads_kernel(Problem p, BwdArgs a) {
  constexpr int NT = kGrThreads, NW = NT / 64;
  constexpr int KS = DK + 16, VS = DV + 16, HS = DK + 16, TS = kTS;
  constexpr int NKS = DK / 32, NVS = DV / 32;
  constexpr int NJV = DV / 32, NJK = DK / 32;   // column tiles per wave: 64 x dv, 64 x dk results
  constexpr int RF = (kChunk * VS > kChunk * TS) ? kChunk * VS : kChunk * TS;
  constexpr int RG = RF;
  static_assert(DV * HS >= kChunk * TS, "dB + dB^T fits the h^T region");
  constexpr int NHP = DK * DV / 4 / NT;         // 16-byte checkpoint pieces per thread
  static_assert(NHP * NT * 4 == DK * DV, "checkpoint pieces");
  __shared__ __align__(16) bf16 sK[kChunk * KS], sQ[kChunk * KS], sDO[kChunk * VS], sT[kChunk * TS];
  __shared__ __align__(16) bf16 sH[DV * HS];   // h^T, then W's low half, then dh'^T, then dB + dB^T
  __shared__ __align__(16) bf16 sF[RF];        // diag(beta) V', then dU, then dP * Gamma
  __shared__ __align__(16) bf16 sR[RG];        // P, then dR
  __shared__ __align__(16) bf16 sU[kChunk * VS];
  __shared__ float sG[kChunk], sGam[kChunk], sD[kChunk], sBet[kChunk];
  __shared__ float sPG[NW][kChunk], sPB[NW][kChunk], sPN[NW];

  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = w & 3, half = w >> 2;
  const int H = p.H;
  const int h = (int)(blockIdx.x % (uint32_t)H);
  const int64_t cg = blockIdx.x / (uint32_t)H;
  const int n = seq_of_chunk(cg, p.chunk_off, p.N, p.T);
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int c = (int)(cg - si.chunk0);
  const int len = min(kChunk, si.len - c * kChunk);
  const int64_t t0 = si.tok0 + (int64_t)c * kChunk;   // the chunk's first token
  const int64_t rqk = (int64_t)H * DK, rv = (int64_t)H * DV;
  const bf16* Kg = reinterpret_cast<const bf16*>(p.k) + t0 * rqk + (int64_t)h * DK;
  const bf16* Qg = reinterpret_cast<const bf16*>(p.q) + t0 * rqk + (int64_t)h * DK;
  const bf16* Vg = reinterpret_cast<const bf16*>(p.v) + t0 * rv + (int64_t)h * DV;
  const bf16* DOg = reinterpret_cast<const bf16*>(a.d_o) + t0 * rv + (int64_t)h * DV;
  const bf16* DVg = reinterpret_cast<const bf16*>(a.dv) + t0 * rv + (int64_t)h * DV;
  const float* hck = a.hchk + (cg * H + h) * (int64_t)(DK * DV);
  const bf16* dck = reinterpret_cast<const bf16*>(a.dhchk) + (cg * H + h) * (int64_t)(2 * DK * DV);
  const bf16* dcl = dck + (int64_t)DK * DV;   // dh'^T's low half (X' operands, read from global)
  const bf16* Tc = reinterpret_cast<const bf16*>(a.tmat) + (cg * H + h) * (int64_t)(kChunk * kChunk);
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- K, Q, dO rows, T, h^T (from the fp32 checkpoint) and the gates into LDS
#pragma unroll
  for (int k = 0; k < kChunk * DK / 8 / NT; ++k) {
    const int idx = tid + NT * k, row = idx / (DK / 8), cp = idx % (DK / 8);
    const int64_t off = row * rqk + cp * 8;
    *reinterpret_cast<u32x4*>(sK + row * KS + cp * 8) = row < len ? *reinterpret_cast<const u32x4*>(Kg + off) : z4;
    *reinterpret_cast<u32x4*>(sQ + row * KS + cp * 8) = row < len ? *reinterpret_cast<const u32x4*>(Qg + off) : z4;
  }
#pragma unroll
  for (int k = 0; k < kChunk * DV / 8 / NT; ++k) {
    const int idx = tid + NT * k, row = idx / (DV / 8), cp = idx % (DV / 8);
    *reinterpret_cast<u32x4*>(sDO + row * VS + cp * 8) =
        row < len ? *reinterpret_cast<const u32x4*>(DOg + row * rv + cp * 8) : z4;
  }
#pragma unroll
  for (int k = 0; k < kChunk * kChunk / 8 / NT; ++k) {
    const int idx = tid + NT * k, row = idx >> 3, cp = idx & 7;
    *reinterpret_cast<u32x4*>(sT + row * TS + cp * 8) = *reinterpret_cast<const u32x4*>(Tc + row * kChunk + cp * 8);
  }
  // checkpoint piece e holds keys 4 (e / DV) .. +3 of value column e % DV (ckpt_offset)
  auto ck_to_lds = [&](const f32x4& x, int e) {
    const int rq = e / DV, cv = e % DV;
    *reinterpret_cast<uint2*>(sH + cv * HS + 4 * rq) = pack_bf16x4(x);
  };
#pragma unroll
  for (int k = 0; k < NHP; ++k) {
    const int e = tid + NT * k;
    ck_to_lds(*reinterpret_cast<const f32x4*>(hck + (int64_t)e * 4), e);
  }
  // gamma_n <h, dh'>: the chain's partial sums, one per 32 value columns
  float hd = 0.f;
  if (tid == 0)
    for (int b = 0; b < DV / kDhCols; ++b) hd += a.gnh[(cg * H + h) * (DV / kDhCols) + b];
  // this lane's V elements (accumulator layout of its 64 x dv tiles) and dV rows (A
  // operands of dK's dV h^T term), loaded with the rest
  float vin[NJV][4];
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s;
      vin[jj][s] = i < len ? (float)Vg[i * rv + 16 * (half * NJV + jj) + r] : 0.f;
    }
  frag dvf[NVS];
#pragma unroll
  for (int ks = 0; ks < NVS; ++ks) {
    const int row = 16 * u + r;
    dvf[ks] = row < len ? *reinterpret_cast<const frag*>(DVg + row * rv + 32 * ks + 8 * q) : __builtin_bit_cast(frag, z4);
  }
  if (w == 0) {
    const float g = lane < len ? p.g[(t0 + lane) * H + h] : 0.f;
    const float G = wave_inclusive_scan_dpp(g);
    const float Gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
    sG[lane] = G;
    sGam[lane] = fast_exp(G);
    sD[lane] = fast_exp(Gn - G);
    sBet[lane] = lane < len ? beta_at(p.beta, (t0 + lane) * H + h, p.beta_bf16) : 0.f;
  }
  sPG[w][lane] = 0.f;
  sPB[w][lane] = 0.f;
  lds_barrier();

  float rg[4] = {0.f, 0.f, 0.f, 0.f};   // dG of rows 16 u + 4 q + s (this wave's column tiles)
  float rb[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta, the same rows
  float gnp = hd;                       // this lane's share of dG at the last row (G_n)

  // ---- (a) P = (Q K^T) * Gamma on this wave's lower blocks, into LDS (the blocks
  //      above are zero).  K K^T and Q K^T are formed again where dA and dP need them
  //      (fewer registers held through the products between).

  auto gram = [&](int ba, int bb, f32x4& kk, f32x4& qk) {
    kk = zero4;
    qk = zero4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const frag kb = op_rows(sK, KS, 16 * bb, 32 * ks);
      kk = Mb::run(op_rows(sK, KS, 16 * ba, 32 * ks), kb, kk);
      qk = Mb::run(op_rows(sQ, KS, 16 * ba, 32 * ks), kb, qk);
    }
  };
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int kb = w + NW * bi;
    if (kb >= 10) break;
    int ba, bb;
    tri_block(kb, ba, bb);
    f32x4 qk = zero4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qk = Mb::run(op_rows(sQ, KS, 16 * ba, 32 * ks), op_rows(sK, KS, 16 * bb, 32 * ks), qk);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * ba + 4 * q + s, j = 16 * bb + r;
      sR[i * TS + j] = (bf16)(j <= i ? qk[s] * fast_exp(sG[i] - sG[j]) : 0.f);
      if (ba != bb) sR[j * TS + i] = (bf16)0.f;
    }
  }
  // ---- (b) V' = V - diag(gamma) K h
  f32x4 vp[NJV];
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj) {
    const int jt = half * NJV + jj;
    f32x4 acc = zero4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc = Mb::run(op_rows(sK, KS, 16 * u, 32 * ks), op_rows(sH, HS, 16 * jt, 32 * ks), acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) vp[jj][s] = vin[jj][s] - sGam[16 * u + 4 * q + s] * acc[s];
  }
  // ---- (c) dQ = diag(gamma) dY h^T and dK = -diag(gamma) dV h^T (first terms), with
  //      their gamma terms of dG: sum_d Q_id dQ_id + sum_d K_id dK_id
  f32x4 dq[NJK], dk[NJK];
#pragma unroll
  for (int jj = 0; jj < NJK; ++jj) {
    dq[jj] = zero4;
    dk[jj] = zero4;
  }
#pragma unroll
  for (int ks = 0; ks < NVS; ++ks) {
    const frag dof = op_rows(sDO, VS, 16 * u, 32 * ks);
#pragma unroll
    for (int jj = 0; jj < NJK; ++jj) {
      const frag hb = op_cols(sH, HS, 32 * ks, 16 * (half * NJK + jj));
      dq[jj] = Mb::run(dof, hb, dq[jj]);
      dk[jj] = Mb::run(dvf[ks], hb, dk[jj]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < NJK; ++jj) {
    const int dt = half * NJK + jj;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s, d = 16 * dt + r;
      dq[jj][s] *= sGam[i] * p.scale;
      dk[jj][s] *= -sGam[i];
      rg[s] += (float)sQ[i * KS + d] * dq[jj][s] + (float)sK[i * KS + d] * dk[jj][s];
    }
  }
  lds_barrier();   // h^T read for the last time

  // ---- W = diag(beta) V' into LDS as a bf16 hi + lo pair (lo in the h^T region, now
  //      free): the gate gradient is sensitive to U's rounding
  bf16* sWl = sH;
  static_assert(DV * HS >= kChunk * VS, "W's low half fits the h^T region");
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s, o = i * VS + 16 * (half * NJV + jj) + r;
      const float x = sBet[i] * vp[jj][s];
      const bf16 hi = (bf16)x;
      sF[o] = hi;
      sWl[o] = (bf16)(x - (float)hi);
    }
  lds_barrier();

  // ---- (e) U = T diag(beta) V' (T lower triangular); the chain's dh'^T into LDS
  f32x4 Ut[NJV];
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj) {
    const int jt = half * NJV + jj;
    f32x4 acc = zero4;
    for (int ks = 0; ks <= (u >> 1); ++ks) {
      const frag ta = op_rows(sT, TS, 16 * u, 32 * ks);
      acc = Mb::run(ta, op_cols(sF, VS, 32 * ks, 16 * jt), acc);
      acc = Mb::run(ta, op_cols(sWl, VS, 32 * ks, 16 * jt), acc);
    }
    Ut[jj] = acc;
#pragma unroll
    for (int s = 0; s < 4; ++s) sU[(16 * u + 4 * q + s) * VS + 16 * jt + r] = (bf16)acc[s];
  }
  lds_barrier();   // W's low half read: the region takes dh'^T
  // the chain's dh'^T (bf16 [value column][key]) into LDS; the low half's X' operands
  // go out now, ahead of the barrier
#pragma unroll
  for (int k = 0; k < DV * DK / 8 / NT; ++k) {
    const int idx = tid + NT * k, row = idx / (DK / 8), cp = idx % (DK / 8);
    *reinterpret_cast<u32x4*>(sH + row * HS + cp * 8) = *reinterpret_cast<const u32x4*>(dck + (int64_t)idx * 8);
  }
  // the low half's operands for one value tile at a time, double-buffered: the first
  // tile's go out before the barrier, each next tile's before the current tile's MFMAs
  auto load_dlo = [&](frag* dst, int jt) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      dst[ks] = *reinterpret_cast<const frag*>(dcl + (int64_t)(16 * jt + r) * DK + 32 * ks + 8 * q);
  };
  frag dlo[2][NKS];
  load_dlo(dlo[0], half * NJV);
  lds_barrier();

  // ---- (f) X' = K dh', and the d terms of dG
  f32x4 X[NJV];
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj) {
    const int jt = half * NJV + jj;
    if (jj + 1 < NJV) load_dlo(dlo[(jj + 1) & 1], jt + 1);
    f32x4 acc = zero4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const frag ka = op_rows(sK, KS, 16 * u, 32 * ks);
      acc = Mb::run(ka, op_rows(sH, HS, 16 * jt, 32 * ks), acc);
      acc = Mb::run(ka, dlo[jj & 1][ks], acc);
    }
    X[jj] = acc;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s;
      const float xu = acc[s] * Ut[jj][s];
      rg[s] -= sD[i] * xu;
      gnp += sD[i] * xu;
    }
  }
  lds_barrier();

  // ---- (h) dU = diag(d) X' + scale P^T dO
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj) {
    const int jt = half * NJV + jj;
    f32x4 acc = zero4;
    for (int ks = u >> 1; ks < 2; ++ks)
      acc = Mb::run(op_cols(sR, TS, 32 * ks, 16 * u), op_cols(sDO, VS, 32 * ks, 16 * jt), acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s;
      sF[i * VS + 16 * jt + r] = (bf16)(sD[i] * X[jj][s] + p.scale * acc[s]);
    }
  }
  lds_barrier();

  // ---- (i) dR = T^T dU, and the V' term of dbeta
#pragma unroll
  for (int jj = 0; jj < NJV; ++jj) {
    const int jt = half * NJV + jj;
    f32x4 acc = zero4;
    for (int ks = u >> 1; ks < 2; ++ks)
      acc = Mb::run(op_cols(sT, TS, 32 * ks, 16 * u), op_cols(sF, VS, 32 * ks, 16 * jt), acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rb[s] += acc[s] * vp[jj][s];
      sR[(16 * u + 4 * q + s) * VS + 16 * jt + r] = (bf16)acc[s];
    }
  }
  // ---- (j) dK += diag(d) U dh'^T
#pragma unroll
  for (int jj = 0; jj < NJK; ++jj) {
    const int dt = half * NJK + jj;
    f32x4 acc = zero4;
#pragma unroll
    for (int ks = 0; ks < NVS; ++ks)
      acc = Mb::run(op_rows(sU, VS, 16 * u, 32 * ks), op_cols(sH, HS, 32 * ks, 16 * dt), acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) dk[jj][s] += sD[16 * u + 4 * q + s] * acc[s];
  }
  lds_barrier();

  // ---- (k) dP = lower(dY U^T) and dA = strict_lower(-dR U^T) on this wave's blocks:
  //      the Gamma terms of dG, the A term of dbeta, dP * Gamma and dB + dB^T into LDS
  bf16* sDPG = sF;
  bf16* sDBS = sH;   // dh'^T was read for the last time in (j)
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int kb = w + NW * bi;
    if (kb < 10) {
      int ba, bb;
      tri_block(kb, ba, bb);
      f32x4 kk, qk;
      gram(ba, bb, kk, qk);
      f32x4 dp = zero4, da = zero4;
#pragma unroll
      for (int ks = 0; ks < NVS; ++ks) {
        const frag ub = op_rows(sU, VS, 16 * bb, 32 * ks);
        dp = Mb::run(op_rows(sDO, VS, 16 * ba, 32 * ks), ub, dp);
        da = Mb::run(op_rows(sR, VS, 16 * ba, 32 * ks), ub, da);
      }
      float colc = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = 16 * ba + 4 * q + s, j = 16 * bb + r;
        const float gam = j <= i ? fast_exp(sG[i] - sG[j]) : 0.f;
        const float dpv = j <= i ? p.scale * dp[s] : 0.f;
        const float dav = j < i ? -da[s] : 0.f;
        const float kg = j < i ? kk[s] * gam : 0.f;
        const float gcon = dpv * qk[s] * gam + dav * sBet[i] * kg;   // dP * P + dA * A
        const float rs = sum16(gcon), rbs = sum16(dav * kg);
        if (r == 0) {
          sPG[w][i] += rs;
          sPB[w][i] += rbs;
        }
        colc += gcon;
        sDPG[i * TS + j] = (bf16)(dpv * gam);
        if (ba != bb) sDPG[j * TS + i] = (bf16)0.f;
        const float db = sBet[i] * dav * gam;
        if (ba != bb || j < i) {
          sDBS[i * TS + j] = (bf16)db;
          sDBS[j * TS + i] = (bf16)db;
        } else if (j == i) {
          sDBS[i * TS + j] = (bf16)0.f;
        }
      }
      colc += __shfl_xor(colc, 16, 64);
      colc += __shfl_xor(colc, 32, 64);
      if (q == 0) sPG[w][16 * bb + r] -= colc;
    }
  }
  lds_barrier();

  // ---- (l) dQ += (dP * Gamma) K;  dK += (dP * Gamma)^T Q + (dB + dB^T) K; store
  bf16* dQg = reinterpret_cast<bf16*>(a.dq) + t0 * rqk + (int64_t)h * DK;
  bf16* dKg = reinterpret_cast<bf16*>(a.dk) + t0 * rqk + (int64_t)h * DK;
#pragma unroll
  for (int jj = 0; jj < NJK; ++jj) {
    const int dt = half * NJK + jj;
    for (int ks = 0; ks <= (u >> 1); ++ks)
      dq[jj] = Mb::run(op_rows(sDPG, TS, 16 * u, 32 * ks), op_cols(sK, KS, 32 * ks, 16 * dt), dq[jj]);
    for (int ks = u >> 1; ks < 2; ++ks)
      dk[jj] = Mb::run(op_cols(sDPG, TS, 32 * ks, 16 * u), op_cols(sQ, KS, 32 * ks, 16 * dt), dk[jj]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      dk[jj] = Mb::run(op_rows(sDBS, TS, 16 * u, 32 * ks), op_cols(sK, KS, 32 * ks, 16 * dt), dk[jj]);
  }
  // ---- the row sums of this wave's tiles, then dG, dbeta and dg per row
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float gs = sum16(rg[s]), bs = sum16(rb[s]);
    if (r == 0) {
      sPG[w][16 * u + 4 * q + s] += gs;
      sPB[w][16 * u + 4 * q + s] += bs;
    }
  }
  {
    float t = gnp;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
    if (lane == 0) sPN[w] = t;
  }
  lds_barrier();
  if (w == 0) {
    float dG = 0.f, db = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      dG += sPG[k][lane];
      db += sPB[k][lane];
    }
    if (lane == kChunk - 1) {
#pragma unroll
      for (int k = 0; k < NW; ++k) dG += sPN[k];
    }
    // dg_t = sum over rows i >= t of dG_i: an inclusive scan of the reversed rows
    const float rev = __shfl(dG, kChunk - 1 - lane, 64);
    const float sc = wave_inclusive_scan_dpp(rev);
    const int t = kChunk - 1 - lane;
    if (t < len) a.dg[(t0 + t) * H + h] = sc;
    if (lane < len) {
      if (p.beta_bf16) reinterpret_cast<bf16*>(a.dbeta)[(t0 + lane) * H + h] = (bf16)db;
      else reinterpret_cast<float*>(a.dbeta)[(t0 + lane) * H + h] = db;
    }
  }
  // dq and dk last: no barrier waits for these stores
#pragma unroll
  for (int jj = 0; jj < NJK; ++jj)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = 16 * u + 4 * q + s, d = 16 * (half * NJK + jj) + r;
      if (i < len) {
        dQg[i * rqk + d] = (bf16)dq[jj][s];
        dKg[i * rqk + d] = (bf16)dk[jj][s];
      }
    }
}

template <int DK>
static hipError_t launch_dh_dk(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  const int nblk = p.dv / kDhCols;
  const int64_t wgs = (a.units + 7) / 8 * 8 * nblk;
  if (wgs > kMaxDispatchItems / kDhThreads) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL(bwd_dh_kernel<DK>, dim3((unsigned)wgs), dim3(kDhThreads), 0, s, ev.start, ev.stop, 0, p, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dh(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  if (a.units == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (!p.qkv_bf16 || p.dv % kDhCols != 0) return hipErrorInvalidValue;
  return p.dk == 128 ? launch_dh_dk<128>(p, a, s, ev) : launch_dh_dk<64>(p, a, s, ev);
}

template <int DK, int DV>
static hipError_t launch_grads_d(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  const int64_t wgs = p.total_chunks * p.H;
  if (wgs > kMaxDispatchItems / kGrThreads) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL((bwd_grads_kernel<DK, DV>), dim3((unsigned)wgs), dim3(kGrThreads), 0, s, ev.start,
                        ev.stop, 0, p, a);
  return hipGetLastError();
}

hipError_t launch_bwd_grads(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev) {
  if (p.total_chunks * p.H == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (!p.qkv_bf16) return hipErrorInvalidValue;
  if (p.dk == 128)
    return p.dv == 128 ? launch_grads_d<128, 128>(p, a, s, ev) : launch_grads_d<128, 64>(p, a, s, ev);
  return p.dv == 128 ? launch_grads_d<64, 128>(p, a, s, ev) : launch_grads_d<64, 64>(p, a, s, ev);
}

}  // namespace gdn
