// Cross-segment merge of the sequence-parallel correction on gfx950.
//
// FlashQLA talk transcript (tokendh.com), sequence-parallel section: each split
// keeps only its segment-end wrong-start state S* and its composed dk x dk
// correction M; a short recurrence over the splits then gives every split's true
// start, after which S and O are recomputed.  With h = S^T:
//
//     h_start(0) = h0 (or 0),   h_start(j+1) = M_j h_start(j) + S*_j
//
// Mapping: one workgroup per (sequence, head, 16 value columns); columns of h are
// independent.  Wave w owns output rows [32w, 32w+32).  M_j h is one 128x128x16
// product per step on MFMA; to keep fp32-level accuracy both factors are split
// into bf16 high and low parts, M h ~= Mh hh + Mh hl + Ml hh.  Pass 1 stores M
// already split, in operand order (mfrag_offset: one 1 KB contiguous block per
// wave and fragment, so the loads coalesce fully), and the operands
// of step j+2 (M fragments, S* tiles) are loaded while step j computes: only the
// MFMA chain through h is serial.  The running state lives in
// LDS as bf16 high/low, K-major by column, so a lane's B operand is one 16-byte
// read.  Heads that take window-lookback starts skip the merge.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
__global__ __launch_bounds__(256) void cp_merge_kernel(Problem p, FwdPlan plan) {
  constexpr int HS = DK + 8;                 // row stride of the bf16 state copies
  constexpr int NKS = DK / 32;
  constexpr int RT = DK / 64;                // row tiles per wave (4 waves x RT x 16 = DK)
  __shared__ __align__(16) bf16 sHi[16 * HS];
  __shared__ __align__(16) bf16 sLo[16 * HS];

  const int nh = blockIdx.x, H = p.H, n = nh / H, h = nh % H;
  const int dv = p.dv, col = 16 * blockIdx.y;
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int L = plan.seg_chunks;
  const int segs = (nch + L - 1) / L;
  if (segs < 2) return;
  if (!plan.cp.force_correction && window_of(plan.cp.best, nh, nch, plan.cp.wmax, plan.cp.thr) > 0)
    return;
  const int64_t sg0 =
      plan.seg_off ? plan.seg_off[n]
                   : (int64_t)n * max((int64_t)1, ((p.T + kChunk - 1) / kChunk + L - 1) / L);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;

  // start state columns [col, col+16) -> LDS (hi/lo), K-major per column
  for (int i = tid; i < DK * 16; i += 256) {
    const int r = i >> 4, cc = i & 15;
    const float x = p.h0 ? p.h0[((int64_t)nh * DK + r) * dv + col + cc] : 0.f;
    const bf16 hi = (bf16)x;
    sHi[cc * HS + r] = hi;
    sLo[cc * HS + r] = (bf16)(x - (float)hi);
  }
  __syncthreads();

  // operands of one step: M_j fragments (row-major hi / lo blocks) and S*_j tiles
  struct Ops {
    bf16x8 mh[RT][NKS], ml[RT][NKS];
    f32x4 s[RT];
  };
  auto load = [&](Ops& o, int j) {
    const int64_t slot = (sg0 + j) * H + h;
    const bf16* Mh = reinterpret_cast<const bf16*>(plan.cp.mcorr) + slot * 2 * DK * DK;
    const bf16* Ml = Mh + DK * DK;
    const float* Sj = plan.cp.sstar + slot * DK * dv;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rb = 16 * (RT * wave + t);
#pragma unroll
      for (int i = 0; i < 4; ++i) o.s[t][i] = Sj[(int64_t)(rb + 4 * q + i) * dv + col + r16];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int64_t at = ((int64_t)((RT * wave + t) * NKS + s) * 64 + lane) * 8;   // mfrag_offset order
        o.mh[t][s] = *reinterpret_cast<const bf16x8*>(Mh + at);
        o.ml[t][s] = *reinterpret_cast<const bf16x8*>(Ml + at);
      }
    }
  };

  // three operand sets in flight: step j computes with set j % 3 while the loads of
  // step j + 2 land in the set step j - 1 used (load counts are the same every step,
  // the index is clamped at the end, so no step waits on loads it does not need)
  const int steps = segs - 1;
  auto body = [&](const Ops& cur, Ops& far, int j) {
    load(far, min(j + 2, steps - 1));
    f32x4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = cur.s[t];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 bh = lds_frag(sHi, HS, r16, 32 * s, q);
      const bf16x8 bl = lds_frag(sLo, HS, r16, 32 * s, q);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        acc[t] = Mma<bf16>::run(cur.mh[t][s], bh, acc[t]);
        acc[t] = Mma<bf16>::run(cur.mh[t][s], bl, acc[t]);
        acc[t] = Mma<bf16>::run(cur.ml[t][s], bh, acc[t]);
      }
    }
    __syncthreads();  // every wave has read the old state
    const int64_t slot = (sg0 + j) * H + h;
    float* Hn = plan.cp.hstart + (slot + H) * DK * dv;   // start of segment j+1
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rb = 16 * (RT * wave + t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb + 4 * q + i;
        const float x = acc[t][i];
        Hn[(int64_t)r * dv + col + r16] = x;
        const bf16 hi = (bf16)x;
        sHi[r16 * HS + r] = hi;
        sLo[r16 * HS + r] = (bf16)(x - (float)hi);
      }
    }
    __syncthreads();
  };
  Ops o0, o1, o2;
  load(o0, 0);
  load(o1, min(1, steps - 1));
  int j = 0;
  for (; j + 3 <= steps; j += 3) {   // no conditions inside: every path issues the same loads
    body(o0, o2, j);
    body(o1, o0, j + 1);
    body(o2, o1, j + 2);
  }
  if (j < steps) body(o0, o2, j);
  if (j + 1 < steps) body(o1, o0, j + 1);
}

hipError_t launch_cp_merge(const Problem& p, const FwdPlan& plan, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  dim3 grid((unsigned)(p.N * p.H), (unsigned)(p.dv / 16));
  if (p.dk == 128) cp_merge_kernel<128><<<grid, 256, 0, s>>>(p, plan);
  else cp_merge_kernel<64><<<grid, 256, 0, s>>>(p, plan);
  return hipGetLastError();
}

}  // namespace gdn
