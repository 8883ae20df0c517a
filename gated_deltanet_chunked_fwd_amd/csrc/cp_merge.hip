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
// independent.  DK/16 waves, wave w owns output rows [16w, 16w+16).  M_j h is one
// DKxDKx16 product per step on MFMA; to keep fp32-level accuracy both factors are
// split into bf16 high and low parts, M h ~= Mh hh + Mh hl + Ml hh (three
// independent accumulator chains, summed at the end).  Pass 1 stores M already
// split and S* as accumulator tiles, both in operand order (one 1 KB contiguous
// block per wave and operand, so the loads coalesce fully).  The step is bound by
// the latency of those loads, not by its few MFMAs, so a ring of NSET operand sets
// keeps the loads of steps j+1 .. j+NSET-1 in flight while step j computes: only
// the MFMA chain through h is serial.  The running state lives in LDS as bf16
// high/low, K-major by column (a lane's B operand is one 16-byte read), in two
// copies used alternately, so each step needs a single barrier.  The column blocks
// of one (sequence, head) run on one XCD and share M through its L2.  Heads that
// take window-lookback starts skip the merge.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
struct MergeCfg {
  static constexpr int NW = DK / 16;     // waves, one 16-row tile each
  static constexpr int NKS = DK / 32;    // contraction steps
  static constexpr int HS = DK + 8;      // row stride of the bf16 state copies
  static constexpr int NSET = DK == 128 ? 4 : 6;   // operand sets in flight (registers permitting)
};

template <int DK>
__global__ __launch_bounds__(64 * MergeCfg<DK>::NW) void cp_merge_kernel(Problem p, FwdPlan plan) {
  using C = MergeCfg<DK>;
  constexpr int NKS = C::NKS, HS = C::HS, NSET = C::NSET;
  __shared__ __align__(16) bf16 sHi[2][16 * HS];
  __shared__ __align__(16) bf16 sLo[2][16 * HS];

  // XCD-aware decode of the 1-D grid: workgroup b runs on XCD b % 8; the column
  // blocks of unit u all go to XCD u % 8
  const int ncb = p.dv / 16;
  const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
  const int nh = (k / ncb) * 8 + xcd, cb = k % ncb;
  if (nh >= p.N * p.H) return;
  const int H = p.H, n = nh / H, h = nh % H;
  const int dv = p.dv, col = 16 * cb;
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

  // start state columns [col, col+16) -> LDS copy 0 (hi/lo), K-major per column
  for (int i = tid; i < DK * 16; i += 64 * C::NW) {
    const int r = i >> 4, cc = i & 15;
    const float x = p.h0 ? p.h0[((int64_t)nh * DK + r) * dv + col + cc] : 0.f;
    const bf16 hi = (bf16)x;
    sHi[0][cc * HS + r] = hi;
    sLo[0][cc * HS + r] = (bf16)(x - (float)hi);
  }
  __syncthreads();

  // operands of one step: this wave's M_j fragments (hi / lo) and S*_j tile
  struct Ops {
    bf16x8 mh[NKS], ml[NKS];
    f32x4 s;
  };
  auto load = [&](Ops& o, int j) {
    const int64_t slot = (sg0 + j) * H + h;
    const bf16* Mh = reinterpret_cast<const bf16*>(plan.cp.mcorr) + slot * 2 * DK * DK;
    const bf16* Ml = Mh + DK * DK;
    const float* Sj = plan.cp.sstar + slot * DK * dv;
    o.s = *reinterpret_cast<const f32x4*>(Sj + ((int64_t)(cb * (DK / 16) + wave) * 64 + lane) * 4);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int64_t at = ((int64_t)(wave * NKS + s) * 64 + lane) * 8;   // mfrag_offset order
      o.mh[s] = *reinterpret_cast<const bf16x8*>(Mh + at);
      o.ml[s] = *reinterpret_cast<const bf16x8*>(Ml + at);
    }
  };

  // Step j computes with set j % NSET and then refills it with the operands of step
  // j + NSET (clamped at the end: load counts are the same every step, so no step
  // waits on loads it does not need).  State copy j % 2 is read, copy (j+1) % 2
  // written: a wave can only write a copy again after the next barrier, which every
  // wave reaches after its reads of that copy.
  const int steps = segs - 1;
  auto store_state = [&](int64_t seg_slot, const f32x4& x) {
    float* Hs = plan.cp.hstart + seg_slot * DK * dv;
#pragma unroll
    for (int i = 0; i < 4; ++i) Hs[(int64_t)(16 * wave + 4 * q + i) * dv + col + r16] = x[i];
  };
  auto body = [&](Ops& cur, int j) {
    const bf16* hHi = sHi[j & 1];
    const bf16* hLo = sLo[j & 1];
    bf16x8 bh[NKS], bl[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      bh[s] = lds_frag(hHi, HS, r16, 32 * s, q);
      bl[s] = lds_frag(hLo, HS, r16, 32 * s, q);
    }
    f32x4 a0 = cur.s, a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      a0 = Mma<bf16>::run(cur.mh[s], bh[s], a0);
      a1 = Mma<bf16>::run(cur.mh[s], bl[s], a1);
      a2 = Mma<bf16>::run(cur.ml[s], bh[s], a2);
    }
    load(cur, min(j + NSET, steps - 1));
    const f32x4 x = a0 + a1 + a2;
    store_state((sg0 + j + 1) * H + h, x);   // start of segment j+1
    bf16* nHi = sHi[(j + 1) & 1];
    bf16* nLo = sLo[(j + 1) & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * q + i;
      const bf16 hi = (bf16)x[i];
      nHi[r16 * HS + r] = hi;
      nLo[r16 * HS + r] = (bf16)(x[i] - (float)hi);
    }
    __syncthreads();
  };
  // Prologue: the compiler sizes each wait in the loop for the worst path into it,
  // so the prologue issues the same memory operations in the same order as a step
  // (a set's loads, then four state stores; here the start state of segment 0, which
  // is its true start); loads issued back to back would make every wait of the
  // loop wait for loads issued one step earlier.
  f32x4 x0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * q + i;
    x0[i] = p.h0 ? p.h0[((int64_t)nh * DK + r) * dv + col + r16] : 0.f;
  }
  Ops o[NSET];
#pragma unroll
  for (int i = 0; i < NSET; ++i) {
    load(o[i], min(i, steps - 1));
    store_state(sg0 * H + h, x0);
    __builtin_amdgcn_sched_barrier(0);
  }
  int j = 0;
  for (; j + NSET <= steps; j += NSET) {   // no conditions inside: every path issues the same loads
#pragma unroll
    for (int i = 0; i < NSET; ++i) body(o[i], j + i);
  }
#pragma unroll
  for (int i = 0; i < NSET - 1; ++i)
    if (j + i < steps) body(o[i], j + i);
}

hipError_t launch_cp_merge(const Problem& p, const FwdPlan& plan, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  const int64_t units = (int64_t)p.N * p.H;
  const unsigned grid = (unsigned)((units + 7) / 8 * 8 * (p.dv / 16));
  if (p.dk == 128) cp_merge_kernel<128><<<grid, 64 * MergeCfg<128>::NW, 0, s>>>(p, plan);
  else cp_merge_kernel<64><<<grid, 64 * MergeCfg<64>::NW, 0, s>>>(p, plan);
  return hipGetLastError();
}

}  // namespace gdn
