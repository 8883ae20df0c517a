// Cross-segment merge of the sequence-parallel correction on gfx950.
//
// FlashQLA talk transcript (tokendh.com), sequence-parallel section: each split
// keeps only its segment-end wrong-start state S* and its composed dk x dk
// correction M; a short recurrence over the splits then gives every split's true
// start, after which S and O are recomputed.  With h = S^T:
//
//     h_start(0) = h0 (or 0),   h_start(j+1) = M_j h_start(j) + S*_j
//
// Each step is an affine map x -> M_j x + S*_j, and affine maps compose, so the
// chain of `steps` maps is evaluated as a two-level tree when it is long: the steps
// are cut into groups of G; (A) every group composes its maps into one,
// [A_g | b_g] = M_e-1 ... M_gG [I | 0] + offsets (all groups in parallel); (B) one
// chain over the group maps gives the start of every group; (C) every group then
// runs its own steps from its start (all groups in parallel).  The serial depth
// falls from `steps` to about 3 sqrt(steps).  Short chains run (C) alone, as one
// group from h0.
//
// Mapping: one workgroup per (sequence, head, [group,] 16 columns); columns are
// independent.  DK/16 waves, wave w owns output rows [16w, 16w+16).  A step is one
// DKxDKx16 product on MFMA; to keep fp32-level accuracy both factors are split
// into bf16 high and low parts, M x ~= Mh xh + Mh xl + Ml xh (three independent
// accumulator chains, summed at the end).  Pass 1 stores M already split and S* as
// accumulator tiles, both in operand order (one 1 KB contiguous block per wave
// and operand, so the loads coalesce fully); (A) writes its group maps the same
// way.  The step is bound by its operand loads, not by its few MFMAs, so a ring of
// NSET operand sets keeps the loads of the next steps in flight: only the MFMA
// chain through the state is serial.  The running state lives in LDS as bf16
// high/low, K-major by column (a lane's B operand is one 16-byte read), in two
// copies used alternately, so each step needs a single barrier.  The column blocks
// of one unit run on one XCD and share the operands through its L2.  Heads that
// take window-lookback starts skip the merge.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
struct MergeCfg {
  static constexpr int NW = DK / 16;     // waves, one 16-row tile each
  static constexpr int NKS = DK / 32;    // contraction steps
  static constexpr int HS = DK + 8;      // row stride of the bf16 state copies
  // operand sets in flight: at DK = 128 (8 waves, 256 registers) four sets spill 60
  // registers and two run the 63-step chain of the long workload 12 us faster
  static constexpr int NSET = DK == 128 ? 2 : 6;
};

// kRun: steps of one group from its start (or the whole chain from h0);
// kCompose: (A), a group's composed map; kGroups: (B), the chain over group maps.
enum { kRun = 0, kCompose = 1, kGroups = 2 };

// G: steps per group; maxg: group slots per (sequence, head) in the grid; tree: the
// group ends are written by (B), so (C) stops one step short of its group's end.
template <int DK, int MODE>
__global__ __launch_bounds__(64 * MergeCfg<DK>::NW) void cp_merge_kernel(Problem p, FwdPlan plan, int G,
                                                                         int maxg, int tree) {
  using C = MergeCfg<DK>;
  constexpr int NKS = C::NKS, HS = C::HS, NSET = C::NSET;
  __shared__ __align__(16) bf16 sHi[2][16 * HS];
  __shared__ __align__(16) bf16 sLo[2][16 * HS];

  if (plan.cp.ncorr && *plan.cp.ncorr == 0u) return;   // no head takes the correction
  // XCD-aware decode of the 1-D grid: workgroup b runs on XCD b % 8; the column
  // blocks of unit u all go to XCD u % 8
  const int dv = p.dv;
  const int ncb = (MODE == kCompose ? DK + dv : dv) / 16;
  const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
  const int64_t unit = (int64_t)(k / ncb) * 8 + xcd;
  const int cb = k % ncb;
  const int64_t nh64 = MODE == kGroups ? unit : unit / maxg;
  const int g = MODE == kGroups ? 0 : (int)(unit % maxg);
  if (nh64 >= (int64_t)p.N * p.H) return;
  const int nh = (int)nh64, H = p.H, n = nh / H, h = nh % H;
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int L = plan.seg_chunks;
  const int segs = (nch + L - 1) / L;
  if (segs < 2) return;
  const int64_t sg0 =
      plan.seg_off ? plan.seg_off[n]
                   : (int64_t)n * max((int64_t)1, ((p.T + kChunk - 1) / kChunk + L - 1) / L);
  if (!plan.cp.force_correction && plan.cp.seg_win[(sg0 + 1) * H + h] > 0) return;   // window head
  const int steps = segs - 1;
  const int ngroups = (steps + G - 1) / G;
  if (g >= ngroups) return;
  // step range [j0, j1) of this workgroup (kGroups: j indexes groups)
  int j0 = 0, j1 = ngroups;
  if constexpr (MODE != kGroups) {
    j0 = g * G;
    j1 = min(j0 + G, steps) - (MODE == kRun && tree ? 1 : 0);
  }
  const int nsteps = j1 - j0;

  // the columns: kCompose covers [A | b] (DK matrix columns, then dv offset columns)
  const bool eye = MODE == kCompose && cb < DK / 16;         // matrix columns start as I
  const int vcol = MODE == kCompose ? (eye ? 0 : 16 * cb - DK) : 16 * cb;   // offset column block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int col = vcol + r16;

  // operand slots: per segment (M_j, S*_j from pass 1) or per group (A_g, b_g)
  const bf16* mat_base = reinterpret_cast<const bf16*>(MODE == kGroups ? plan.cp.gmat : plan.cp.mcorr);
  const float* vec_base = MODE == kGroups ? plan.cp.gvec : plan.cp.sstar;
  auto state_slot = [&](int64_t seg) { return plan.cp.hstart + (seg * H + h) * DK * dv; };

  // start state: rows 16 wave + 4q + i of column col
  f32x4 x0;
  {
    const float* src = nullptr;
    if constexpr (MODE == kRun) {
      src = g == 0 ? p.h0 + (int64_t)nh * DK * dv : state_slot(sg0 + j0);
      if (g == 0 && !p.h0) src = nullptr;
    } else if constexpr (MODE == kGroups) {
      src = p.h0 ? p.h0 + (int64_t)nh * DK * dv : nullptr;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * q + i;
      if constexpr (MODE == kCompose) x0[i] = (eye && r == 16 * cb + r16) ? 1.f : 0.f;
      else x0[i] = src ? src[(int64_t)r * dv + col] : 0.f;
    }
  }
  auto put_state = [&](int copy, const f32x4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * q + i;
      const bf16 hi = (bf16)x[i];
      sHi[copy][r16 * HS + r] = hi;
      sLo[copy][r16 * HS + r] = (bf16)(x[i] - (float)hi);
    }
  };
  put_state(0, x0);
  __syncthreads();

  // operands of one step: this wave's matrix fragments (hi / lo) and offset tile
  struct Ops {
    bf16x8 mh[NKS], ml[NKS];
    f32x4 s;
  };
  auto load = [&](Ops& o, int j) {
    const int64_t slot = (sg0 + j) * H + h;
    const bf16* Mh = mat_base + slot * 2 * DK * DK;
    const bf16* Ml = Mh + DK * DK;
    const float* Sj = vec_base + slot * DK * dv;
    o.s = *reinterpret_cast<const f32x4*>(Sj + ((int64_t)((vcol >> 4) * (DK / 16) + wave) * 64 + lane) * 4);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int64_t at = ((int64_t)(wave * NKS + s) * 64 + lane) * 8;   // mfrag_offset order
      o.mh[s] = *reinterpret_cast<const bf16x8*>(Mh + at);
      o.ml[s] = *reinterpret_cast<const bf16x8*>(Ml + at);
    }
  };
  // per-step output: the start of the next segment (kRun) or of the next group
  // (kGroups); kCompose keeps its state to the end
  auto store_state = [&](int j, const f32x4& x) {
    if constexpr (MODE != kCompose) {
      const int64_t seg = MODE == kRun ? sg0 + j + 1 : sg0 + min((j + 1) * G, steps);
      float* Hs = state_slot(seg);
#pragma unroll
      for (int i = 0; i < 4; ++i) Hs[(int64_t)(16 * wave + 4 * q + i) * dv + col] = x[i];
    }
  };

  // Step j computes with set j % NSET and then refills it with the operands of step
  // j + NSET (clamped at the end: load counts are the same every step, so no step
  // waits on loads it does not need).  State copy j % 2 is read, copy (j+1) % 2
  // written: a wave can only write a copy again after the next barrier, which every
  // wave reaches after its reads of that copy.
  f32x4 x = x0;
  auto body = [&](Ops& cur, int jj) {   // jj = j - j0
    const bf16* hHi = sHi[jj & 1];
    const bf16* hLo = sLo[jj & 1];
    bf16x8 bh[NKS], bl[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      bh[s] = lds_frag(hHi, HS, r16, 32 * s, q);
      bl[s] = lds_frag(hLo, HS, r16, 32 * s, q);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 a0 = eye ? zero : cur.s, a1 = zero, a2 = zero;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      a0 = Mma<bf16>::run(cur.mh[s], bh[s], a0);
      a1 = Mma<bf16>::run(cur.mh[s], bl[s], a1);
      a2 = Mma<bf16>::run(cur.ml[s], bh[s], a2);
    }
    load(cur, j0 + min(jj + NSET, nsteps - 1));
    x = a0 + a1 + a2;
    store_state(j0 + jj, x);
    put_state((jj + 1) & 1, x);
    __syncthreads();
  };
  if (nsteps > 0) {
    // Prologue: the compiler sizes each wait in the loop for the worst path into it,
    // so the prologue issues the same memory operations in the same order as a step
    // (a set's loads, then the step's state stores; here the start state to its own
    // slot); loads issued back to back would make every wait of the loop wait for
    // loads issued one step earlier.
    Ops o[NSET];
#pragma unroll
    for (int i = 0; i < NSET; ++i) {
      load(o[i], j0 + min(i, nsteps - 1));
      if constexpr (MODE == kRun) {
        float* Hs = state_slot(sg0 + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Hs[(int64_t)(16 * wave + 4 * q + e) * dv + col] = x0[e];
      } else if constexpr (MODE == kGroups) {
        float* Hs = state_slot(sg0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Hs[(int64_t)(16 * wave + 4 * q + e) * dv + col] = x0[e];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    int jj = 0;
    for (; jj + NSET <= nsteps; jj += NSET) {   // no conditions inside: every path issues the same loads
#pragma unroll
      for (int i = 0; i < NSET; ++i) body(o[i], jj + i);
    }
#pragma unroll
    for (int i = 0; i < NSET - 1; ++i)
      if (jj + i < nsteps) body(o[i], jj + i);
  }

  if constexpr (MODE == kCompose) {
    // the group map: matrix columns as bf16 high / low MFMA operands (mfrag_offset),
    // offset columns as accumulator tiles (sfrag_offset)
    const int64_t slot = (sg0 + g) * H + h;
    if (eye) {
      bf16* ghi = reinterpret_cast<bf16*>(plan.cp.gmat) + slot * 2 * DK * DK;
      bf16* glo = ghi + DK * DK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t at = mfrag_offset<DK>(16 * wave + 4 * q + i, 16 * cb + r16);
        const bf16 hi = (bf16)x[i];
        ghi[at] = hi;
        glo[at] = (bf16)(x[i] - (float)hi);
      }
    } else {
      *reinterpret_cast<f32x4*>(plan.cp.gvec + slot * DK * dv + sfrag_offset<DK>(16 * wave + 4 * q, col)) = x;
    }
  }
}

// ev: start recorded from the first kernel's dispatch, stop from the last one's.
template <int DK>
static hipError_t launch_merge_dk(const Problem& p, const FwdPlan& plan, int max_steps, hipStream_t s,
                            KernelEvents ev) {
  const dim3 nt(64 * MergeCfg<DK>::NW);
  const int64_t nh = (int64_t)p.N * p.H;
  const int ncb = p.dv / 16;
  auto grid = [&](int64_t units, int cbs) { return dim3((unsigned)((units + 7) / 8 * 8 * cbs)); };
  {   // the widest launch (the group maps, or the whole chain) must fit a dispatch
    int G = 1;
    while ((int64_t)G * G < max_steps) ++G;
    const int64_t maxg = max_steps > kMergeTreeMinSteps ? (max_steps + G - 1) / G : 1;
    if ((nh * maxg + 7) / 8 * 8 > kMaxDispatchItems / ((int64_t)(DK + p.dv) / 16 * nt.x))
      return hipErrorInvalidConfiguration;
  }
  if (max_steps <= kMergeTreeMinSteps) {
    hipExtLaunchKernelGGL(cp_merge_kernel<DK, kRun>, grid(nh, ncb), nt, 0, s, ev.start, ev.stop, 0, p, plan,
                          max(max_steps, 1), 1, 0);
    return hipGetLastError();
  }
  int G = 1;
  while ((int64_t)G * G < max_steps) ++G;   // G = ceil(sqrt(steps))
  const int maxg = (max_steps + G - 1) / G;
  hipExtLaunchKernelGGL(cp_merge_kernel<DK, kCompose>, grid(nh * maxg, (DK + p.dv) / 16), nt, 0, s, ev.start,
                        nullptr, 0, p, plan, G, maxg, 1);
  hipExtLaunchKernelGGL(cp_merge_kernel<DK, kGroups>, grid(nh, ncb), nt, 0, s, nullptr, nullptr, 0, p, plan,
                        G, 1, 1);
  hipExtLaunchKernelGGL(cp_merge_kernel<DK, kRun>, grid(nh * maxg, ncb), nt, 0, s, nullptr, ev.stop, 0, p,
                        plan, G, maxg, 1);
  return hipGetLastError();
}

hipError_t launch_cp_merge(const Problem& p, const FwdPlan& plan, int max_steps, hipStream_t s,
                           KernelEvents ev) {
  if (p.N == 0 || max_steps < 1) {
    ev.record_empty(s);
    return hipSuccess;
  }
  return p.dk == 128 ? launch_merge_dk<128>(p, plan, max_steps, s, ev)
                     : launch_merge_dk<64>(p, plan, max_steps, s, ev);
}

}  // namespace gdn
