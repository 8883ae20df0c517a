// Steps 2-4 of the chunked WY form, fused, on gfx950: per (sequence, head,
// value-column block, segment) a workgroup walks the chunks in order with the
// state resident in registers, and writes only O and the final state.
//
// FlashQLA talk transcript (tokendh.com): chunked-WY section (W/U projections,
// chunk-serial state recurrence, output from the state); pain-points section
// (W, U and S must not round-trip through HBM); algebraic-rewrites section
// (forward merge: form "V minus S" first, then apply gamma).  With h = S^T the
// state at chunk start, G the chunk-local cumsum of g, gamma = exp(G),
// Gamma_rs = exp(G_r - G_s) (r >= s), d = exp(G_last - G) and T from step 1:
//
//   V' = V - diag(gamma) K h                      (merged W/U form)
//   U  = T diag(beta) V'
//   O  = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)
//   h <- gamma_last h + K^T (diag(d) U)
//
// Mapping.  4 or 8 waves (two per SIMD with 8); each wave owns NCW = 16 value
// columns of h for all dk rows, as 16x16 fp32 accumulator tiles in "tile order" (gdn_device.h),
// so h, V' and U feed the next MFMA straight from registers.  Per chunk the
// workgroup stages K, Q, T, the gates and its V columns in LDS (the global loads
// of chunk c+1 go out in four parts while chunk c is computed, and bf16 chunks are
// double-buffered, so chunk c+1 is staged at the end of chunk c's step), computes
// P = (QK^T)*Gamma once (tiles split over the waves), and each wave then runs its
// columns: K^T for the state update and V in accumulator layout come from the
// row-major tiles through LDS transpose reads.  O is produced transposed (MFMA
// operands swapped), so each lane ends with four consecutive value columns of one
// query row; it is finished and stored at the start of the next chunk's step.
// Lookback chunks (window starts) produce no O and skip Q; T's zero upper-right
// 32 x 32 quadrant is never loaded.  Value columns are independent; only T and P
// are shared between them.
#include <type_traits>



#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename E, int DK, int NCW, int NW>
struct FwdCfg {
  static constexpr int NWAVES = NW;         // waves per workgroup (4 or 8)
  static constexpr int NT = 64 * NW;        // threads per workgroup
  static constexpr int BV = NWAVES * NCW;   // value columns per workgroup
  static constexpr int NCT = NCW / 16;      // column tiles per wave
  static constexpr int NKT = DK / 16;       // dk tiles of the state
  static constexpr int NKS = DK / 32;       // contraction steps over dk
  static constexpr bool BF = sizeof(E) == 2;
  // Row strides (elements).  bf16 tiles that feed fragment reads are stored in tile
  // order with a stride of 8 (mod 32) dwords: 16-byte fragment reads and 8-byte
  // transpose reads are then free of bank conflicts on gfx950's LDS.
  static constexpr int KS = BF ? DK + 16 : DK + 4;        // sK, sQ
  static constexpr int CS = BF ? kChunk + 16 : kChunk + 4; // sT, sP
  static constexpr int VS = BF ? BV + 16 : BV + 4;        // sV
};

// One chunk's inputs held in registers between the global loads and the LDS
// stores, so the loads of chunk c+1 are in flight while chunk c is computed.
// Nothing touches the loaded registers until store(): masking of rows past the
// chunk end (zero there; beta = g = 0) and the beta conversion happen at store
// time, so no wait for the loads is forced before the chunk's compute.
// WITH_Q: pass 1 and the checkpoint pass produce no output, so they neither load nor
// stage Q.
template <typename E, int DK, int BV, int NTH, bool WITH_Q>
struct ChunkRegs {
  static constexpr int EPV = 16 / (int)sizeof(E);
  static constexpr int VPRK = DK / EPV, VPRV = BV / EPV, VPRT = kChunk / EPV;
  static constexpr int NK = kChunk * VPRK / NTH, NV = kChunk * VPRV / NTH, NT = kChunk * VPRT / NTH;
  static_assert(NK * NTH == kChunk * VPRK && NV * NTH == kChunk * VPRV && NT * NTH == kChunk * VPRT,
                "chunk tiles must split evenly over the threads");
  u32x4 k[NK], q[NK], v[NV], t[NT];
  // 16-byte piece i of a chunk's T lies in the upper-right 32 x 32 quadrant
  static __device__ __forceinline__ bool t_quadrant(int i) {
    return i / VPRT < kChunk / 2 && (i % VPRT) * EPV >= kChunk / 2;
  }
  float g;
  uint32_t b;   // raw beta bits (bf16 in the low half, or fp32)
  int len;

  // Per-thread offsets inside a full chunk (fixed for the whole walk): k, v in bytes
  // (32-bit, added to the chunk's uniform base pointer, so a load needs no 64-bit
  // address arithmetic), g in elements.
  struct Offsets {
    uint32_t k[NK], v[NV];
    int g;
    __device__ __forceinline__ void init(int row_qk, int row_v, int row_g, int tid) {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int i = tid + NTH * j;
        k[j] = (uint32_t)((i / VPRK) * row_qk + (i % VPRK) * EPV) * (uint32_t)sizeof(E);
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = tid + NTH * j;
        v[j] = (uint32_t)((i / VPRV) * row_v + (i % VPRV) * EPV) * (uint32_t)sizeof(E);
      }
      g = (tid & (kChunk - 1)) * row_g;
    }
  };

  // qb/kb/vb/gb/betab point at the chunk's first token (head and column offsets
  // applied); rows past the chunk end read the chunk's first row instead (masked
  // to zero in store()).  The loads go out in four parts spread over the step
  // (PART 0: g, beta, K; 1: Q; 2: V; 3: T): issuing a whole chunk at once fills the
  // CU's vector-memory queue and stalls the waves that issue last.  Q and V carry the
  // nontemporal hint (streamed, not kept in the caches): no other workgroup reads a
  // chunk's Q, only the next segment's lookback reads its V, and the cache space
  // they leave stays with K and T, which K1 has just written or read (measured 0-4%
  // faster per call, never slower; the hint on K or T, or on the O stores, was not).
  template <int PART>
  __device__ __forceinline__ void load(const E* qb, const E* kb, const E* vb, const E* ts,
                                       const float* gb, const void* betab, bool beta_bf16,
                                       int len_, const Offsets& of, int tid) {
    const bool full = len_ == kChunk;
    if constexpr (PART == 0) {
      len = len_;
      const int og = (full || (tid & (kChunk - 1)) < len_) ? of.g : 0;
      g = gb[og];
      if (beta_bf16) b = reinterpret_cast<const uint16_t*>(betab)[og];
      else b = reinterpret_cast<const uint32_t*>(betab)[og];
    }
    if constexpr (PART == 0 || (PART == 1 && WITH_Q)) {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int r = (tid + NTH * j) / VPRK;
        const uint32_t o = (full || r < len_) ? of.k[j] : (uint32_t)((tid + NTH * j) % VPRK) * 16u;
        if constexpr (PART == 0) k[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kb) + o);
        else q[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(qb) + o));
      }
    }
    // V is loaded even when it is not used (vzero: masked at store time), so every
    // path issues the same loads and the compiler's memory-counter waits for older
    // stores never have to drain these prefetches early.
    if constexpr (PART == 2) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int r = (tid + NTH * j) / VPRV;
        const uint32_t o = (full || r < len_) ? of.v[j] : (uint32_t)((tid + NTH * j) % VPRV) * 16u;
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(vb) + o));
      }
    }
    if constexpr (PART == 3) {
      // T's upper-right 32 x 32 quadrant is zero and never read (the U product's
      // 32-column steps stay at or below the diagonal): not loaded
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int i = tid + NTH * j;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        t[j] = zero;
        if (!t_quadrant(i))
          t[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(ts) + (uint32_t)i * 16u);
      }
    }
  }

  // SQ = false: the chunk produces no output (a lookback chunk), Q is not staged
  template <int KS, int CS, int VS, bool SQ = WITH_Q>
  __device__ __forceinline__ void store(E* sK, E* sQ, E* sV, E* sT, float* sB, bool beta_bf16,
                                        bool vzero, int tid) const {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (len == kChunk && !vzero) {   // full chunk: no masking
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int i = tid + NTH * j, r = i / VPRK, cv = i % VPRK;
        const int lr = tord(r);
        *reinterpret_cast<u32x4*>(sK + lr * KS + cv * EPV) = k[j];
        if constexpr (WITH_Q && SQ) *reinterpret_cast<u32x4*>(sQ + lr * KS + cv * EPV) = q[j];
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = tid + NTH * j, r = i / VPRV, cv = i % VPRV;
        *reinterpret_cast<u32x4*>(sV + r * VS + cv * EPV) = v[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int i = tid + NTH * j, r = i / VPRK, cv = i % VPRK;
        const bool ok = r < len;
        const int lr = tord(r);
        *reinterpret_cast<u32x4*>(sK + lr * KS + cv * EPV) = ok ? k[j] : zero;
        if constexpr (WITH_Q && SQ) *reinterpret_cast<u32x4*>(sQ + lr * KS + cv * EPV) = ok ? q[j] : zero;
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = tid + NTH * j, r = i / VPRV, cv = i % VPRV;
        *reinterpret_cast<u32x4*>(sV + r * VS + cv * EPV) = (r < len && !vzero) ? v[j] : zero;
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int i = tid + NTH * j, r = i / VPRT, cv = i % VPRT;
      if (!t_quadrant(i)) *reinterpret_cast<u32x4*>(sT + tord(r) * CS + cv * EPV) = t[j];
    }
    if (tid < kChunk) {
      const float bf = beta_bf16 ? __uint_as_float(b << 16) : __uint_as_float(b);
      sB[tid] = tid < len ? bf : 0.f;
    }
  }
};

// P tile pairs (query tile, key tile) in tile order: tiles 0 and 1 hold rows
// 0..31 interleaved, tiles 2 and 3 rows 32..63, so the twelve pairs with some
// key <= query are (0|1, 0|1) and (2|3, 0..3), dealt round-robin to the waves.
__device__ __forceinline__ void p_pair(int i, int& qt, int& kt) {
  if (i < 4) { qt = i >> 1; kt = i & 1; }
  else { qt = 2 + ((i - 4) >> 2); kt = (i - 4) & 3; }
}

// PASS (kPass3 / kPass1 / kCkpt) is a template parameter so that each pass compiles
// to its own straight-line code and shows up as its own kernel in profiles.
template <typename E, int DK, int NCW, int NW, int PASS>
__global__ __launch_bounds__(64 * NW, (NW == 4 && (PASS == kPass3 || sizeof(E) == 4)) ? 1 : 2) void fused_forward_kernel(Problem p,
                                                                                      FwdPlan plan) {
  using Cfg = FwdCfg<E, DK, NCW, NW>;
  using M = Mma<E>;
  using frag = typename M::frag;
  constexpr int BV = Cfg::BV, NCT = Cfg::NCT, NKT = Cfg::NKT, NKS = Cfg::NKS;
  constexpr int KS = Cfg::KS, CS = Cfg::CS, VS = Cfg::VS;

  constexpr bool OUT = PASS == kPass3;
  // Staging buffers: bf16 chunks are double-buffered (chunk c+1 is staged at the end
  // of chunk c's step, so one barrier per chunk suffices); fp32 tiles only fit once.
  constexpr int NB = sizeof(E) == 2 ? 2 : 1;
  __shared__ __align__(16) E sKb[NB][kChunk * KS];     // tile-order rows
  __shared__ __align__(16) E sQb[NB][OUT ? kChunk * KS : 8];  // tile-order rows
  __shared__ __align__(16) E sTb[NB][kChunk * CS];     // tile-order rows
  // P of chunks c and c-1 (O of a chunk is formed during the next chunk): tile-order
  // query rows, natural keys
  __shared__ __align__(16) E sP[OUT ? 2 : 1][OUT ? kChunk * CS : 8];
  __shared__ __align__(16) E sVb[NB][kChunk * VS];     // natural rows
  __shared__ __align__(16) float sGb[NB][kChunk], sGamb[NB][kChunk], sGamSb[NB][kChunk],
      sDecb[NB][kChunk], sBetb[NB][kChunk];
  // the buffer set of the chunk being computed (the step lambdas read through these)
  E *sK = sKb[0], *sQ = sQb[0], *sT = sTb[0], *sV = sVb[0];
  float *sG = sGb[0], *sGam = sGamb[0], *sGamS = sGamSb[0], *sDec = sDecb[0], *sBet = sBetb[0];
  auto use_buffers = [&](int b) {
    sK = sKb[b]; sQ = sQb[b]; sT = sTb[b]; sV = sVb[b];
    sG = sGb[b]; sGam = sGamb[b]; sGamS = sGamSb[b]; sDec = sDecb[b]; sBet = sBetb[b];
  };

  if constexpr (PASS == kPass1) {
    if (plan.cp.ncorr && *plan.cp.ncorr == 0u) return;   // no head takes the correction
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar table reads
  const int r16 = lane & 15, q = lane >> 4;
  const int H = p.H, dv = p.dv;
  // XCD-aware decode of the 1-D grid: workgroups are dealt to the 8 XCDs round-robin
  // by id, so every column block of one unit gets id = unit (mod 8) and the unit's
  // K, T (and shared V) reads are served by one XCD's L2.  Padding ids past the last
  // unit exit at once.
  const int64_t bid = blockIdx.x;
  // column blocks per unit: pass 1 also runs dk identity columns after the dv value
  // columns (the backward's maps: the identity columns alone)
  const bool bwd_maps = PASS == kPass1 && plan.bwd_maps;
  const int ncb = ((PASS == kPass1) ? (bwd_maps ? DK : dv + DK) : dv) / BV;
  const int64_t rest = bid >> 3;
  const int cb = (int)(rest % ncb);
  const int64_t unit = (rest / ncb) * 8 + (bid & 7);
  if (unit >= plan.units) return;
  const int col0 = (bwd_maps ? dv : 0) + cb * BV;   // first (value or identity) column
  const int wcol = wave * NCW;             // wave's first column inside the block

  // Pass 1 takes the gate scan's work list when there is one: only units that run
  // are dispatched, ahead of none that exit (exiting workgroups dispatched first
  // leave the working ones packed two to a CU where one each would fit), and a
  // pair's segments, one run of the list, spread over all XCDs.  Without it pass 1
  // numbers every (segment, head) head-major, to the same spreading end.  Pass 3
  // numbers them segment-major, in the plan's segment order when there is one
  // (packed input: longest segments first), so units dispatched together have
  // similar lengths.
  int h;
  int64_t sg;                              // global segment index
  if constexpr (PASS == kPass1) {
    if (plan.cp.p1_slots) {   // (entries read back are clamped to the slots)
      if (unit >= (int64_t)plan.cp.ncorr[1]) return;
      const int64_t segs_all =
          plan.seg_off ? (int64_t)plan.seg_off[p.N]
                       : (int64_t)p.N * max((int64_t)1, ((p.T + kChunk - 1) / kChunk + plan.seg_chunks - 1) /
                                                            plan.seg_chunks);
      const int64_t slot = min(max((int64_t)plan.cp.p1_slots[unit], (int64_t)0), segs_all * H - 1);
      h = (int)(slot % H);
      sg = slot / H;
    } else {
      const int64_t nseg = plan.units / H;   // segments over all sequences
      h = (int)(unit / nseg);
      sg = unit - (int64_t)h * nseg;
    }
  } else {
    h = (int)(unit % H);
    sg = plan.seg_order ? plan.seg_order[unit / H] : unit / H;   // longest segments first
  }
  int n, seg;
  if (plan.seg_off) {
    n = seq_of_chunk(sg, plan.seg_off, p.N, 0);
    seg = (int)(sg - plan.seg_off[n]);
  } else if (p.cu) {   // packed without segment tables: one segment per sequence
    n = (int)sg;
    seg = 0;
  } else {
    const int64_t nch_all = (p.T + kChunk - 1) / kChunk;
    const int64_t segs = max((int64_t)1, (nch_all + plan.seg_chunks - 1) / plan.seg_chunks);
    n = (int)(sg / segs);
    seg = (int)(sg - (int64_t)n * segs);
  }
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  const int c_begin = seg * plan.seg_chunks;
  const int c_end = min(nch, c_begin + plan.seg_chunks);
  const int nh = n * H + h;
  const bool last_seg = c_end >= nch;
  // (clamped: a window read from a workspace the gate scan did not fill stays inside
  // the segment's sequence)
  const int W = (plan.cp.seg_win && !plan.cp.force_correction)
                    ? min(max(plan.cp.seg_win[sg * H + h], 0), c_begin) : 0;

  // start state and the chunk range: [c_start, c_end) is run, O is written from c_out
  enum { kZero, kH0, kBuf, kEye };
  int init = kZero, c_start = c_begin, c_out = c_begin;
  bool mcols = false;   // pass 1: this block carries the transition-matrix columns
  if constexpr (PASS == kPass1) {
    if (bwd_maps) {
      if (seg == 0) return;   // the backward's merge needs no map of a first segment
    } else {
      // last segments and window heads need no pass 1; a head's windows are all set or
      // all zero, and its second segment (there is one: this is not the last) holds one
      if (last_seg) return;
      if (plan.cp.seg_win && !plan.cp.force_correction && plan.cp.seg_win[(sg - seg + 1) * H + h] > 0)
        return;
    }
    mcols = col0 >= dv;
    init = mcols ? kEye : kZero;
    c_out = c_end;
  } else if (seg == 0) {
    init = p.h0 ? kH0 : kZero;
  } else if (W > 0) {
    c_start = c_begin - W;
    if (c_start <= 0) { c_start = 0; init = p.h0 ? kH0 : kZero; }
  } else {
    init = kBuf;
  }
  const int vcol0 = mcols ? 0 : col0;  // value columns addressed by this block

  const int row_qk = H * DK, row_v = H * dv;   // element strides between tokens
  const E* Qb = reinterpret_cast<const E*>(p.q) + si.tok0 * row_qk + (int64_t)h * DK;
  const E* Kb = reinterpret_cast<const E*>(p.k) + si.tok0 * row_qk + (int64_t)h * DK;
  const E* Vb = reinterpret_cast<const E*>(p.v) + si.tok0 * row_v + (int64_t)h * dv + vcol0;
  E* Ob = reinterpret_cast<E*>(p.o) + si.tok0 * row_v + (int64_t)h * dv + vcol0 + wcol;
  const float* Gb = p.g + si.tok0 * H + h;
  const int bsz = p.beta_bf16 ? 2 : 4;
  const char* Bb = reinterpret_cast<const char*>(p.beta) + (si.tok0 * H + h) * bsz;
  const E* Tm = reinterpret_cast<const E*>(plan.Tmat);

  // ---- initial state (tile order: slot i of lane group q in tile t is dk row prow(t, 4q+i))
  f32x4 hs[NKT][NCT];
  {
    const int64_t sg_slot = sg * H + h;
    const float* src = init == kH0 ? p.h0 + (int64_t)nh * DK * dv
                                   : (init == kBuf ? plan.cp.hstart + sg_slot * DK * dv : nullptr);
    const int mc = col0 - dv + wcol + r16;   // identity column (pass-1 matrix block)
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = prow(t, 4 * q + i);
          float x = 0.f;
          if (src) x = src[(int64_t)r * dv + col0 + wcol + ct * 16 + r16];
          else if (init == kEye) x = (r == mc + ct * 16) ? 1.f : 0.f;
          hs[t][ct][i] = x;
        }
  }

  // Prefetch depth: the global loads of chunk c + PF are issued while chunk c is
  // computed, from PF register sets used in turn.  Pass 1 has the registers for two.
  constexpr int PF = (PASS != kPass3) ? 2 : 1;
  using Stage = ChunkRegs<E, DK, BV, Cfg::NT, PASS == kPass3>;
  Stage pf[PF];
  typename Stage::Offsets offs;
  offs.init(row_qk, row_v, H, tid);
  auto issue_part = [&](auto part_tag, Stage& st, int c) {
    constexpr int PART = decltype(part_tag)::value;
    const int64_t t0 = (int64_t)c * kChunk;
    const E* ts = Tm + ((si.chunk0 + c) * H + h) * (int64_t)(kChunk * kChunk);
    __builtin_amdgcn_sched_barrier(0);
    st.template load<PART>(Qb + t0 * row_qk, Kb + t0 * row_qk, Vb + t0 * row_v, ts, Gb + t0 * H,
                           Bb + t0 * H * bsz, p.beta_bf16, min(kChunk, si.len - c * kChunk), offs, tid);
    __builtin_amdgcn_sched_barrier(0);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  if (c_start < c_end) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int cc = min(c_start + k, c_end - 1);
      issue_part(P0{}, pf[k], cc);
      issue_part(P1{}, pf[k], cc);
      issue_part(P2{}, pf[k], cc);
      issue_part(P3{}, pf[k], cc);
    }
  }

  // per-row gates in tile order: rows prow(u, 4q) .. +3 are consecutive, one 16-byte read
  auto rows4 = [&](const float* v, int u) {
    return *reinterpret_cast<const f32x4*>(v + prow(u, 4 * q));
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // O of a chunk is completed during the next chunk (after its first barrier), from
  // these registers and that chunk's P: Yp = scale diag(gamma) Q h (transposed
  // tiles), ubp = U packed as MFMA operands.
  f32x4 Yp[4][NCT];
  frag ubp[2][NCT];
  auto emit_o = [&](int c, int len) {
    E* ob = Ob + (int64_t)c * kChunk * row_v;
    const E* sp = sP[c & 1];
    frag aP[6];   // P fragments (u, s), ordered as the T fragments of the U product
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s <= (u >> 1); ++s) aP[u < 2 ? u : 2 * u - 2 + s] = lds_frag(sp, CS, 16 * u + r16, 32 * s, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int s = 0; s <= (u >> 1); ++s) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Yp[u][ct] = M::run(ubp[s][ct], aP[u < 2 ? u : 2 * u - 2 + s], Yp[u][ct]);
      }
    }
    if constexpr (sizeof(E) == 2) {
      // 16-byte stores: for the tile pair (u, u+1), v_permlane16_swap hands lane group
      // q^1 the other group's four columns, so an even group holds eight consecutive
      // columns of tile u's row and an odd group those of tile u+1's row
#pragma unroll
      for (int u = 0; u < 4; u += 2) {
        const int row = (q & 1) ? prow(u + 1, r16) : prow(u, r16);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const uint2 a = pack_bf16x4(Yp[u][ct]), b = pack_bf16x4(Yp[u + 1][ct]);
          const auto sx = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
          const auto sy = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
          const u32x4 v = {sx[0], sy[0], sx[1], sy[1]};
          if (row < len) *reinterpret_cast<u32x4*>(ob + row * row_v + 16 * ct + 8 * (q >> 1)) = v;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = prow(u, r16);
        if (row < len) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) store4(ob + row * row_v + 16 * ct + 4 * q, Yp[u][ct]);
        }
      }
    }
  };

  auto pstep = [&](int c) {
    // ---- P = scale (Q K^T) * Gamma for this chunk's O (formed during the next chunk):
    //      rows = queries in tile order, columns = keys in natural order; computed as
    //      P^T = K Q^T so a lane holds four consecutive keys
    {
      E* sp = sP[c & 1];
#pragma unroll
      for (int pt = 0; pt < (12 + NW - 1) / NW; ++pt) {
        const int pi = wave + NW * pt;
        if (pi < 12) {
          int qt, kt;
          p_pair(pi, qt, kt);
          f32x4 acc = zero4;
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            acc = M::run(lds_frag(sK, KS, 16 * kt + r16, 32 * s, q),
                         lds_frag(sQ, KS, 16 * qt + r16, 32 * s, q), acc);
          const int qrow = prow(qt, r16), key0 = prow(kt, 4 * q);
          const float Gq = sG[qrow];
          const f32x4 Gk = *reinterpret_cast<const f32x4*>(sG + key0);
          E* dst = sp + (16 * qt + r16) * CS + key0;
          f32x4 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = key0 + i <= qrow ? p.scale * acc[i] * fast_exp(Gq - Gk[i]) : 0.f;
          store4(dst, pv);   // four adjacent keys: one 8-byte (bf16) or 16-byte store
        }
      }
    }
  };

  // One chunk after staging; EMIT (compile-time) selects whether O is produced, so
  // each variant is straight-line code.
  auto step = [&](auto emit_tag, int c, float gC, auto&& load_part) {
    constexpr bool EMIT = decltype(emit_tag)::value;
    if constexpr (EMIT) pstep(c);
    load_part(P1{});
    // ---- X = K h; Y^T = h^T Q^T (operands swapped: a lane holds four consecutive value
    //      columns of one query row, the layout of the O store); first products start at zero
    f32x4 X[4][NCT];
    // the step's operand fragments are read as one batch ahead of their MFMAs (the
    // scheduling barrier keeps the compiler from trading the reads in flight for
    // registers, which would expose one LDS round trip per MFMA).  A wave raises its
    // issue priority over its MFMA batches (here, in U and in the state update): the
    // SIMD's other wave usually runs the same phase, and favouring the wave that has its
    // operands measured about 1% faster per call on every workload.
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      frag aK[4], aQ[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        aK[u] = lds_frag(sK, KS, 16 * u + r16, 32 * s, q);
        if constexpr (EMIT) aQ[u] = lds_frag(sQ, KS, 16 * u + r16, 32 * s, q);
      }
      frag hb[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) hb[ct] = M::pack(hs[2 * s][ct], hs[2 * s + 1][ct]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) X[u][ct] = M::run(aK[u], hb[ct], s == 0 ? zero4 : X[u][ct]);
        if constexpr (EMIT) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) Yp[u][ct] = M::run(hb[ct], aQ[u], s == 0 ? zero4 : Yp[u][ct]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (EMIT) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float gs = sGamS[prow(u, r16)];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Yp[u][ct] = Yp[u][ct] * gs;
      }
    }
    load_part(P2{});
    // ---- W = diag(beta) (V - diag(gamma) X), in place; V read in accumulator layout
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int cb = wcol + 16 * ct;
        const f32x4 vv = col_read4(sV, VS, prow(u, 4 * q), cb + r16, cb + 4 * (r16 & 3));
        X[u][ct] = rows4(sBet, u) * (vv - rows4(sGam, u) * X[u][ct]);
      }
    // ---- U = T W (T lower triangular: row tiles 0,1 need contraction step 0 only).
    //      The checkpoint pass (bf16) carries W, and d U below, as bf16 hi + lo pairs:
    //      the backward's gate gradient is sensitive to the states' rounding.
    constexpr bool SPLIT = PASS == kCkpt && sizeof(E) == 2;
    frag wb[2][NCT], wl[2][NCT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        wb[s][ct] = M::pack(X[2 * s][ct], X[2 * s + 1][ct]);
        if constexpr (SPLIT) wl[s][ct] = pack_residual(X[2 * s][ct], X[2 * s + 1][ct]);
      }
    f32x4 U[4][NCT];
    {
      frag aT[6];   // T fragments (u, s): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int s = 0; s <= (u >> 1); ++s) aT[u < 2 ? u : 2 * u - 2 + s] = lds_frag(sT, CS, 16 * u + r16, 32 * s, q);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int s = 0; s <= (u >> 1); ++s)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            U[u][ct] = M::run(aT[u < 2 ? u : 2 * u - 2 + s], wb[s][ct], s == 0 ? zero4 : U[u][ct]);
            if constexpr (SPLIT) U[u][ct] = M::run(aT[u < 2 ? u : 2 * u - 2 + s], wl[s][ct], U[u][ct]);
          }
    }
      __builtin_amdgcn_s_setprio(0);
    load_part(P3{});
    frag ubd[2][NCT], ubl[2][NCT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if constexpr (EMIT) ubp[s][ct] = M::pack(U[2 * s][ct], U[2 * s + 1][ct]);
        const f32x4 dlo = U[2 * s][ct] * rows4(sDec, 2 * s), dhi = U[2 * s + 1][ct] * rows4(sDec, 2 * s + 1);
        ubd[s][ct] = M::pack(dlo, dhi);
        if constexpr (SPLIT) ubl[s][ct] = pack_residual(dlo, dhi);
      }
    // ---- h <- gamma_last h + K^T (diag(d) U); K^T fragments by LDS transpose reads,
    //      two dk tiles' fragments read as a batch ahead of their MFMAs
#pragma unroll
    for (int t0 = 0; t0 < NKT; t0 += 2) {
      frag aKt[2][2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int t = t0 + dt;
        const int own = prow(t, r16), supply = prow(t, 4 * (r16 & 3));
#pragma unroll
        for (int s = 0; s < 2; ++s)
          aKt[dt][s] = col_frag(sK, KS, 32 * s + 4 * q, 32 * s + 16 + 4 * q, own, supply);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) hs[t0 + dt][ct] *= gC;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            hs[t0 + dt][ct] = M::run(aKt[dt][s], ubd[s][ct], hs[t0 + dt][ct]);
            if constexpr (SPLIT) hs[t0 + dt][ct] = M::run(aKt[dt][s], ubl[s][ct], hs[t0 + dt][ct]);
          }
    }
      __builtin_amdgcn_s_setprio(0);
  };

  // Stages chunk cs (registers of st) in buffer b: the gates of chunk cs are scanned in
  // registers (every wave holds all rows: lane = chunk row); returns gamma_last.
  // q_tag (compile-time): whether Q is staged (a lookback chunk has no output).
  auto stage = [&](auto q_tag, Stage& st, int cs, int b) {
    const int len = min(kChunk, si.len - cs * kChunk);
    const float G = wave_inclusive_scan_dpp(lane < len ? st.g : 0.f);
    const float Glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), kChunk - 1));
    st.template store<KS, CS, VS, decltype(q_tag)::value>(sKb[b], sQb[b], sVb[b], sTb[b], sBetb[b],
                                                          p.beta_bf16, mcols, tid);
    if (wave == 0) {
      const float gam = fast_exp(G);
      sGb[b][lane] = G;
      sGamb[b][lane] = gam;
      sGamSb[b][lane] = gam * p.scale;
      sDecb[b][lane] = fast_exp(Glast - G);
    }
    return fast_exp(Glast);
  };

  // One chunk: ld receives the loads of chunk c+PF (past the last chunk this reloads
  // it, unused: the load count per step stays fixed, which keeps the step free of
  // waits on them); part 0 goes out after the previous chunk's O stores, the others
  // from inside the step.  With two buffers, sg (holding chunk c+1) is staged at the
  // end of the step, so the next chunk starts right after the one barrier.
  int len_prev = 0;
  float gC = 0.f;
  // q_tag (compile-time): whether chunk c + PF is loaded with its Q (false while it is
  // still a lookback chunk: no output, so no Q traffic).
  auto chunk = [&](auto q_tag, Stage& ld, Stage& sg, int c) {
    constexpr bool LOADQ = decltype(q_tag)::value;
    const int len = min(kChunk, si.len - c * kChunk);
    if constexpr (PASS == kCkpt) {   // the state at this chunk's start
      float* dst = plan.ckpt + ((si.chunk0 + c) * H + h) * (int64_t)DK * dv;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          *reinterpret_cast<f32x4*>(dst + ckpt_offset(prow(t, 4 * q), col0 + wcol + ct * 16 + r16, dv)) =
              hs[t][ct];
    }
    if constexpr (NB == 1) {
      gC = stage(std::true_type{}, ld, c, 0);
      __syncthreads();
    }
    use_buffers(c % NB);
    const int cn = min(c + PF, c_end - 1);
    auto load_part = [&](auto part) {
      if constexpr (LOADQ || decltype(part)::value != 1) issue_part(part, ld, cn);
    };
    if constexpr (OUT) {
      if (c - 1 >= c_out && c - 1 >= c_start) emit_o(c - 1, len_prev);
    }
    issue_part(P0{}, ld, cn);
    if constexpr (OUT) {
      if (c >= c_out) step(std::true_type{}, c, gC, load_part);
      else step(std::false_type{}, c, gC, load_part);
    } else {
      step(std::false_type{}, c, gC, load_part);
    }
    len_prev = len;
    if constexpr (NB == 2) gC = stage(q_tag, sg, min(c + 1, c_end - 1), (c + 1) % NB);
    __syncthreads();
  };
  int c = c_start;
  if (c_start < c_end) {
    if constexpr (NB == 2) {
      gC = stage(std::true_type{}, pf[0], c_start, c_start % NB);
      __syncthreads();
    }
    if constexpr (PF == 1) {
      if constexpr (OUT) {   // lookback chunks followed by another lookback chunk: no Q
        for (; c + 1 < c_out && c < c_end; ++c) chunk(std::false_type{}, pf[0], pf[0], c);
      }
      for (; c < c_end; ++c) chunk(std::true_type{}, pf[0], pf[0], c);
    } else {
      for (; c + 2 <= c_end; c += 2) {   // no conditions inside: fixed load counts
        chunk(std::true_type{}, pf[0], pf[1], c);
        chunk(std::true_type{}, pf[1], pf[0], c + 1);
      }
      if (c < c_end) chunk(std::true_type{}, pf[0], pf[1], c);
    }
  }
  if constexpr (OUT) {
    if (c_end - 1 >= c_out && c_end - 1 >= c_start) emit_o(c_end - 1, len_prev);
  }

  // ---- end state: final state (pass 3, last segment), S* (pass 1 value columns), or
  //      M (pass 1 identity columns) as bf16 high and low parts for the merge's MFMAs,
  //      in the merge's operand order (mfrag_offset)
  if (PASS == kPass1 && mcols) {
    // the backward's maps: the transpose, at the segment's backward slot
    int64_t slot = sg * H + h;
    if (bwd_maps) {
      const int64_t sg0 = sg - seg;
      const int S = plan.seg_off ? (int)(plan.seg_off[n + 1] - plan.seg_off[n])
                                 : (int)max((int64_t)1, ((p.T + kChunk - 1) / kChunk + plan.seg_chunks - 1) /
                                                            plan.seg_chunks);
      slot = bwd_slot(sg0, S, seg) * H + h;
    }
    bf16* mhi = reinterpret_cast<bf16*>(plan.cp.mcorr) + slot * 2 * DK * DK;
    bf16* mlo = mhi + DK * DK;
    const int mc = col0 - dv + wcol + r16;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = hs[t][ct][i];
          const bf16 hi = (bf16)x;
          const int r = prow(t, 4 * q + i), c = mc + ct * 16;
          const int64_t at = bwd_maps ? mfrag_offset<DK>(c, r) : mfrag_offset<DK>(r, c);
          mhi[at] = hi;
          mlo[at] = (bf16)(x - (float)hi);
        }
    return;
  }
  if constexpr (PASS == kPass1) {
    // S* as the merge's accumulator tiles (sfrag_offset): the four rows a lane holds
    // in a tile are consecutive (prow(t, 4q + i) = prow(t, 4q) + i), so each tile
    // leaves as one 16-byte store per lane
    float* dst = plan.cp.sstar + (sg * H + h) * DK * dv;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(dst + sfrag_offset<DK>(prow(t, 4 * q), col0 + wcol + ct * 16 + r16)) =
            hs[t][ct];
  } else if (PASS == kPass3 && last_seg && p.hT) {
    float* dst = p.hT + (int64_t)nh * DK * dv + col0;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(int64_t)prow(t, 4 * q + i) * dv + wcol + ct * 16 + r16] = hs[t][ct][i];
  }
}

// 1-D grid of ceil(units / 8) * 8 * column blocks (see the decode in the kernel).
template <typename E, int DK, int PASS>
static hipError_t launch_dk(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  // pass 1 also runs dk transition-matrix columns after the dv value columns (the
  // backward's maps: those alone)
  const int cols = PASS == kPass1 ? (plan.bwd_maps ? DK : p.dv + DK) : p.dv;
  const int64_t groups = (plan.units + 7) / 8;
  if (groups * 8 > kMaxDispatchItems / (4 * cols))   // 4 threads per column in either shape
    return hipErrorInvalidConfiguration;
  if constexpr (sizeof(E) == 2) {
    // 128 columns per workgroup as 8 waves x 16 columns: two waves per SIMD.  Pass 1
    // always takes 64-column workgroups: both shapes reach the same throughput per CU,
    // and pass 1 usually runs few (sequence, head) pairs, so the narrower blocks
    // spread its units over twice as many CUs.
    if (p.dv % 128 == 0 && cols % 128 == 0 &&
        (PASS == kPass3 ? plan.value_block != 64 : plan.pass1_block == 128)) {
      const int ncb = cols / 128;
      hipExtLaunchKernelGGL(fused_forward_kernel<E, DK, 16, 8, PASS>, dim3((unsigned)(groups * 8 * ncb)),
                            dim3(512), 0, s, ev.start, ev.stop, 0, p, plan);
      return hipGetLastError();
    }
  }
  // 64 columns per workgroup as 4 waves x 16 columns (fp32 tiles only fit LDS this way)
  const int ncb = cols / 64;
  hipExtLaunchKernelGGL(fused_forward_kernel<E, DK, 16, 4, PASS>, dim3((unsigned)(groups * 8 * ncb)),
                        dim3(256), 0, s, ev.start, ev.stop, 0, p, plan);
  return hipGetLastError();
}

template <typename E, int DK>
static hipError_t launch_pass(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  if (plan.mode == kPass1) return launch_dk<E, DK, kPass1>(p, plan, s, ev);
  if (plan.mode == kCkpt) return launch_dk<E, DK, kCkpt>(p, plan, s, ev);
  return launch_dk<E, DK, kPass3>(p, plan, s, ev);
}

hipError_t launch_fused_forward(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  if (plan.units == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (p.qkv_bf16) return p.dk == 128 ? launch_pass<bf16, 128>(p, plan, s, ev) : launch_pass<bf16, 64>(p, plan, s, ev);
  return p.dk == 128 ? launch_pass<float, 128>(p, plan, s, ev) : launch_pass<float, 64>(p, plan, s, ev);
}

}  // namespace gdn
