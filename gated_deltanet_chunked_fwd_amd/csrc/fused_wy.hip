// Steps 1-4 of the chunked WY form in one pass on gfx950 (bf16 storage): per
// (sequence, head, segment) one workgroup walks the chunks with the state of all
// value columns in registers, forms each chunk's inverse itself, and writes only O
// and the final state.  Neither the inverse T nor W, U or S ever reaches HBM.
//
// FlashQLA talk transcript (tokendh.com): chunked-WY section (step 1, the chunk's
// K K^T and its inverse; steps 2-4, the projections, the chunk-serial state
// recurrence and the output); pain-points section (no W/U/S round trip through
// HBM); algebraic-rewrites section (Gamma in log space; the forward merge "form V
// minus S first, then apply gamma").  With h = S^T the state at chunk start, G the
// chunk-local cumsum of g, gamma = exp(G), Gamma_rs = exp(G_r - G_s) (r >= s),
// d = exp(G_last - G):
//
//   A  = strict_lower(diag(beta) K K^T * Gamma),  T = (I + A)^{-1}        (step 1)
//   V' = V - diag(gamma) K h,   U = (T diag(beta)) V'                      (step 2)
//   O  = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)                     (step 4)
//   h <- gamma_last h + K^T (diag(d) U)                                    (step 3)
//
// Roles.  Only the last three lines depend on h; step 1 and P = scale (Q K^T) *
// Gamma do not, so they are formed ahead of the recurrence by other waves:
//   * NCH = 4 "chain" waves own CW = BV / 4 value columns each (all dk rows of h
//     in fp32 accumulator tiles, tile order, gdn_device.h) and run, per chunk, only
//     X = K h, Y = Q h, V', U, O and the state update.  Every K, Q, K^T, T and P
//     fragment a chain wave reads from LDS feeds CW / 16 MFMAs (one per 16-column
//     tile).  Each chain wave also stages its own V columns: loaded from HBM one
//     step ahead, written to its private LDS columns at the start of the step.
//   * NP = 4 "prep" waves own every fourth chunk.  A prep wave loads its chunk's
//     rows from HBM straight into MFMA operand registers, scans the gates, forms
//     the gated Gram matrix and its inverse (16 x 16 diagonal blocks by forward
//     substitution in fp32, the rest by two doubling levels of MFMA products) and
//     P, and stages K, Q, T, P and the gate tables in LDS for the chain.
// One workgroup barrier per chunk step.  During step i the chain computes chunk i
// from LDS buffer set i % 2 (K: ring slot i % 3).  A prep wave spreads one chunk
// over four steps, one phase per step (see the schedule at the prep loop); each
// step has exactly one prep wave in each phase.  The first NP + 1 steps only
// prepare (the chain waits at their barriers).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

template <int DK, int BV>
struct WyCfg {
  static constexpr int NCH = 4;                // chain waves
  static constexpr int CW = BV / NCH;          // value columns per chain wave (16 or 32)
  static constexpr int NCT = CW / 16;          // 16-column tiles per chain wave
  static constexpr int NP = 4;                 // prep waves
  static constexpr int NW = NCH + NP;
  static constexpr int NT = 64 * NW;
  static constexpr int NKS = DK / 32;          // contraction steps over dk
  static constexpr int NKT = DK / 16;          // dk tiles of the state
  // LDS row strides (elements): rows feeding 16-byte fragment reads and 8-byte
  // transpose reads are 8 (mod 32) dwords apart (conflict-free on gfx950's LDS)
  static constexpr int KS = DK + 16;           // sK, sQ: tile-order rows
  static constexpr int VS = BV + 16;           // sV: natural rows
  static constexpr int VPR = CW / 8;           // 16-byte pieces per row of a chain wave's V
  static constexpr int NVP = kChunk * VPR / 64;  // V pieces per chain lane
  // T and P: the six 16 x 32 operand fragments of a lower-triangular 64 x 64 matrix
  // (tri_frag), each stored as 64 lanes x 8 elements in lane order
  static constexpr int FR = 512;
  static constexpr int TF = 6;
  // fp32 scratch of the diagonal-block substitution, shared by the prep waves (one of
  // them substitutes in any step): the diagonal A blocks (row-major, block stride
  // ABS) and the diagonal T blocks (column-major, column stride TCS)
  static constexpr int ABS = 260, TCS = 20, TBS = 16 * TCS;
  static constexpr int INV = 4 * ABS + 4 * TBS;
};

// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format; accesses at or past the resource's byte size are dropped (stores) or
// read as zero (loads).
constexpr int kRawBufferFlags = 0x00020000;

// The ten 16 x 16 blocks (a, b), b <= a, of a lower-triangular 64 x 64 chunk matrix.
__device__ __forceinline__ void lower_block(int i, int& a, int& b) {
  a = i < 1 ? 0 : i < 3 ? 1 : i < 6 ? 2 : 3;
  b = i - (a * (a + 1)) / 2;
}

// Operand fragments of a lower-triangular chunk matrix whose rows are in tile order
// (row slot 16 u + r) and whose columns are natural: fragment (u, s) covers row
// tile u and columns 32 s .. 32 s + 31; tiles 0 and 1 need s = 0 only.
__device__ __forceinline__ constexpr int tri_frag(int u, int s) { return u < 2 ? u : 2 * u - 2 + s; }

// Element offset, in the fragment-ordered storage, of the four entries that lane
// (r, q) holds of block (a, b) (row 16 a + r, columns 16 b + 4 q .. +3).
__device__ __forceinline__ int tri_offset(int a, int b, int r, int q) {
  const int slot = tord(16 * a + r);
  const int u = slot >> 4, rr = slot & 15;
  const int fq = 2 * (b & 1) + (q >> 1);
  return tri_frag(u, b >> 1) * 512 + (16 * fq + rr) * 8 + 4 * (q & 1);
}

// Orders this wave's LDS accesses across its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// D(X^T), D(Y), acc -> acc + D(X Y) for 16 x 16 blocks held in accumulator layout:
// slot e of lane (r, q) is X^T[4q+e][r] and Y[4q+e][r]; one bf16 16x16x16 MFMA on
// the operands rounded to bf16 (T leaves as bf16, a rounding of the same size).
__device__ __forceinline__ f32x4 mm16(const f32x4& xt, const f32x4& y, f32x4 acc) {
  const i16x4 a = __builtin_bit_cast(i16x4, pack_bf16x4(xt));
  const i16x4 b = __builtin_bit_cast(i16x4, pack_bf16x4(y));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}

// An opaque zero (an instruction the compiler cannot see through): per-lane indices
// offset by it are recomputed inside a loop instead of being hoisted and spilled.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// One chunk held by a prep wave from its first loads to its last LDS write.
template <int DK>
struct PrepChunk {
  bf16x8 kf[4][DK / 32];    // K rows 16a + r, columns 32s + 8q .. +7 (lane (r, q))
  bf16x8 qf[4][DK / 32];    // Q, same layout
  float g;                  // gate of row = lane, as loaded (masked in gates_gram)
  uint32_t braw;            // beta of row = lane, raw storage bits (bf16 or fp32)
  int len;                  // rows of the chunk
  f32x4 ad[4];              // D(A_aa): diagonal blocks of A, slot i = A[16a+4q+i][16a+r]
  f32x4 at[6];              // D(A_ab^T), b < a (order of lower_block without the diagonal)
  f32x4 td[4], tdt[4];      // D(T_aa), D(T_aa^T)
  uint2 tb[10];             // T blocks, bf16, lane (r, q): row 16a + r, columns 16b + 4q .. +3
  uint2 pb[10];             // P blocks, same layout (query rows, key columns)
};

}  // namespace

// PASS: kPass3 (steps 1-4 with O) or kPass1 (the split's pass 1: a segment from a zero
// state on the value columns -> S*, and with V = 0 from the identity on dk more columns
// -> M; every chunk a lookback step, no Q, no O; the chunk inverses formed here as in
// pass 3, so a split plan runs no separate chunk-inverse kernel).
template <int DK, int BV, int PASS>
__global__ __launch_bounds__(512, 1) void fused_wy_kernel(Problem p, FwdPlan plan) {
  using Cfg = WyCfg<DK, BV>;
  static_assert(Cfg::NT == 512, "launch bounds");
  using M = Mma<bf16>;
  using frag = bf16x8;
  constexpr int NCH = Cfg::NCH, NP = Cfg::NP, NKS = Cfg::NKS, NKT = Cfg::NKT, NCT = Cfg::NCT;
  constexpr int KS = Cfg::KS, VS = Cfg::VS, FR = Cfg::FR;

  __shared__ __align__(16) bf16 sK[3][kChunk * KS];   // ring of three: chunk i in slot i % 3
  __shared__ __align__(16) bf16 sQ[2][kChunk * KS];
  __shared__ __align__(16) bf16 sV[kChunk * VS];      // each chain wave: its own columns
  __shared__ __align__(16) bf16 sT[2][Cfg::TF * FR];
  __shared__ __align__(16) bf16 sP[2][Cfg::TF * FR];
  __shared__ __align__(16) float sGam[2][kChunk], sGamS[2][kChunk], sDec[2][kChunk];
  __shared__ float sGC[2];
  __shared__ __align__(16) float sGB[NP][2 * kChunk];
  __shared__ __align__(16) float sInv[Cfg::INV];

  constexpr bool P1 = PASS == kPass1;
  if constexpr (P1) {
    if (plan.cp.ncorr && *plan.cp.ncorr == 0u) return;   // no head takes the correction
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int H = p.H, dv = p.dv;

  // ---- unit decode (XCD-aware: the column blocks of one unit share id mod 8, so they
  //      run on one XCD and share its L2 for K, Q, g, beta).  A launch has fewer than
  //      2^32 / 512 workgroups, so 32-bit arithmetic covers every index here.  Pass 1
  //      runs dk identity columns after the dv value columns, takes its units from the
  //      gate scan's work list when there is one (so only units that run are
  //      dispatched), else numbers every (segment, head) head-major.
  const uint32_t bid = blockIdx.x;
  // (dk < dv: the one matrix block is half used; its columns past dk stay zero and
  // are not stored)
  const uint32_t ncb = (uint32_t)((P1 ? dv + DK + BV - 1 : dv) / BV);
  const uint32_t rest = bid >> 3;
  const int cb = (int)(rest % ncb);
  const uint32_t unit = (rest / ncb) * 8u + (bid & 7u);
  if ((int64_t)unit >= plan.units) return;
  const int col0 = cb * BV;
  int h;
  int64_t sg;
  if constexpr (P1) {
    if (plan.cp.p1_slots) {   // (entries read back are clamped to the slots)
      if (unit >= plan.cp.ncorr[1]) return;
      const int64_t segs_all =
          plan.seg_off ? (int64_t)plan.seg_off[p.N]
                       : (int64_t)p.N * max((int64_t)1, ((p.T + kChunk - 1) / kChunk + plan.seg_chunks - 1) /
                                                            plan.seg_chunks);
      const int64_t slot = min(max((int64_t)plan.cp.p1_slots[unit], (int64_t)0), segs_all * H - 1);
      h = (int)(slot % H);
      sg = slot / H;
    } else {
      const uint32_t nseg = (uint32_t)(plan.units / H);   // segments over all sequences
      h = (int)(unit / nseg);
      sg = (int64_t)(unit - (uint32_t)h * nseg);
    }
  } else {
    h = (int)(unit % (uint32_t)H);
    const uint32_t sgu = unit / (uint32_t)H;
    sg = plan.seg_order ? (int64_t)plan.seg_order[sgu] : (int64_t)sgu;
  }
  int n, seg;
  if (plan.seg_off) {
    n = seq_of_chunk(sg, plan.seg_off, p.N, 0);
    seg = (int)(sg - plan.seg_off[n]);
  } else if (p.cu) {   // packed without segment tables: one segment per sequence
    n = (int)sg;
    seg = 0;
  } else {
    const uint32_t nch_all = (uint32_t)((p.T + kChunk - 1) / kChunk);
    const uint32_t sc = (uint32_t)plan.seg_chunks;
    const uint32_t segs = max(1u, (nch_all + sc - 1) / sc);
    n = (int)((uint32_t)sg / segs);
    seg = (int)((uint32_t)sg - (uint32_t)n * segs);
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
  // start state and chunk range: [c_start, c_end) is run, O is written from c_out
  enum { kZero, kH0, kBuf, kEye };
  int init = kZero, c_start = c_begin;
  int c_out = c_begin;
  bool mcols = false;   // pass 1: this block carries the transition-matrix columns
  if constexpr (P1) {
    // last segments and window heads need no pass 1; a head's windows are all set or
    // all zero, and its second segment (there is one: this is not the last) holds one
    if (last_seg) return;
    if (plan.cp.seg_win && !plan.cp.force_correction && plan.cp.seg_win[(sg - seg + 1) * H + h] > 0) return;
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
  const int nrun = max(0, c_end - c_start);

  // T and P blocks above the diagonal are zero and never written
  for (int e = tid; e < 2 * Cfg::TF * FR / 8; e += Cfg::NT) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(&sT[0][0])[e] = z;
    reinterpret_cast<u32x4*>(&sP[0][0])[e] = z;
  }

  const int row_qk = H * DK, row_v = H * dv;   // element strides between tokens
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if (wave < NCH) {
    // =========================== chain wave ===========================
    const int wcol = wave * Cfg::CW;           // wave's first column inside the block
    f32x4 hs[NKT][NCT];
    const int mc = col0 - dv + wcol + r16;   // identity column (pass 1's matrix blocks)
    {
      const float* src = init == kH0 ? p.h0 + (int64_t)nh * DK * dv
                                     : (init == kBuf ? plan.cp.hstart + (sg * H + h) * DK * dv : nullptr);
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hs[t][j][i] = src ? src[(int64_t)prow(t, 4 * q + i) * dv + col0 + wcol + 16 * j + r16]
                              : (init == kEye && prow(t, 4 * q + i) == mc + 16 * j ? 1.f : 0.f);
    }
    bf16* Ob = reinterpret_cast<bf16*>(p.o) + si.tok0 * row_v + (int64_t)h * dv + col0 + wcol;
    const bf16* Vb = reinterpret_cast<const bf16*>(p.v) + si.tok0 * row_v + (int64_t)h * dv + col0 + wcol;
    // per-lane indices, re-derived at every step from an opaque zero
    int cr16 = r16, cq = q, clane = lane;
    // this wave's V columns of chunk i, loaded one step ahead (rows past a partial
    // chunk's end read its last row: their beta is zero, so they contribute nothing)
    u32x4 vr[Cfg::NVP];
    auto load_v = [&](int i) {
      if (mcols) {   // V = 0 on the transition-matrix columns
#pragma unroll
        for (int j = 0; j < Cfg::NVP; ++j) vr[j] = u32x4{0u, 0u, 0u, 0u};
        return;
      }
      const int c = c_start + i;
      const int len = min(kChunk, si.len - c * kChunk);
      const char* vc = reinterpret_cast<const char*>(Vb + (int64_t)c * kChunk * row_v);
#pragma unroll
      for (int j = 0; j < Cfg::NVP; ++j) {
        const int idx = clane + 64 * j, row = min(idx / Cfg::VPR, len - 1), cv = (idx % Cfg::VPR) * 8;
        vr[j] = *reinterpret_cast<const u32x4*>(vc + (uint32_t)(row * row_v + cv) * 2u);
      }
    };
    // One chunk step; EMIT (compile-time): whether the chunk produces O (lookback
    // chunks do not: no Q product, no O), so each variant is straight-line code.
    // O of chunk i leaves through the V columns: at the end of the step each lane puts
    // its packed O pieces into this wave's V columns (free once V' is formed), and at
    // the top of the next step, after the V loads have landed, reads them back and
    // stores them.  The O stores therefore go out after the wait for the V loads, and
    // that wait (vmcnt counts loads and stores, which may complete out of order, so
    // any outstanding store makes it wait for everything) only ever covers stores a
    // step old.  The buffer resource ends after row len - 1: the hardware drops the
    // stores of rows past a partial chunk's end, so no store sits behind a branch.
    auto o_slot = [&](int u, int j) {
      const int row = (cq & 1) ? prow(u + 1, cr16) : prow(u, cr16);
      return row * VS + wcol + 16 * j + 8 * (cq >> 1);
    };
    auto flush_o = [&](int i) {
      const int c = c_start + i;
      const int len = min(kChunk, si.len - c * kChunk);
      const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
          Ob + (int64_t)c * kChunk * row_v, (short)0, len * row_v * 2, kRawBufferFlags);
#pragma unroll
      for (int u = 0; u < 4; u += 2) {
        const int row = (cq & 1) ? prow(u + 1, cr16) : prow(u, cr16);
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(sV + o_slot(u, j));
          __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, (row * row_v + 16 * j + 8 * (cq >> 1)) * 2, 0, 0);
        }
      }
    };
    // FLUSH (compile-time): the previous step produced O that is still to be stored.
    auto chain_step = [&](auto emit_tag, auto flush_tag, int i) {
      constexpr bool EMIT = decltype(emit_tag)::value;
      if constexpr (decltype(flush_tag)::value) flush_o(i - 1);
      const int b = i & 1;
      const bf16* cK = sK[i % 3];
      const bf16* cQ = sQ[b];
      const bf16* cT = sT[b];
      const bf16* cP = sP[b];
      auto rows4 = [&](const float* v, int u) { return *reinterpret_cast<const f32x4*>(v + prow(u, 4 * cq)); };
      // ---- this chunk's V columns into LDS (the next chunk's loads go out once the
      //      X and Y fragments are dead)
#pragma unroll
      for (int j = 0; j < Cfg::NVP; ++j) {
        const int idx = clane + 64 * j, row = idx / Cfg::VPR, cv = (idx % Cfg::VPR) * 8;
        *reinterpret_cast<u32x4*>(sV + row * VS + wcol + cv) = vr[j];
      }
      wave_lds_sync();
      i16x4 vraw[4][NCT];   // V in accumulator layout, read during the last X/Y step
      frag aT[6];           // T fragments, read there too
      f32x4 gamr[4];        // gamma of this lane's rows, read there too
      // ---- X = K h and Y^T = h^T Q^T (transposed: a lane holds four consecutive value
      //      columns of one query row, the layout of the O store).  Every K and Q
      //      fragment feeds one MFMA per column tile.  Software-pipelined over the
      //      contraction steps: step ks + 1's fragments are read while step ks's
      //      products run, and the scheduling barriers keep it at that (two steps of
      //      fragments live, not all of them).
      f32x4 X[4][NCT], Yp[4][NCT];
      {
        frag fk[2][4], fq[2][4];
        auto read = [&](int ks) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            fk[ks & 1][u] = lds_frag(cK, KS, 16 * u + cr16, 32 * ks, cq);
            if constexpr (EMIT) fq[ks & 1][u] = lds_frag(cQ, KS, 16 * u + cr16, 32 * ks, cq);
          }
        };
        read(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if (ks + 1 < NKS) read(ks + 1);
          if (ks + 1 == NKS) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int j = 0; j < NCT; ++j) {
                const int col = wcol + 16 * j;
                vraw[u][j] = col_read4_raw(sV, VS, prow(u, 4 * cq), col + cr16, col + 4 * (cr16 & 3));
              }
#pragma unroll
            for (int f = 0; f < 6; ++f) aT[f] = *reinterpret_cast<const frag*>(cT + f * FR + 8 * clane);
#pragma unroll
            for (int u = 0; u < 4; ++u) gamr[u] = rows4(sGam[b], u);
          }
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            const frag hb = M::pack(hs[2 * ks][j], hs[2 * ks + 1][j]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              X[u][j] = M::run(fk[ks & 1][u], hb, ks == 0 ? zero4 : X[u][j]);
              if constexpr (EMIT) Yp[u][j] = M::run(hb, fq[ks & 1][u], ks == 0 ? zero4 : Yp[u][j]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      load_v(min(i + 1, nrun - 1));
      // ---- V - diag(gamma) X, in place (diag(beta) is folded into the stored T)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          f32x4 vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = __uint_as_float(((uint32_t)(uint16_t)vraw[u][j][e]) << 16);
          X[u][j] = vv - gamr[u] * X[u][j];
        }
      }
      // ---- K^T fragments of the state update (LDS transpose reads), pipelined over pairs
      //      of dk tiles; the first pair is read here, ahead of U
      frag kt[2][2][2];   // [buffer][tile of the pair][contraction step]
      frag aP[6];         // P fragments (output chunks), read during the last pair
      float gsr[4];       // gamma * scale of this lane's query rows, read there too
      auto read_kt = [&](int t0) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int t = t0 + dt;
          const int own = prow(t, cr16), supply = prow(t, 4 * (cr16 & 3));
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            kt[(t0 >> 1) & 1][dt][ks] = col_frag(cK, KS, 32 * ks + 4 * cq, 32 * ks + 16 + 4 * cq, own, supply);
        }
      };
      read_kt(0);
      f32x4 decr[4];   // exp(G_last - G) of this lane's rows
#pragma unroll
      for (int u = 0; u < 4; ++u) decr[u] = rows4(sDec[b], u);
      // ---- U = T V' (T lower triangular: row tiles 0, 1 need contraction step 0 only)
      f32x4 U[4][NCT];
      {
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          frag wb[2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) wb[ks] = M::pack(X[2 * ks][j], X[2 * ks + 1][j]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int ks = 0; ks <= (u >> 1); ++ks)
              U[u][j] = M::run(aT[tri_frag(u, ks)], wb[ks], ks == 0 ? zero4 : U[u][j]);
        }
      }
      frag ubp[2][NCT], ubd[2][NCT];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          if constexpr (EMIT) ubp[ks][j] = M::pack(U[2 * ks][j], U[2 * ks + 1][j]);
          ubd[ks][j] = M::pack(U[2 * ks][j] * decr[2 * ks], U[2 * ks + 1][j] * decr[2 * ks + 1]);
        }
      // ---- h <- gamma_last h + K^T (diag(d) U)
      const float gC = sGC[b];
      {
#pragma unroll
        for (int t0 = 0; t0 < NKT; t0 += 2) {
          if (t0 + 2 < NKT) read_kt(t0 + 2);
          if constexpr (EMIT) {
            if (t0 + 2 == NKT) {
#pragma unroll
              for (int f = 0; f < 6; ++f) aP[f] = *reinterpret_cast<const frag*>(cP + f * FR + 8 * clane);
#pragma unroll
              for (int u = 0; u < 4; ++u) gsr[u] = sGamS[b][prow(u, cr16)];
            }
          }
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
              hs[t0 + dt][j] *= gC;
#pragma unroll
              for (int ks = 0; ks < 2; ++ks)
                hs[t0 + dt][j] = M::run(kt[(t0 >> 1) & 1][dt][ks], ubd[ks][j], hs[t0 + dt][j]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- O = scale diag(gamma) Q h + P U, stored 16 bytes per lane
      if constexpr (EMIT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            Yp[u][j] = Yp[u][j] * gsr[u];
#pragma unroll
            for (int ks = 0; ks <= (u >> 1); ++ks) Yp[u][j] = M::run(ubp[ks][j], aP[tri_frag(u, ks)], Yp[u][j]);
          }
        }
        // for the tile pair (u, u+1), v_permlane16_swap hands lane group q^1 the other
        // group's four columns: an even group then holds eight consecutive columns of
        // tile u's row, an odd group those of tile u+1's row
#pragma unroll
        for (int u = 0; u < 4; u += 2)
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            const uint2 a = pack_bf16x4(Yp[u][j]), bb = pack_bf16x4(Yp[u + 1][j]);
            const auto sx = __builtin_amdgcn_permlane16_swap(a.x, bb.x, false, false);
            const auto sy = __builtin_amdgcn_permlane16_swap(a.y, bb.y, false, false);
            const u32x4 v = {sx[0], sy[0], sx[1], sy[1]};
            *reinterpret_cast<u32x4*>(sV + o_slot(u, j)) = v;
          }
      }
    };
    // the prep waves fill the first buffer sets during NP + 1 steps
    if (nrun > 0) load_v(0);
    for (int s = -NP - 1; s < 0; ++s) __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    auto refresh_lanes = [&]() {
      const int z = opaque_zero();
      cr16 = r16 + z;
      cq = q + z;
      clane = lane + z;
    };
    // lookback chunks (no O) come first; one loop per variant keeps each loop body
    // straight-line for the register allocator.  The first output step (nothing to
    // store yet) is peeled; the last one's O is stored after the loop.
    const int nlook = min(nrun, c_out - c_start);
    int i = 0;
    for (; i < nlook; ++i) {
      refresh_lanes();
      chain_step(std::false_type{}, std::false_type{}, i);
      __syncthreads();
    }
    if (i < nrun) {
      refresh_lanes();
      chain_step(std::true_type{}, std::false_type{}, i);
      __syncthreads();
      ++i;
    }
    for (; i < nrun; ++i) {
      refresh_lanes();
      chain_step(std::true_type{}, std::true_type{}, i);
      __syncthreads();
    }
    if (nrun > nlook) {
      refresh_lanes();
      flush_o(nrun - 1);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (P1) {
      if (mcols) {
        // M as bf16 high and low parts in the merge's operand order (mfrag_offset)
        bf16* mhi = reinterpret_cast<bf16*>(plan.cp.mcorr) + (sg * H + h) * 2 * DK * DK;
        bf16* mlo = mhi + DK * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int j = 0; j < NCT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (mc + 16 * j >= DK) continue;   // a half-used block's spare columns
              const float x = hs[t][j][i];
              const bf16 hi = (bf16)x;
              const int64_t at = mfrag_offset<DK>(prow(t, 4 * q + i), mc + 16 * j);
              mhi[at] = hi;
              mlo[at] = (bf16)(x - (float)hi);
            }
      } else {
        // S* as the merge's accumulator tiles (sfrag_offset): a lane's four rows of a
        // tile are consecutive, one 16-byte store per tile
        float* dst = plan.cp.sstar + (sg * H + h) * DK * dv;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int j = 0; j < NCT; ++j)
            *reinterpret_cast<f32x4*>(dst + sfrag_offset<DK>(prow(t, 4 * q), col0 + wcol + 16 * j + r16)) = hs[t][j];
      }
    } else if (last_seg && p.hT) {
      float* dst = p.hT + (int64_t)nh * DK * dv + col0 + wcol;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(int64_t)prow(t, 4 * q + i) * dv + 16 * j + r16] = hs[t][j][i];
    }
  } else {
    // =========================== prep wave ===========================
    const int pw = wave - NCH;                 // owns chunks c_start + i, i = pw (mod NP)
    float* sG = sGB[pw];                       // chunk-local cumulative gate, per row
    float* sB = sG + kChunk;                   // beta, per row
    float* sAd = sInv;                         // diagonal A blocks, row-major, stride 16
    float* sTd = sInv + 4 * Cfg::ABS;          // diagonal T blocks, column-major, stride TCS
    const bf16* Kb = reinterpret_cast<const bf16*>(p.k) + si.tok0 * row_qk + (int64_t)h * DK;
    const bf16* Qb = reinterpret_cast<const bf16*>(p.q) + si.tok0 * row_qk + (int64_t)h * DK;
    const float* Gb = p.g + si.tok0 * H + h;
    const int bsz = p.beta_bf16 ? 2 : 4;
    const char* Bb = reinterpret_cast<const char*>(p.beta) + (si.tok0 * H + h) * bsz;
    PrepChunk<DK> R;
    // per-lane indices used below, re-derived at every pass of the step loop from an
    // opaque zero: their address arithmetic stays inside the loop (a few VALU
    // operations) instead of being hoisted out and spilled to scratch
    int lr16 = r16, lq = q, llane = lane;

    // Rows past a partial chunk's end read the chunk's last row instead (always inside
    // the sequence) and are left as they are: their beta and g are zeroed in
    // gates_gram, which zeroes every contribution of such a row (A's rows, V', U), and
    // their O rows are never stored.  Nothing is computed from a loaded value until a
    // later phase, so issuing a batch of loads never waits for it.
    auto row_off = [&](int a, int len) { return (uint32_t)(min(16 * a + lr16, len - 1) * row_qk + 8 * lq) * 2u; };
    // ---- K, g and beta of chunk i (for step 1)
    auto load_kgb = [&](int i) {
      const int c = c_start + i;
      const int len = min(kChunk, si.len - c * kChunk);
      R.len = len;
      const int64_t t0 = (int64_t)c * kChunk;
      const char* kc = reinterpret_cast<const char*>(Kb + t0 * row_qk);
      const int64_t ti = (t0 + min(llane, len - 1)) * H;
      R.g = Gb[ti];
      if (p.beta_bf16) R.braw = reinterpret_cast<const uint16_t*>(Bb)[ti];
      else R.braw = reinterpret_cast<const uint32_t*>(Bb)[ti];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t off = row_off(a, len);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) R.kf[a][ks] = *reinterpret_cast<const frag*>(kc + off + 64u * ks);
      }
    };
    // ---- Q of chunk i (for P and the LDS write).  A lookback chunk produces no
    //      output and needs no Q: it re-reads its own K rows instead (just loaded, so
    //      served by the cache), which keeps the load count of every phase fixed.
    auto load_kq = [&](int i, bool withq) {
      const int c = c_start + i;
      const int len = R.len;
      const int64_t t0 = (int64_t)c * kChunk;
      const char* qc = reinterpret_cast<const char*>((withq ? Qb : Kb) + t0 * row_qk);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t off = row_off(a, len);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) R.qf[a][ks] = *reinterpret_cast<const frag*>(qc + off + 64u * ks);
      }
    };

    // ---- gates, the Gram tiles of K K^T, and A = strict_lower(diag(beta) K K^T * Gamma)
    //      in registers: diagonal blocks D(A_aa), off-diagonal blocks transposed D(A_ab^T)
    auto gates_gram = [&]() {
      const bool real = llane < R.len;   // rows past the chunk end: g = 0, beta = 0
      const float bv = p.beta_bf16 ? __uint_as_float(R.braw << 16) : __uint_as_float(R.braw);
      const float G = wave_inclusive_scan_dpp(real ? R.g : 0.f);
      sG[llane] = G;
      sB[llane] = real ? bv : 0.f;
      f32x4 gd[4], go[6];   // D(K_a K_a^T), D(K_b K_a^T) for b < a
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        int a, b;
        lower_block(k, a, b);
        f32x4 acc = zero4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = M::run(R.kf[b][ks], R.kf[a][ks], acc);
        if (a == b) gd[a] = acc;
        else go[(a * (a - 1)) / 2 + b] = acc;
      }
      wave_lds_sync();
      float Gc[4], Bc[4];
      f32x4 Gr[4], Br[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        Gc[a] = sG[16 * a + lr16];
        Bc[a] = sB[16 * a + lr16];
        Gr[a] = *reinterpret_cast<const f32x4*>(sG + 16 * a + 4 * lq);
        Br[a] = *reinterpret_cast<const f32x4*>(sB + 16 * a + 4 * lq);
      }
      // A[m][k] = beta_m exp(G_m - G_k) (K K^T)[m][k], k < m
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * lq + i;
          R.ad[a][i] = lr16 < m ? Br[a][i] * fast_exp(Gr[a][i] - Gc[a]) * gd[a][i] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < a; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            R.at[(a * (a - 1)) / 2 + b][i] = Bc[a] * fast_exp(Gc[a] - Gr[b][i]) * go[(a * (a - 1)) / 2 + b][i];
      }
    };

    // ---- T_bb = (I + A_bb)^{-1} for the four diagonal blocks, in fp32: lane (r, q)
    //      solves column r of block q by forward substitution on the shared scratch
    auto solve_diag = [&]() {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) sAd[a * Cfg::ABS + (4 * lq + i) * 16 + lr16] = R.ad[a][i];
      wave_lds_sync();
      {
        const float* arow = sAd + lq * Cfg::ABS;
        float x[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          float acc = (m == lr16) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < (m + 3) / 4; ++j) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(arow + m * 16 + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * j + e < m) acc -= a4[e] * x[4 * j + e];
          }
          x[m] = acc;
        }
        float* tcol = sTd + lq * Cfg::TBS + lr16 * Cfg::TCS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = {x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
          *reinterpret_cast<f32x4*>(tcol + 4 * j) = v;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        R.td[a] = *reinterpret_cast<const f32x4*>(sTd + a * Cfg::TBS + lr16 * Cfg::TCS + 4 * lq);
#pragma unroll
        for (int i = 0; i < 4; ++i) R.tdt[a][i] = sTd[a * Cfg::TBS + (4 * lq + i) * Cfg::TCS + lr16];
      }
    };

    // ---- the off-diagonal blocks by two doubling levels: T_10 = -T_11 A_10 T_00,
    //      T_32 = -T_33 A_32 T_22, then the lower-left 32 x 32 quadrant from the two
    //      diagonal quadrants; T leaves as bf16 in the LDS-write layout
    auto doubling = [&]() {
      auto at = [&](int a, int b) -> const f32x4& { return R.at[(a * (a - 1)) / 2 + b]; };
      const f32x4 R10 = mm16(at(1, 0), R.td[0], zero4);
      const f32x4 T10 = -mm16(R.tdt[1], R10, zero4);
      const f32x4 T10T = -mm16(R10, R.tdt[1], zero4);
      const f32x4 R32 = mm16(at(3, 2), R.td[2], zero4);
      const f32x4 T32T = -mm16(R32, R.tdt[3], zero4);
      const f32x4 R20 = mm16(at(2, 1), T10, mm16(at(2, 0), R.td[0], zero4));
      const f32x4 R21 = mm16(at(2, 1), R.td[1], zero4);
      const f32x4 R30 = mm16(at(3, 1), T10, mm16(at(3, 0), R.td[0], zero4));
      const f32x4 R31 = mm16(at(3, 1), R.td[1], zero4);
      const f32x4 T20T = -mm16(R20, R.tdt[2], zero4);
      const f32x4 T21T = -mm16(R21, R.tdt[2], zero4);
      const f32x4 T30T = -mm16(R30, R.tdt[3], mm16(R20, T32T, zero4));
      const f32x4 T31T = -mm16(R31, R.tdt[3], mm16(R21, T32T, zero4));
      // T diag(beta) leaves for the chain: block (a, b) scaled by beta of its columns
      // 16 b + 4 q .. +3 (zero on rows past a partial chunk's end).
      // lower_block order: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
      f32x4 bc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bc[c] = *reinterpret_cast<const f32x4*>(sB + 16 * c + 4 * lq);
      R.tb[0] = pack_bf16x4(R.tdt[0] * bc[0]);
      R.tb[1] = pack_bf16x4(T10T * bc[0]);
      R.tb[2] = pack_bf16x4(R.tdt[1] * bc[1]);
      R.tb[3] = pack_bf16x4(T20T * bc[0]);
      R.tb[4] = pack_bf16x4(T21T * bc[1]);
      R.tb[5] = pack_bf16x4(R.tdt[2] * bc[2]);
      R.tb[6] = pack_bf16x4(T30T * bc[0]);
      R.tb[7] = pack_bf16x4(T31T * bc[1]);
      R.tb[8] = pack_bf16x4(T32T * bc[2]);
      R.tb[9] = pack_bf16x4(R.tdt[3] * bc[3]);
    };

    // ---- P = scale (Q K^T) * Gamma, lower blocks; lane (r, q) of block (a, b): query
    //      16a + r, keys 16b + 4q .. +3 (as K_b Q_a^T)
    auto p_tiles = [&](bool withq) {
      if (withq) {
#pragma unroll
        for (int k = 0; k < 10; ++k) {
          int a, b;
          lower_block(k, a, b);
          f32x4 acc = zero4;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = M::run(R.kf[b][ks], R.qf[a][ks], acc);
          const int qrow = 16 * a + lr16, key0 = 16 * b + 4 * lq;
          const float Gq = sG[qrow];
          const f32x4 Gk = *reinterpret_cast<const f32x4*>(sG + key0);
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = key0 + e <= qrow ? p.scale * acc[e] * fast_exp(Gq - Gk[e]) : 0.f;
          R.pb[k] = pack_bf16x4(pv);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 10; ++k) R.pb[k] = make_uint2(0u, 0u);
      }
    };

    // ---- K of chunk i into its ring slot i % 3 (free from step i - 2 on: the chain
    //      read it last for chunk i - 3)
    auto write_k = [&](int i) {
      bf16* dst = sK[i % 3];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int lr = tord(16 * a + lr16);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) *reinterpret_cast<frag*>(dst + lr * KS + 32 * ks + 8 * lq) = R.kf[a][ks];
      }
    };

    // ---- Q, T, P and the gate tables of chunk i, into buffer set i % 2
    auto write = [&](int i, bool withq) {
      const int b = i & 1;
      if (withq) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int lr = tord(16 * a + lr16);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) *reinterpret_cast<frag*>(sQ[b] + lr * KS + 32 * ks + 8 * lq) = R.qf[a][ks];
        }
      }
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        int a, bb;
        lower_block(k, a, bb);
        const int off = tri_offset(a, bb, lr16, lq);
        *reinterpret_cast<uint2*>(sT[b] + off) = R.tb[k];
        if (withq) *reinterpret_cast<uint2*>(sP[b] + off) = R.pb[k];
      }
      const float G = sG[llane];
      const float Glast = sG[kChunk - 1];   // rows past the chunk end repeat the last real G
      const float gam = fast_exp(G);
      sGam[b][llane] = gam;
      sGamS[b][llane] = gam * p.scale;
      sDec[b][llane] = fast_exp(Glast - G);
      if (llane == 0) sGC[b] = fast_exp(Glast);
    };

    // Step schedule (step s: the chain computes chunk s; s < 0: preparation only).
    // This wave owns chunks i = pw, pw + NP, ...; for chunk i:
    //   K, g, beta loads issued at step i - 6 (first owned chunk: at the start)
    //   step i - 4: gates, Gram tiles, A in registers; K and Q loads issued
    //   step i - 3: diagonal-block substitution (the shared scratch), doubling -> T
    //   step i - 2: P; K into its ring slot; K, g, beta loads of chunk i + NP issued
    //   step i - 1: Q, T, P and the gate tables into buffer set i % 2
    // Written as one straight pass per owned chunk so that the compiler sees which
    // registers each phase holds; loads past the last chunk reload the last chunk
    // (unused), so every phase defines the same registers.  Every wave executes one
    // barrier per step, nrun + NP + 1 in all.
    static_assert(NP == 4, "one pass of the loop below is the NP = 4 steps of one owned chunk");
    auto refresh_lanes = [&]() {
      const int z = opaque_zero();
      lr16 = r16 + z;
      lq = q + z;
      llane = lane + z;
    };
    // every prep wave issues its first chunk's loads at once: only chunk 0 waits for
    // them in the preparation steps
    int s = -NP - 1;
    refresh_lanes();
    if (nrun > 0) load_kgb(min(pw, nrun - 1));
    for (; s < pw - NP; ++s) __syncthreads();
    for (int i = pw; i < nrun; i += NP) {
      const bool withq = c_start + i >= c_out;
      refresh_lanes();
      gates_gram();        // s == i - 4
      load_kq(i, withq);
      __syncthreads();
      ++s;
      solve_diag();        // s == i - 3
      doubling();
      __syncthreads();
      ++s;
      p_tiles(withq);      // s == i - 2
      write_k(i);
      load_kgb(min(i + NP, nrun - 1));
      __syncthreads();
      ++s;
      write(i, withq);     // s == i - 1
      __syncthreads();
      ++s;
    }
    for (; s < nrun; ++s) __syncthreads();
  }
}

// 1-D grid of ceil(units / 8) * 8 workgroups per column block (see the decode in the
// kernel); pass 3: one block of all dv value columns; pass 1: (dv + dk) / dv blocks.
template <int DK, int BV, int PASS>
static hipError_t launch_wy_dk(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  using Cfg = WyCfg<DK, BV>;
  const int ncb = (PASS == kPass1 ? p.dv + DK + BV - 1 : p.dv) / BV;
  const int64_t groups = (plan.units + 7) / 8;
  if (groups * 8 * ncb > kMaxDispatchItems / Cfg::NT) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL((fused_wy_kernel<DK, BV, PASS>), dim3((unsigned)(groups * 8 * ncb)), dim3(Cfg::NT), 0, s,
                        ev.start, ev.stop, 0, p, plan);
  return hipGetLastError();
}

template <int PASS>
static hipError_t launch_wy_pass(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  if (p.dk == 128)
    return p.dv == 128 ? launch_wy_dk<128, 128, PASS>(p, plan, s, ev) : launch_wy_dk<128, 64, PASS>(p, plan, s, ev);
  return p.dv == 128 ? launch_wy_dk<64, 128, PASS>(p, plan, s, ev) : launch_wy_dk<64, 64, PASS>(p, plan, s, ev);
}

hipError_t launch_fused_wy(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev) {
  if (plan.units == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if (!p.qkv_bf16 || (plan.mode != kPass3 && plan.mode != kPass1)) return hipErrorInvalidValue;
  return plan.mode == kPass1 ? launch_wy_pass<kPass1>(p, plan, s, ev) : launch_wy_pass<kPass3>(p, plan, s, ev);
}

}  // namespace gdn
