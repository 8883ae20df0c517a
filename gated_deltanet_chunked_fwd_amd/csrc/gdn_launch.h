// Internal host-side launch interface between the ABI layer and the kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;  // chunk length of the WY form

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;         // device cu_seqlens or null
  const int32_t* chunk_off;  // device [N+1] chunk offsets (packed only) or null
  void* o;
  float* hT;
  int64_t T;                 // tokens per batch row (dense) / total tokens (packed)
  int64_t total_chunks;
  int N, H, dk, dv;
  int qkv_bf16;              // 1: q/k/v/o/T are bf16, 0: fp32
  int beta_bf16;
  float scale;
};

constexpr int kWindowMaxCap = 16;  // longest lookback window the gate scan can return

// Sequence-split state shared by the split passes (all null when no split).
struct CpBuffers {
  int force_correction;     // 1: every split head uses the wrong-start correction
  float* sstar;             // [total_segs, H] x [dk x dv] fp32 wrong-start (zero-start) segment
                            // end states, each in accumulator-tile order (sfrag_offset)
  void* mcorr;              // [total_segs, H] x {hi, lo} x [dk, dk] bf16: segment transition
                            // matrices M split as M = hi + lo (hi block first), each block
                            // in MFMA operand order (mfrag_offset in gdn_device.h)
  float* hstart;            // [total_segs, H, dk, dv] true segment start states
  void* gmat;               // long merge chains, per group of steps (slot of the group's first
  float* gvec;              // segment): composed map A (as mcorr) and offset b (as sstar)
  // (nullable) two counters written by the gate scan: [0] the (sequence, head) pairs
  // without an admissible window (when it is zero the correction launches, the
  // restricted chunk inverse, pass 1 and the merge, return at once instead of finding
  // that per unit) and [1] the entries of p1_slots
  const uint32_t* ncorr;
  // (nullable, needs ncorr) pass 1's work list: the slots s * H + h of the segments,
  // all but each sequence's last, of the pairs without a window, one run per pair in
  // the order the gate scan's workgroups finished (the order changes no result)
  const int32_t* p1_slots;
  // per (segment, head) slot s * H + h: the lookback window, in chunks, of the
  // segment's start (gate scan); 0 for first segments and for every slot of a
  // (sequence, head) that takes the correction
  const int32_t* seg_win;
};

// Merge chains of more steps than this run as a two-level tree (cp_merge.hip): about
// where the tree's three launches (35 us + 3.2 us * sqrt(steps) on MI355X) beat one
// serial launch (7 us + 0.75 us per step).
constexpr int kMergeTreeMinSteps = 72;
// An AQL dispatch counts the work-items of a grid dimension in 32 bits.
constexpr int64_t kMaxDispatchItems = 0xFFFFFFFFLL;

// Work description for one launch of the fused forward kernel.  A work unit is
// (sequence, head, segment); the kernel grid covers units x column blocks.
//   kPass3: steps 2-4 with O; a segment starts from h0 (first segment), from a
//           zero state a window of chunks earlier (window heads) or from hstart
//           (correction heads); the last segment writes the final state.
//   kPass1: correction heads only, all but the last segment: run the segment from
//           a zero state (value columns -> sstar) and, with V = 0, from the
//           identity (extra dk columns -> mcorr); no O.  With cp.p1_slots a unit is
//           an entry of that list (units: its capacity), else every (segment, head).
//   kCkpt:  the backward's checkpoints: every sequence as one segment from h0 (or
//           0), value columns only, no O; the state at the start of every chunk goes
//           to ckpt (below).
enum { kPass3 = 0, kPass1 = 1, kCkpt = 2 };
// Checkpoint layout: per (chunk, head) a dk x dv fp32 state, rows in groups of four
// interleaved by column, element (r, c) at ((r / 4) * dv + c) * 4 + r % 4 (four
// consecutive rows of one column are one 16-byte store).
__host__ __device__ constexpr int64_t ckpt_offset(int r, int c, int dv) {
  return ((int64_t)(r >> 2) * dv + c) * 4 + (r & 3);
}
struct FwdPlan {
  const void* Tmat;          // chunk inverses [total_chunks, H, 64, 64]
  int seg_chunks;            // chunks per segment (>= max chunks of any sequence: one segment)
  const int32_t* seg_off;    // device [N+1] segment offsets (packed + split) or null
  const int32_t* seg_order;  // device [total_segs] pass 3's segment order (longest first) or null
  int64_t units;             // number of (sequence, head, segment) units
  int value_block;           // value columns per workgroup: 64, 128, or 0 (widest that fits)
  int pass1_block;           // pass-1 columns per workgroup: 128 (if requested), else 64
  int mode;                  // kPass3, kPass1 or kCkpt
  CpBuffers cp;
  float* ckpt;               // kCkpt: [total_chunks, H] x (dk x dv, ckpt_offset) fp32
  // kPass1 for the backward's split: identity columns only, every segment but each
  // sequence's first, the transpose of the segment's transition M stored (as cp.mcorr)
  // at the backward's slot of the segment (bwd_slot)
  int bwd_maps;
};

// The backward's split runs a sequence's segments last to first through the merge, so
// segment seg of a sequence with S segments starting at global index sg0 uses slot
// sg0 + S - 1 - seg (the merge's step k reads the maps and offsets of slot sg0 + k and
// writes the state of slot sg0 + k + 1).
__host__ __device__ constexpr int64_t bwd_slot(int64_t sg0, int S, int seg) { return sg0 + (S - 1 - seg); }

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s);
// seg_order (nullable, needs seg_off): pass 3's segment order, longest first.
hipError_t launch_plan_tables(const int32_t* cu, int N, int seg_chunks, int32_t* chunk_off,
                              int32_t* seg_off, int32_t* seg_order, hipStream_t s);
// Packed inputs of at most this many sequences get a longest-first segment order.
constexpr int kSegOrderMaxSeqs = 1024;
// Optional start / stop events of a single-kernel launch, recorded from the kernel's
// own dispatch (hipExtLaunchKernel): timing a stage this way adds no packets to the
// stream, where a separate event record costs a few microseconds of idle GPU.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  // a launcher that has nothing to launch still marks the (empty) interval
  void record_empty(hipStream_t s) const {
    if (start) (void)hipEventRecord(start, s);
    if (stop) (void)hipEventRecord(stop, s);
  }
};
// ncorr_zero (nullable): the gate scan's two counters (CpBuffers::ncorr), set to zero
// here (the scan that follows adds to them).
hipError_t launch_chunk_gate_sums(const Problem& p, float* csum, hipStream_t s, KernelEvents ev = {},
                                  uint32_t* ncorr_zero = nullptr);
// best (nullable): the per-(sequence, head) maxima of run sums for W = 1..wmax.
// seg_win (nullable): per (segment, head) windows of a plan that cuts sequences into
// segments of seg_chunks chunks (seg_off: packed segment offsets, else dense); a
// segment start takes the smallest W <= min(wmax, its chunk index) whose W chunks
// before it sum to <= thr, or W = its chunk index (the sequence start); a
// (sequence, head) with a start that has none gets 0 in every slot, adds 1 to
// ncorr[0] (nullable) and, with p1_slots (nullable, needs ncorr), appends the slots
// of its segments but the last to p1_slots (p1_cap entries), counted in ncorr[1].
hipError_t launch_gate_scan(const Problem& p, const float* csum, int64_t max_chunks, int wmax,
                            uint32_t* best, hipStream_t s, KernelEvents ev = {}, float thr = 0.f,
                            uint32_t* ncorr = nullptr, int seg_chunks = 0, const int32_t* seg_off = nullptr,
                            int32_t* seg_win = nullptr, int32_t* p1_slots = nullptr, int64_t p1_cap = 0);
hipError_t launch_gate_finalize(const Problem& p, const uint32_t* best, int wmax, float thr,
                                int32_t* out, hipStream_t s);
// max_steps: the most segment boundaries of any sequence (segments - 1).
hipError_t launch_cp_merge(const Problem& p, const FwdPlan& plan, int max_steps, hipStream_t s,
                           KernelEvents ev = {});
// csum (nullable): [total_chunks, H] per-chunk gate sums, written on the side.
// full = false: T's zero upper-right 32 x 32 quadrant is left unwritten (the fused
// forward never reads it).
hipError_t launch_chunk_inverse(const Problem& p, void* t_out, float* csum, bool full,
                                hipStream_t s, KernelEvents ev = {});
// One pass, bf16 only (fused_wy.hip): the chunk inverse formed in the kernel; kPass3
// (steps 1-4 with O) or kPass1 (the split's pass 1, S* and M; with cp.p1_slots a unit
// is an entry of the work list).  A workgroup covers dv columns.
hipError_t launch_fused_wy(const Problem& p, const FwdPlan& plan, hipStream_t s, KernelEvents ev = {});
hipError_t launch_fused_forward(const Problem& p, const FwdPlan& plan, hipStream_t s,
                                KernelEvents ev = {});

// Backward (chunk_bwd.hip): gradients of <dO, O> + <dhT, hT>.  Workgroup shares of
// dq, dk (fp32 [blocks, tokens, H, dk]) and dbeta, dg (fp32 [blocks, tokens, H]) are
// summed by the second kernel; hchk holds the state at every chunk start
// ([total_chunks, H] x dk x dv fp32 in ckpt_offset order, written by the forward's
// kCkpt pass before the backward kernel runs).  dhT and dh0 may be null.
//   kBwdFull:  the gradients; with a split, each segment starts from the state
//              gradient at its end (seg_g, the merge's output; dhT for a sequence's
//              last segment) and only a first segment writes dh0.
//   kBwdChain: the split's pass 1: every segment but a sequence's first, from a zero
//              state gradient, only the state-gradient chain (no checkpoint, no
//              gradient written); the gradient at the segment's start goes to seg_b.
enum { kBwdFull = 0, kBwdChain = 1 };
struct BwdArgs {
  const void* d_o;
  const float* dhT;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  void* dbeta;
  float* dh0;
  float* hchk;
  float* dq_p;
  float* dk_p;
  float* dbeta_p;
  float* dg_p;
  int64_t total_tokens;
  // the split of the reverse sweep: seg_chunks = 0 walks every sequence whole; else a
  // unit is (segment, head), segments numbered as in the forward's split (seg_off for
  // packed input, else the same count for every sequence), units = segments x H
  int seg_chunks;
  const int32_t* seg_off;
  int64_t units;
  int mode;                  // kBwdFull or kBwdChain
  float* seg_b;              // kBwdChain: per bwd_slot, dk x dv fp32 (sfrag_offset order)
  const float* seg_g;        // kBwdFull with a split: per bwd_slot, [dk, dv] fp32 (natural)
  // bf16 path (chunk_bwd_mfma.hip): the chunk inverses (K1, [total_chunks, H, 64, 64]
  // bf16, the zero upper-right quadrant written); the chain's checkpoints of the state
  // gradient dh' after every chunk, as its bf16 transpose split hi + lo
  // ([total_chunks, H] x {hi, lo} x [dv, dk]);
  // and gamma_n <h, dh'> of every chunk in fp32, one partial sum per 32 value columns
  // ([total_chunks, H, dv / 32])
  const void* tmat;
  void* dhchk;
  float* gnh;
};
constexpr int kBwdColumnBlock = 32;   // value columns per backward workgroup
hipError_t launch_chunk_bwd(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev = {});
// bf16 q / k / v (chunk_bwd_mfma.hip): the state-gradient chain (dv, the checkpoints
// of dh', dh0; kBwdChain: only the segment offsets), then the gradients of every
// (chunk, head) from hchk and dhchk (dq, dk, dbeta, dg).
hipError_t launch_bwd_dh(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev = {});
hipError_t launch_bwd_grads(const Problem& p, const BwdArgs& a, hipStream_t s, KernelEvents ev = {});

}  // namespace gdn
