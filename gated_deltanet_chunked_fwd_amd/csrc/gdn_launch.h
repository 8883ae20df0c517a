// Internal host-side launch interface between the ABI layer and the kernels.
#pragma once
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

// Work description for one launch of the fused forward kernel.  A work unit is
// (sequence, head, segment); the kernel grid is (dv / BV, units).
struct FwdPlan {
  const void* Tmat;          // chunk inverses [total_chunks, H, 64, 64]
  int seg_chunks;            // chunks per segment (>= max chunks of any sequence: one segment)
  const int32_t* seg_off;    // device [N+1] segment offsets (packed + split) or null
  int64_t units;             // number of (sequence, head, segment) units
  int value_block;           // value columns per workgroup: 64, 128, or 0 (widest that fits)
};

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s);
hipError_t launch_chunk_inverse(const Problem& p, void* t_out, hipStream_t s);
hipError_t launch_fused_forward(const Problem& p, const FwdPlan& plan, hipStream_t s);

}  // namespace gdn
