// Gate scan on gfx950: the window-lookback lengths.  The forward pass takes one per
// segment start (the W chunks right before it); the stand-alone entry point one per
// (sequence, head), from the largest gate sum over every run of W consecutive chunks
// (W = 1..wmax).
//
// FlashQLA talk transcript (tokendh.com), sliding-window section: with alpha < 1
// and ||I - beta k k^T|| <= 1 a state's influence decays by alpha per token, so a
// head whose gate is not identically 1 has a window beyond which old state no
// longer matters; a light kernel scans each head's gates (cost of about one gate
// cumsum) to pick the heads that may start a segment from a lookback window.
//
// Decision: the error of starting W chunks early from a zero state is at most
// ||S_old|| exp(sum of g over those chunks), so a start may use W if the W chunks
// before it have gate sum <= log_eps - margin (margin 1e-3 absorbs the fp32
// summation error), and a head may use W at every start if every run of W
// consecutive chunks does.  The smallest such W <= wmax is used; 0 = none.
//
// The chunk gate sums come from the chunk-inverse kernel, which forms the chunk's
// cumulative gate anyway (or, for the stand-alone entry point, from
// chunk_gate_sums_kernel with the same wave scan, so both give identical sums).
// gate_window_max: one block per (sequence, head) forms the segment windows (forward
// pass) or the maximum run sum per W (block_run_max) into best[nh][W] (floats as
// order-preserving uints; 0 = no such run, so no reset is needed), which
// gate_window_finalize turns into W for the stand-alone entry point (window_of).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Per (chunk, head): the sum of the chunk's gates, as the last entry of the
// chunk-local inclusive wave scan (one wave per chunk-head, lane = chunk row).
__global__ __launch_bounds__(256) void chunk_gate_sums_kernel(Problem p, float* __restrict__ csum,
                                                              uint32_t* __restrict__ ncorr_zero) {
  const int lane = threadIdx.x & 63;
  if (ncorr_zero && blockIdx.x == 0 && threadIdx.x < 2) ncorr_zero[threadIdx.x] = 0u;
  const int HG = (p.H + 3) / 4;
  const int64_t cg = blockIdx.x / HG;
  const int h = (int)(blockIdx.x % HG) * 4 + (threadIdx.x >> 6);
  if (h >= p.H) return;
  const int n = seq_of_chunk(cg, p.chunk_off, p.N, p.T);
  const SeqInfo si = seq_info(n, p.cu, p.chunk_off, p.T);
  const int c = (int)(cg - si.chunk0);
  const int len = min(kChunk, si.len - c * kChunk);
  const float gv = lane < len ? p.g[(si.tok0 + (int64_t)c * kChunk + lane) * p.H + h] : 0.f;
  const float G = wave_inclusive_scan(gv);
  if (lane == kChunk - 1) csum[cg * p.H + h] = G;
}

// NT threads = run starts per pass of the gate-window scan: 256 for sequences of up
// to 512 chunks, 1024 for longer ones (fewer serial passes when there are few blocks).
template <int NT>
__global__ __launch_bounds__(NT) void gate_window_max_kernel(const float* __restrict__ csum,
                                                                       const int32_t* __restrict__ cu,
                                                                       const int32_t* __restrict__ chunk_off,
                                                                       int64_t T, int N, int H, int wmax,
                                                                       uint32_t* __restrict__ best, float thr,
                                                                       uint32_t* __restrict__ ncorr, int seg_chunks,
                                                                       const int32_t* __restrict__ seg_off,
                                                                       int32_t* __restrict__ seg_win,
                                                                       int32_t* __restrict__ p1_slots, int64_t p1_cap) {
  __shared__ float sums[NT + kWindowMaxCap];
  __shared__ float red[NT / 64 * kWindowMaxCap];
  const int nh = blockIdx.x, n = nh / H, h = nh % H;
  const SeqInfo si = seq_info(n, cu, chunk_off, T);
  const int nch = (si.len + kChunk - 1) / kChunk;
  // per-segment windows, first: the W chunks right before a segment start bound the
  // error of starting it from zero W chunks early (one thread per start)
  const int L = seg_chunks;
  const int segs = seg_win ? max(1, (nch + L - 1) / L) : 0;
  const int64_t sb = seg_off ? (int64_t)seg_off[n] : (int64_t)n * segs;   // dense: equal lengths
  int miss = 0;
  for (int j = 1 + (int)threadIdx.x; j < segs; j += NT) {
    const int st = j * L, lim = min(wmax, st);
    float c[kWindowMaxCap];   // the (up to) 16 chunk sums before the start, loaded at once
#pragma unroll
    for (int k = 0; k < kWindowMaxCap; ++k)   // index kept inside the sequence
      c[k] = csum[(si.chunk0 + max(st - 1 - k, 0)) * H + h];
    int W = 0;
    float acc = 0.f;
#pragma unroll
    for (int k = 1; k <= kWindowMaxCap; ++k) {
      acc += k <= lim ? c[k - 1] : 0.f;
      if (W == 0 && k <= lim && (k == st || acc <= thr)) W = k;
    }
    seg_win[(sb + j) * H + h] = W;
    miss |= W == 0;
  }
  // a pair with a start that has no window takes the correction: no slot keeps a
  // window, and its segments but the last are pass-1 units, a run of segs - 1 list
  // entries reserved here (so the atomic's round trip overlaps a maximum scan)
  const bool corr = seg_win && __syncthreads_or(miss);
  uint32_t base = 0;
  if (corr) {
    for (int j = (int)threadIdx.x; j < segs; j += NT) seg_win[(sb + j) * H + h] = 0;
    if (threadIdx.x == 0 && ncorr) {
      atomicAdd(ncorr, 1u);
      if (p1_slots) base = atomicAdd(ncorr + 1, (uint32_t)(segs - 1));
    }
  } else if (seg_win && threadIdx.x == 0) {
    seg_win[sb * H + h] = 0;
  }

  if (best) {
    const float v = block_run_max<NT>(csum, si.chunk0, nch, H, h, wmax, sums, NT + kWindowMaxCap, red);
    const int w = threadIdx.x;   // thread w holds the maximum for runs of w + 1 chunks
    if (w < kWindowMaxCap)       // 0 = no run of that length
      best[nh * kWindowMaxCap + w] = (w < wmax && v > -INFINITY) ? ordered_bits(v) : 0u;
  }
  if (!corr || !p1_slots || !ncorr) return;
  __shared__ uint32_t sbase;
  if (threadIdx.x == 0) sbase = base;
  __syncthreads();
  // (bounded: a count an earlier scan left unreset can run past the list)
  for (int j = (int)threadIdx.x; j + 1 < segs; j += NT)
    if ((int64_t)sbase + j < p1_cap) p1_slots[sbase + j] = (int32_t)((sb + j) * H + h);
}

// Packed input: the chunk / segment offset tables, and (split plans) the order in
// which pass 3 takes the segments: longest first (list scheduling: the long units
// start early and the short ones fill the tail).  Every full segment (seg_chunks
// chunks) comes first, in sequence order; then the last segment of every sequence,
// ranked by its length (longest first, ties in sequence order), the rank of each
// counted by its own thread.
__global__ __launch_bounds__(256) void plan_tables_kernel(const int32_t* __restrict__ cu, int N,
                                                          int seg_chunks, int32_t* __restrict__ chunk_off,
                                                          int32_t* __restrict__ seg_off,
                                                          int32_t* __restrict__ seg_order) {
  if (threadIdx.x == 0) {
    int32_t acc = 0, sacc = 0;
    chunk_off[0] = 0;
    if (seg_off) seg_off[0] = 0;
    for (int n = 0; n < N; ++n) {
      const int nch = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
      acc += nch;
      chunk_off[n + 1] = acc;
      if (seg_off) {
        sacc += max(1, (nch + seg_chunks - 1) / seg_chunks);  // empty sequences keep one unit
        seg_off[n + 1] = sacc;
      }
    }
  }
  if (!seg_order) return;   // (N <= kSegOrderMaxSeqs when the table is requested)
  __shared__ int last[kSegOrderMaxSeqs];   // chunks of each sequence's last segment
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int nch = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    last[n] = nch - (max(1, (nch + seg_chunks - 1) / seg_chunks) - 1) * seg_chunks;
  }
  __syncthreads();   // also publishes thread 0's seg_off to the workgroup
  const int full = seg_off[N] - N;   // full segments over all sequences
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int s0 = seg_off[n], segs = seg_off[n + 1] - s0;
    for (int j = 0; j + 1 < segs; ++j) seg_order[s0 - n + j] = s0 + j;
    const int len = last[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) rank += (last[m] > len || (last[m] == len && m < n)) ? 1 : 0;
    seg_order[full + rank] = s0 + segs - 1;
  }
}

__global__ void gate_window_finalize_kernel(const uint32_t* __restrict__ best,
                                            const int32_t* __restrict__ cu,
                                            const int32_t* __restrict__ chunk_off, int64_t T,
                                            int N, int H, int wmax, float thr,
                                            int32_t* __restrict__ out) {
  const int nh = blockIdx.x * blockDim.x + threadIdx.x;
  if (nh >= N * H) return;
  const SeqInfo si = seq_info(nh / H, cu, chunk_off, T);
  out[nh] = window_of(best, nh, (si.len + kChunk - 1) / kChunk, wmax, thr);
}

hipError_t launch_plan_tables(const int32_t* cu, int N, int seg_chunks, int32_t* chunk_off,
                              int32_t* seg_off, int32_t* seg_order, hipStream_t s) {
  plan_tables_kernel<<<1, 256, 0, s>>>(cu, N, seg_chunks, chunk_off, seg_off, seg_order);
  return hipGetLastError();
}

hipError_t launch_chunk_gate_sums(const Problem& p, float* csum, hipStream_t s, KernelEvents ev,
                                  uint32_t* ncorr_zero) {
  if (p.total_chunks == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  const int64_t blocks = p.total_chunks * ((p.H + 3) / 4);
  if (blocks > kMaxDispatchItems / 256) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL(chunk_gate_sums_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ev.start, ev.stop, 0,
                        p, csum, ncorr_zero);
  return hipGetLastError();
}

hipError_t launch_gate_scan(const Problem& p, const float* csum, int64_t max_chunks, int wmax,
                            uint32_t* best, hipStream_t s, KernelEvents ev, float thr, uint32_t* ncorr,
                            int seg_chunks, const int32_t* seg_off, int32_t* seg_win, int32_t* p1_slots,
                            int64_t p1_cap) {
  if (p.N == 0) {
    ev.record_empty(s);
    return hipSuccess;
  }
  if ((int64_t)p.N * p.H > kMaxDispatchItems / 1024) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(p.N * p.H));
  if (best && max_chunks > 512)   // (segment windows alone: a pass of 256 starts is plenty)
    hipExtLaunchKernelGGL(gate_window_max_kernel<1024>, grid, dim3(1024), 0, s, ev.start, ev.stop, 0, csum,
                          p.cu, p.chunk_off, p.T, p.N, p.H, wmax, best, thr, ncorr, seg_chunks, seg_off,
                          seg_win, p1_slots, p1_cap);
  else
    hipExtLaunchKernelGGL(gate_window_max_kernel<256>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, csum,
                          p.cu, p.chunk_off, p.T, p.N, p.H, wmax, best, thr, ncorr, seg_chunks, seg_off,
                          seg_win, p1_slots, p1_cap);
  return hipGetLastError();
}

hipError_t launch_gate_finalize(const Problem& p, const uint32_t* best, int wmax, float thr,
                                int32_t* out, hipStream_t s) {
  const int nh = p.N * p.H;
  if (nh == 0) return hipSuccess;
  gate_window_finalize_kernel<<<(nh + 255) / 256, 256, 0, s>>>(best, p.cu, p.chunk_off, p.T, p.N,
                                                               p.H, wmax, thr, out);
  return hipGetLastError();
}

}  // namespace gdn
